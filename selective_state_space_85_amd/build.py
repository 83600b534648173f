"""Build libssscan.so in-tree for gfx950 with hipcc.

    python -m selective_state_space_85_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libssscan.so")
SOURCES = [os.path.join(CSRC, n) for n in ("ss_kernels.hip", "ss_bwd.hip", "ss_conv.hip", "ss_ssd.hip", "ss_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 (v_pk_*_f32) is switched off for all device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra_flags or []) + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (res.returncode, res.stdout, res.stderr))
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
