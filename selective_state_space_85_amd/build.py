"""Build libssscan.so in-tree for gfx950 with hipcc.

    python -m selective_state_space_85_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libssscan.so")
SOURCES = [os.path.join(CSRC, n) for n in ("ss_kernels.hip", "ss_bwd.hip", "ss_conv.hip", "ss_ssd.hip", "ss_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 (v_pk_*_f32) is switched off for all device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (res.returncode, res.stdout, res.stderr))
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)


def build(verbose: bool = False, extra_flags=None, sources=None, out=None) -> str:
    """Compile every HIP source (one hipcc per source, in parallel) and link them into
    LIB_PATH (always recompiles)."""
    sources = list(sources or SOURCES)
    out = out or LIB_PATH
    flags = FLAGS + list(extra_flags or [])
    tmpdir = tempfile.mkdtemp(prefix="ssbuild")
    tmp = out + ".tmp%d" % os.getpid()
    try:
        objs = [os.path.join(tmpdir, "%d_%s.o" % (i, os.path.basename(src))) for i, src in enumerate(sources)]
        jobs = max(1, min(len(sources), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(jobs) as pool:
            list(pool.map(lambda so: _run([HIPCC] + flags + ["-c", so[0], "-o", so[1]], verbose),
                          zip(sources, objs)))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
        if os.path.exists(tmp):
            os.remove(tmp)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
