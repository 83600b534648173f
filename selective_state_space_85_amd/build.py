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
# the measurement probes (stream and ALU-issue kernels), a library of their own
PROBE_DIR = os.path.join(PKG, "probe")
PROBE_SOURCES = [os.path.join(PROBE_DIR, "ss_probe.hip")]
PROBE_LIB_PATH = os.path.join(PROBE_DIR, "libssprobe.so")
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


def build(verbose: bool = False, extra_flags=None, sources=None, out=None, probes: bool = True) -> str:
    """Compile every HIP source (one hipcc per source, in parallel) and link them into
    LIB_PATH, and the probe sources into PROBE_LIB_PATH (always recompiles).  With
    ``sources``/``out`` given, only that library is built."""
    targets = [(list(sources), out or LIB_PATH)] if sources else [(SOURCES, out or LIB_PATH)]
    if probes and not sources:
        targets.append((PROBE_SOURCES, PROBE_LIB_PATH))
    flags = FLAGS + ["-I", PROBE_DIR] + list(extra_flags or [])
    tmpdir = tempfile.mkdtemp(prefix="ssbuild")
    tmps = [o + ".tmp%d" % os.getpid() for _, o in targets]
    try:
        jobs_list = []
        for t, (srcs, _) in enumerate(targets):
            for i, src in enumerate(srcs):
                jobs_list.append((src, os.path.join(tmpdir, "%d_%d_%s.o" % (t, i, os.path.basename(src)))))
        jobs = max(1, min(len(jobs_list), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(jobs) as pool:
            list(pool.map(lambda so: _run([HIPCC] + flags + ["-c", so[0], "-o", so[1]], verbose), jobs_list))
        k = 0
        for (srcs, o), tmp in zip(targets, tmps):
            objs = [obj for _, obj in jobs_list[k:k + len(srcs)]]
            k += len(srcs)
            _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
            os.replace(tmp, o)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
        for tmp in tmps:
            if os.path.exists(tmp):
                os.remove(tmp)
    return targets[0][1]


if __name__ == "__main__":
    print(build(verbose=True))
