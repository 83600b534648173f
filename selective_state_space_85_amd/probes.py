"""ctypes view of libssprobe.so (probe/ss_probe.h): the HBM stream and vector-ALU issue
probes that give the ceilings the scan is measured against.  Used by the bench only."""
from __future__ import annotations

import ctypes
import os
from typing import Dict

import torch

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probe", "libssprobe.so")
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError("libssprobe.so is not built (%s); run "
                               "`python -m selective_state_space_85_amd.build`" % PROBE_LIB_PATH)
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        vp = ctypes.c_void_p
        lib.ss_probe_stream.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp]
        lib.ss_probe_stream.restype = ctypes.c_int
        lib.ss_probe_alu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        lib.ss_probe_alu.restype = ctypes.c_int
        lib.ss_probe_alu_wg.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        lib.ss_probe_alu_wg.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(name: str, rc: int) -> None:
    if rc != 0:
        raise RuntimeError("%s: hipError_t %d" % (name, rc))


def stream_rate(n_read: int, bytes_each: int = 1 << 30, reps: int = 5, device: str = "cuda") -> Dict[str, float]:
    """GB/s of a plain stream with ``n_read`` input arrays and one output (``bytes_each``
    bytes each), event-timed over ``reps`` launches after one warm-up launch."""
    lib = load()
    words = bytes_each // 4
    ins = [torch.empty(words, dtype=torch.int32, device=device).fill_(i + 1) for i in range(n_read)]
    out = torch.empty(words, dtype=torch.int32, device=device)
    s = torch.cuda.current_stream()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = [ptr(ins[0]), ptr(ins[1]) if n_read > 1 else None, ptr(ins[2]) if n_read > 1 else None, ptr(out)]
    blocks = 256 * 16

    def launch():
        _check("ss_probe_stream", lib.ss_probe_stream(*args, bytes_each, n_read, blocks,
                                                      ctypes.c_void_p(s.cuda_stream)))

    launch()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        launch()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    moved = (n_read + 1) * bytes_each
    del ins, out
    return {"read_write": "%d:1" % n_read, "bytes_per_launch": moved, "ms": ms, "GB/s": moved / (ms * 1e-3) / 1e9}


KINDS = ("fma", "exp2", "scan element: mul, exp2, mul, fma, fma", "dependent fma chain", "dependent exp2 chain",
         "scan element without exp2", "scan element, exp2 batched per two rows", "fma waves beside exp2 waves",
         "scan element, exp2 batched, workgroup in phase", "exp2 + 2 independent fma", "exp2 + 4 independent fma",
         "exp2 + 8 independent fma")


def alu_rate(kind: int, iters: int = 0, waves_per_simd: int = 4, device: str = "cuda",
             wg_waves_per_simd: int = 1) -> Dict[str, float]:
    """The vector-ALU issue probe with ``waves_per_simd`` waves resident on every SIMD (see
    ss_probe.h for the kinds).  Returns per wave64 instruction group: the shader-clock
    cycles one SIMD spends (median over waves of s_memtime cycles / groups, divided by
    the waves sharing the SIMD: the issue cost when the SIMD is saturated), the same per
    wave (the latency when one wave runs alone), the chip-wide rate of lane-groups per
    second from event time, and the shader clock implied by s_memtime against the
    100 MHz reference clock."""
    lib = load()
    groups_per_iter = 128 if kind in (2, 5, 6, 8) else (8 if kind >= 9 else 16)
    if iters <= 0:
        iters = {0: 16384, 1: 8192, 2: 1024, 3: 8192, 4: 2048, 5: 1024, 6: 1024, 7: 8192, 8: 1024, 9: 8192,
                 10: 8192, 11: 4096}[kind]
    threads = 256 * wg_waves_per_simd  # a workgroup holds wg_waves_per_simd waves on each SIMD
    blocks = 256 * waves_per_simd // wg_waves_per_simd
    cycles = torch.zeros(blocks * threads // 64 * 2, dtype=torch.int64, device=device)
    sink = torch.empty(blocks * threads, dtype=torch.float32, device=device)
    s = torch.cuda.current_stream()

    def launch():
        _check("ss_probe_alu", lib.ss_probe_alu_wg(kind, iters, blocks, threads, ctypes.c_void_p(cycles.data_ptr()),
                                                   ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(s.cuda_stream)))

    launch()  # warms the clocks up
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    launch()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    c = cycles.cpu().double().view(-1, 2)
    cyc = float(c[:, 0].median())
    ref = float(c[:, 1].median())
    groups = float(blocks) * threads * iters * groups_per_iter  # lane-groups over the chip
    per_wave = cyc / (iters * groups_per_iter)
    return {"kind": KINDS[kind], "waves_per_simd": waves_per_simd, "wg_waves_per_simd": wg_waves_per_simd,
            "iters": iters,
            "cycles_per_wave_group_per_simd": per_wave / waves_per_simd,
            "cycles_per_group_per_wave": per_wave,
            "lane_groups_per_s": groups / (ms * 1e-3), "ms": ms,
            "shader_clock_GHz": cyc / ref * 0.1 if ref > 0 else None}
