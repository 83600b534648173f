#!/usr/bin/env python3
"""Benchmark of the selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--extras a,b,... | --no-extras]

One step = one ss_scan_fwd call over the large-layer workload (B=8, L=2048,
D=5120, N=16; bf16 u/delta/B/C/z and y, fp32 A/D and state, D skip and silu(z)
gate), inputs already resident in device memory.  Over the first ~60
back-to-back steps the part's clock dips (per-step time ~0.31 -> 0.40 ms) and
climbs back (~0.28-0.30 ms from about step 70 on), so a short region right
after a short warmup mostly times the dip.  Before the W warmup steps the bench
therefore runs the same step back to back for ``--settle-ms`` (100 ms, about
300 steps; 0 turns it off) and reports that phase as ``settle``; the timed
region is then the sustained rate.  The warmup's own average is reported as
``warmup_ms_per_step``; every later section also runs its workload back to back
for 60 ms before timing it.  Prints ONE JSON line:
elements/s (B*L*D*N per second), the roofline of the scan kernel (algorithmic
HBM bytes per launch over its event-timed duration, against 8 TB/s), and the
fp64 CPU oracle timed on a bounded sample of the same workload.

Extra objects: ``decode_step`` (ss_step on the B=256, D=5120 recurrent-step
workload: chained on the same operands, with the last-level cache flushed
before each token, and 1000 chained tokens with fresh operands),
``decode_graph`` (single-sequence decode, B=1: 64 chained ss_step calls
launched one by one against the same loop captured once in a hipGraph and
replayed), ``parity`` (the timed output against the oracle on every
channel, taken in the CPU-baseline leg, the one place the oracle runs; it runs
even when the oracle's timed repetitions are skipped), ``probes`` (the
measured ceilings: a 3:1 read:write HBM stream like the scan's, a plain copy,
and the issue cost of fp32 fma, v_exp_f32 and the scan's per-element group),
``copy_reference`` (a plain 1 GiB device copy, the scale for the HBM
counters), ``flushed`` (the same scan timed with the 256 MB last-level cache flushed
before every step), ``options`` (the same layer with the softplus(delta +
bias) step size and/or the zero-order-hold input term), ``configs``
(the small-model layer and the long context at their own shapes, both
chunked: the small layer's 128-row chunks take an aggregate pass, the carries
and an emit pass; the long context's 4096-row chunks run first from their own
starts, then the carries, then each later chunk's head is rerun from its carry
until the carry has decayed below fp32 resolution), ``backward``
(ss_scan_bwd on the same layer: all input gradients from dy; and the training
path, ss_scan_fwd_ckpt keeping every 16th state and ss_scan_bwd_ckpt reusing
them), ``conv1d``
(ss_conv1d_silu producing the layer's u from the x half of a (B, L, 2D)
in-projection output, with its HBM roofline) and ``ssd`` (ss_ssd_fwd, the
multi-head recurrence on the matrix cores, B=8 L=2048, 64 heads of 64
channels, dstate 128).  ``--extras`` picks which of the sections after the
timed region run (flushed, options, backward, configs, conv1d, ssd, decode;
decode covers decode_step and decode_graph); all by default.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "selective-scan elements/s (B·L·D·N) + achieved HBM GB/s vs peak, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_scan_large_layer.txt")


# the sections run after the timed region, each timing one more workload or option, each
# after running it back to back for SETTLE_MS (the clock moves for some tens of ms after
# the load changes: a ~50 us call takes ~48 us for its first 200 calls, 45.5 after ~600)
SETTLE_MS = 60.0
EXTRA_SECTIONS = ("flushed", "options", "backward", "configs", "conv1d", "ssd", "decode")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # the part's clock settles over the first ~60 steps of back-to-back scans (a dip to
    # ~0.40 ms per step, then a climb back to ~0.29 ms), so the default warmup runs past it
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="run the step back to back for this long before the warmup steps "
                         "(untimed; 0 = off), so that short runs time the settled clock")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle's timed repetitions (the parity check of the timed output still runs)")
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads and flushed timing")
    ap.add_argument("--extras", default="all",
                    help="comma-separated extra sections to run (default all): " + ",".join(EXTRA_SECTIONS))
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the ceiling probes and the plain device copy of known size (counter scaling)")
    args = ap.parse_args()
    args.extra_set = set() if args.no_extras else (
        set(EXTRA_SECTIONS) if args.extras == "all" else set(x for x in args.extras.split(",") if x))
    unknown = args.extra_set - set(EXTRA_SECTIONS)
    if unknown:
        ap.error("unknown --extras section(s): %s" % ",".join(sorted(unknown)))
    return args


# the sources that define the scan kernel and how it is launched (the backward, conv1d and
# SSD kernels live in files of their own)
SCAN_SOURCES = ("ss_api.cpp", "ss_device.h", "ss_internal.h", "ss_kernels.hip")


def kernel_source_hash(names=SCAN_SOURCES) -> str:
    """Hash of the code of the given kernel sources (default: the scan kernel's; None:
    every file): comments and whitespace are left out, so that only a change of the
    code marks counter figures stored for those kernels as stale."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_85_amd", "csrc")
    for name in sorted(os.listdir(csrc) if names is None else names):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def read_traffic(src_hash: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel sources; otherwise None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def alu_cobound(w, ms_step, alg_bytes, probe=None):
    """The vector-ALU ceiling of the same step.

    Measured: the chip-wide rate of the scan's per-element group (mul, exp2, mul, fma,
    fma; the ALU probe's kind 2, four waves per SIMD) gives ``floor_ms`` = elements /
    rate, the time the recurrence's arithmetic alone takes at full issue; ``frac`` is that
    floor over the step's time.  The per-row work (delta*u, the D skip, silu(z), the bf16
    rounding: about 10 issue slots per (b, t, d) row, 0.6 per element at N = 16) is not in
    the probe and is added from unit counts as ``per_row_ms``.

    Derived from unit counts and clock (256 CUs x 64 fp32 lanes x 2.4 GHz, no packed
    fp32), ``ceilings_ms`` gives each bound alone: HBM at the 8 TB/s spec, the
    transcendentals (one exp2 per element, exp2 and reciprocal per gated row) at the
    probe's measured v_exp_f32 cycles, and the other vector operations at the measured
    fma cycles."""
    rows = w.elements // w.dstate
    per_row = 1 + (1 if w.has_D else 0) + (7 if w.has_z else 0) + 1
    peak_slots = 256 * 64 * 2.4e9
    simd_cycles_per_s = 1024 * 2.4e9
    exp_cyc = probe["exp2"]["cycles_per_wave_group_per_simd"] if probe else 8.7
    fma_cyc = probe["fma"]["cycles_per_wave_group_per_simd"] if probe else 4.0
    transcendentals = w.elements + (2 * rows if w.has_z else 0)
    other_ops = 4 * w.elements + rows * (per_row - (4 if w.has_z else 0))
    out = {"bound": "alu",
           "ceilings_ms": {"hbm_8TBps": alg_bytes / 8e12 * 1e3,
                           "transcendental": transcendentals / 64 * exp_cyc / simd_cycles_per_s * 1e3,
                           "valu_other": other_ops / 64 * fma_cyc / simd_cycles_per_s * 1e3},
           "per_row_ms": rows * per_row / peak_slots * 1e3}
    if probe:
        rate = probe["scan_element"]["lane_groups_per_s"]
        out["measured_element_rate_per_s"] = rate
        out["floor_ms"] = w.elements / rate * 1e3 + out["per_row_ms"]
        out["frac"] = out["floor_ms"] / ms_step
        out["source"] = "ALU probe (kind 2, event-timed) + per-row slots from unit counts"
    return out


def run_probes(log):
    """The ceilings, measured on this GPU: HBM streams (3:1 read:write like the scan's u,
    delta, z -> y; and a plain copy), and the ALU issue probe for fma, exp2 and the scan's
    element group."""
    from selective_state_space_85_amd import probes

    res = {"stream_3r1w": probes.stream_rate(3), "copy_1r1w": probes.stream_rate(1)}
    for kind, name in ((0, "fma"), (1, "exp2"), (2, "scan_element")):
        res[name] = probes.alu_rate(kind)
    log("probes: stream 3:1 %.0f GB/s, copy %.0f GB/s; cycles per wave64 instruction: fma %.2f, exp2 %.2f; "
        "scan element group %.2f" % (res["stream_3r1w"]["GB/s"], res["copy_1r1w"]["GB/s"],
                                     res["fma"]["cycles_per_wave_group_per_simd"],
                                     res["exp2"]["cycles_per_wave_group_per_simd"],
                                     res["scan_element"]["cycles_per_wave_group_per_simd"]))
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CPU_ORACLE_SECONDS = 10.0  # the oracle repeats the whole workload for at least this long


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the scan would shard over batch and channels with no exchange). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as wl
    import selective_state_space_85_amd as ss

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    w = wl.WORKLOADS["large"]

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    log("generating %s inputs (B=%d L=%d D=%d N=%d, %s)" % (w.name, w.batch, w.seqlen, w.dim, w.dstate, w.dtype))
    inp = wl.workload_inputs(w, seed=0)

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)

    t = {k: to_dev(v) for k, v in inp.items()}
    T, K = ss.scan_plan(w.batch, w.seqlen, w.dim, w.dstate)
    ws_bytes = ss.scan_workspace_bytes(w.batch, w.seqlen, w.dim, w.dstate)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
    y = torch.empty_like(t["u"])
    stream = torch.cuda.current_stream(device)

    def step():
        ss.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], out=y, workspace=ws)

    log("plan: chunk_len=%d n_chunks=%d, workspace %d bytes; warmup %d" % (T, K, ws_bytes, args.warmup))
    # settle phase: the step back to back, in groups of 32 between synchronisations, until
    # --settle-ms have passed (untimed; the clock's dip and recovery happen here)
    settle_steps = 0
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    while (time.perf_counter() - c0) * 1e3 < args.settle_ms:
        for _ in range(32):
            step()
        settle_steps += 32
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - c0
    if settle_steps:
        log("settle: %d steps in %.1f ms" % (settle_steps, settle_s * 1e3))
    # the warmup is timed too (reported beside the timed region, not used for the metric)
    ew0 = torch.cuda.Event(enable_timing=True)
    ew1 = torch.cuda.Event(enable_timing=True)
    ew0.record(stream)
    for _ in range(args.warmup):
        step()
    ew1.record(stream)
    torch.cuda.synchronize()
    ms_warm = ew0.elapsed_time(ew1) / args.warmup if args.warmup > 0 else None

    # timed region: K back-to-back steps, events on the launch stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    # the timed output, kept for the CPU-baseline leg's parity check (later sections reuse y)
    y_timed = y.clone()
    log("timed %d steps: %.3f ms/step (events), wall %.3f s" % (args.steps, ms_step, wall))

    elements = w.elements
    alg_bytes = wl.algorithmic_bytes_scan(w.batch, w.seqlen, w.dim, w.dstate, w.dtype, w.has_D, w.has_z)
    achieved_gbs = alg_bytes / (ms_step * 1e-3) / 1e9
    value = elements / (ms_step * 1e-3)
    src_hash = kernel_source_hash()
    traffic = read_traffic(src_hash)

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_ms_per_step": ms_warm,
        "settle": {"ms": settle_s * 1e3, "steps": settle_steps,
                   "note": "untimed back-to-back steps before the warmup, past the clock's dip"},
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; u,B,C,z~N(0,1), delta=softplus(N(-2,1)), A=-(n+1)exp(U(-.5,.5)), D~N(0,1))",
        "config": {"workload": "large-model layer B=8 L=2048 D=5120 N=16, bf16 I/O, fp32 state, D skip + silu(z) gate",
                   "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim, "dstate": w.dstate,
                   "chunk_len": T, "n_chunks": K},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "kernel": "ss_scan_fwd: scan_kernel (emit)%s" % (" + aggregate + carry" if K > 1 else ""),
                     "kernel_source_hash": src_hash,
                     },
    }

    probe = None
    if not args.no_probes:
        probe = run_probes(log)
        result["probes"] = probe
        stream_gbs = probe["stream_3r1w"]["GB/s"]
        result["roofline"]["measured_stream_GB/s"] = stream_gbs
        result["roofline"]["frac_of_measured_stream"] = achieved_gbs / stream_gbs
    result["roofline"]["co_bound"] = alu_cobound(w, ms_step, alg_bytes, probe)

    if not args.no_probes:
        n = 256 << 20  # 1 GiB of fp32 read, 1 GiB written
        a = torch.empty(n, dtype=torch.float32, device=device).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            b.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        result["copy_reference"] = {"bytes_read": n * 4, "bytes_written": n * 4, "ms": ms,
                                    "GB/s": 2 * n * 4 / (ms * 1e-3) / 1e9}
        del a, b

    extras = args.extra_set
    if extras:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)

        def settle(fn, ms=SETTLE_MS):
            # run the workload back to back for a while first: like the timed region's
            # warmup, this times it at the settled clock, not during the ramp after a change
            fn()
            torch.cuda.synchronize()
            c0 = time.perf_counter()
            while (time.perf_counter() - c0) * 1e3 < ms:
                for _ in range(4):
                    fn()
                torch.cuda.synchronize()

        def timed(fn, reps=10):
            settle(fn)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        if "flushed" in extras:
            # the same scan with the last-level cache flushed before each step
            scratch = torch.empty(1 << 28, dtype=torch.float32, device=device)  # 1 GiB
            times = []
            for _ in range(10):
                scratch.fill_(1.0)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step()
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            del scratch
            fl = float(np.median(times))
            result["flushed"] = {"ms_per_step_median": fl, "elements/s": elements / (fl * 1e-3),
                                 "alg_GB/s": alg_bytes / (fl * 1e-3) / 1e9}

        if "options" in extras:
            # the same layer with the step-size / input-term options
            raw = wl.with_raw_delta(inp, seed=0, cfg_id=w.cfg_id)
            dl_raw, bias = to_dev(raw["delta"]), to_dev(raw["delta_bias"])
            opt_res = {}
            for name, kw in (("softplus+bias", dict(delta_softplus=True)), ("zoh", dict(zoh=True)),
                             ("softplus+bias+zoh", dict(delta_softplus=True, zoh=True))):
                sp = kw.get("delta_softplus", False)

                def ostep():
                    ss.scan_fwd(t["u"], dl_raw if sp else t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                out=y, workspace=ws, delta_bias=bias if sp else None, **kw)

                settle(ostep)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(20):
                    ostep()
                e1.record(stream)
                torch.cuda.synchronize()
                oms = e0.elapsed_time(e1) / 20
                opt_res[name] = {"ms_per_step": oms, "elements/s": elements / (oms * 1e-3),
                                 "alg_GB/s": (alg_bytes + 4 * w.dim * sp) / (oms * 1e-3) / 1e9}
            result["options"] = opt_res

        if "backward" in extras:
            # the backward on the same layer
            dy_t = torch.randn(w.batch, w.seqlen, w.dim, device=device, generator=torch.Generator(device).manual_seed(5)
                               ).to(torch.bfloat16)
            bws = torch.empty(ss.scan_bwd_workspace_bytes(w.batch, w.seqlen, w.dim, w.dstate), dtype=torch.uint8,
                              device=device)

            def bstep():
                ss.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy_t, D=t["D"], z=t["z"], workspace=bws)

            settle(bstep)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                bstep()
            e1.record(stream)
            torch.cuda.synchronize()
            bms = e0.elapsed_time(e1) / 10
            del bws

            # training path: the forward keeps every 16th state, the backward reuses them
            ck = torch.empty(ss.scan_ckpt_shape(w.batch, w.seqlen, w.dim, w.dstate), device=device)
            cws = torch.empty(ss.scan_bwd_workspace_bytes(w.batch, w.seqlen, w.dim, w.dstate, with_ckpt=True),
                              dtype=torch.uint8, device=device)
            yk = torch.empty_like(t["u"])

            def fkstep():
                ss.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], out=yk, workspace=ws,
                            ckpt=ck)

            def bkstep():
                ss.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy_t, D=t["D"], z=t["z"], workspace=cws,
                            ckpt=ck)

            fk_ms, bk_ms = timed(fkstep), timed(bkstep)

            # the same training pair under the zero-order-hold input term
            def fzstep():
                ss.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], out=yk, workspace=ws,
                            ckpt=ck, zoh=True)

            def bzstep():
                ss.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy_t, D=t["D"], z=t["z"], workspace=cws,
                            ckpt=ck, zoh=True)

            fz_ms, bz_ms = timed(fzstep), timed(bzstep)
            result["backward"] = {"ms_per_step": bms, "elements/s": elements / (bms * 1e-3),
                                  "vs_forward": bms / ms_step, "note": "panel + checkpoint pass + adjoint + reduce",
                                  "training": {"fwd_ckpt_ms": fk_ms, "bwd_from_ckpt_ms": bk_ms,
                                               "fwd_plus_bwd_ms": fk_ms + bk_ms,
                                               "fwd_plus_standalone_bwd_ms": ms_step + bms,
                                               "ckpt_bytes": ck.numel() * 4,
                                               "note": "ss_scan_fwd_ckpt keeps the state every 16 rows; "
                                                       "ss_scan_bwd_ckpt skips the checkpoint pass"},
                                  "training_zoh": {"fwd_ckpt_ms": fz_ms, "bwd_from_ckpt_ms": bz_ms,
                                                   "fwd_plus_bwd_ms": fz_ms + bz_ms}}
            del ck, cws, yk

        if "configs" in extras:
            # the other scan configurations at their own shapes: the small-model layer and the
            # long context, whose automatic plans cut the sequence into chunks.  Inputs drawn on
            # the device with the configurations' distributions.
            cfgs = {}
            for name in ("small", "long"):
                cw_ = wl.WORKLOADS[name]
                gen = torch.Generator(device).manual_seed(100 + cw_.cfg_id)
                shp = (cw_.batch, cw_.seqlen, cw_.dim)
                tdt = torch.bfloat16 if cw_.dtype == wl.BF16 else torch.float32
                cu_ = torch.randn(shp, device=device, generator=gen).to(tdt)
                cd_ = torch.nn.functional.softplus(torch.randn(shp, device=device, generator=gen) * cw_.delta_sigma
                                                   + cw_.delta_mu).to(tdt)
                cB_ = torch.randn(cw_.batch, cw_.seqlen, cw_.dstate, device=device, generator=gen).to(tdt)
                cC_ = torch.randn(cw_.batch, cw_.seqlen, cw_.dstate, device=device, generator=gen).to(tdt)
                cA_ = to_dev(wl.make_A(cw_.dim, cw_.dstate, cw_.a_perturbed, cfg_id=cw_.cfg_id))
                cD_ = torch.randn(cw_.dim, device=device, generator=gen) if cw_.has_D else None
                cz_ = torch.randn(shp, device=device, generator=gen).to(tdt) if cw_.has_z else None
                cy_ = torch.empty_like(cu_)
                cT, cK = ss.scan_plan(cw_.batch, cw_.seqlen, cw_.dim, cw_.dstate)
                cws = torch.empty(max(ss.scan_workspace_bytes(cw_.batch, cw_.seqlen, cw_.dim, cw_.dstate), 1),
                                  dtype=torch.uint8, device=device)

                def cstep_():
                    ss.scan_fwd(cu_, cd_, cA_, cB_, cC_, D=cD_, z=cz_, out=cy_, workspace=cws)

                # calls of tens of microseconds: enough of them to average over the clock's moves
                cms = timed(cstep_, reps=400 if name == "small" else 20)
                cel = cw_.batch * cw_.seqlen * cw_.dim * cw_.dstate
                cby = wl.algorithmic_bytes_scan(cw_.batch, cw_.seqlen, cw_.dim, cw_.dstate, cw_.dtype, cw_.has_D,
                                                cw_.has_z)
                cfgs[name] = {"workload": "%s: B=%d L=%d D=%d N=%d, %s" % (cw_.note, cw_.batch, cw_.seqlen, cw_.dim,
                                                                          cw_.dstate, cw_.dtype),
                              "chunk_len": cT, "n_chunks": cK, "ms_per_call": cms, "elements/s": cel / (cms * 1e-3),
                              "alg_GB/s": cby / (cms * 1e-3) / 1e9,
                              "frac_of_8TB/s": cby / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS}
                del cu_, cd_, cB_, cC_, cz_, cy_, cws
            result["configs"] = cfgs

        if "conv1d" in extras:
            # the block's causal depthwise convolution + SiLU producing u (x read in place from xz)
            xz = torch.randn(w.batch, w.seqlen, 2 * w.dim, device=device,
                             generator=torch.Generator(device).manual_seed(6)).to(torch.bfloat16)
            cw = torch.randn(w.dim, 4, device=device, generator=torch.Generator(device).manual_seed(7)) * 0.5
            cb = torch.randn(w.dim, device=device, generator=torch.Generator(device).manual_seed(8))
            cu = torch.empty(w.batch, w.seqlen, w.dim, dtype=torch.bfloat16, device=device)

            def cstep():
                ss.conv1d_silu(xz[..., :w.dim], cw, cb, out=cu)

            settle(cstep)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                cstep()
            e1.record(stream)
            torch.cuda.synchronize()
            cms = e0.elapsed_time(e1) / 20
            cbytes = 2 * 2 * w.batch * w.seqlen * w.dim + 4 * w.dim * 5  # x read + u written (bf16), weights, bias
            cgbs = cbytes / (cms * 1e-3) / 1e9
            result["conv1d"] = {"workload": "B=8 L=2048 D=5120 bf16, width 4, x = first half of xz (B, L, 2D)",
                                "ms": cms, "alg_bytes": cbytes, "alg_GB/s": cgbs, "frac_of_8TB/s": cgbs / HBM_PEAK_GBS}
            del xz, cu

        if "ssd" in extras:
            # the multi-head (Mamba-2) recurrence on the matrix cores
            sb, sl, sh, sn = 8, 2048, 64, 128
            si = wl.ssd_inputs(sb, sl, sh, 64, sn, seed=0)
            stt = {k: to_dev(v) for k, v in si.items() if v is not None}
            sy = torch.empty_like(stt["x"])

            def sstep():
                ss.ssd_fwd(stt["x"], stt["dt"], stt["A"], stt["B"], stt["C"], D=stt["D"], out=sy)

            settle(sstep)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                sstep()
            e1.record(stream)
            torch.cuda.synchronize()
            sms = e0.elapsed_time(e1) / 20
            sbytes = wl.algorithmic_bytes_ssd(sb, sl, sh, 64, sn)
            # executed bf16 MFMA 32x32x16 per 64-row chunk and head: 24 (C B^T, upper block skipped)
            # + 64 (C S_in, hi + lo) + 24 (M X, hi + lo, upper half skipped) + 64 (state, hi + lo)
            sflops = 176 * 32 * 32 * 16 * 2 * (sl // 64) * sb * sh
            result["ssd"] = {"workload": "B=8 L=2048 H=64 headdim=64 dstate=128 bf16, D skip",
                             "ms": sms, "alg_bytes": sbytes, "alg_GB/s": sbytes / (sms * 1e-3) / 1e9,
                             "frac_of_8TB/s": sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "mfma_TFLOP/s": sflops / (sms * 1e-3) / 1e12,
                             "frac_of_2.5PF": sflops / (sms * 1e-3) / 2.5e15}
            del stt, sy

            # the same layer at dstate 256: a launch per half of the state entries, the second
            # adding the first's fp32 part of y to its own
            si = wl.ssd_inputs(sb, sl, sh, 64, 256, seed=0)
            stt = {k: to_dev(v) for k, v in si.items() if v is not None}
            sy = torch.empty_like(stt["x"])
            sws = torch.empty(ss.ssd_workspace_bytes(sb, sl, sh, 64, 256), dtype=torch.uint8, device=device)

            def sstep256():
                ss.ssd_fwd(stt["x"], stt["dt"], stt["A"], stt["B"], stt["C"], D=stt["D"], out=sy, workspace=sws)

            settle(sstep256)
            e0.record(stream)
            for _ in range(20):
                sstep256()
            e1.record(stream)
            torch.cuda.synchronize()
            result["ssd"]["dstate256"] = {"ms": e0.elapsed_time(e1) / 20,
                                          "alg_bytes": wl.algorithmic_bytes_ssd(sb, sl, sh, 64, 256)}
            del stt, sy, sws

        if "decode" in extras:
            # recurrent step workload: one token for B=256, D=5120, state in place
            sw = wl.WORKLOADS["step"]
            sp = wl.step_params(sw)
            si = wl.step_inputs(sw, 0)
            st = {k: to_dev(v) for k, v in si.items()}
            A5, D5, h5 = to_dev(sp["A"]), to_dev(sp["D"]), to_dev(sp["h0"])
            y5 = torch.empty_like(st["u"])

            def dstep():
                ss.step(h5, st["u"], st["delta"], A5, st["B"], st["C"], D=D5, z=st["z"], out=y5)

            settle(dstep)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(100):
                dstep()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / 100
            sb = wl.algorithmic_bytes_step(sw.batch, sw.dim, sw.dstate, sw.dtype, sw.has_D, sw.has_z)
            # cold: the 256 MB last-level cache flushed before each token (median of 20)
            scratch = torch.empty(1 << 28, dtype=torch.float32, device=device)
            cold = []
            for _ in range(20):
                scratch.fill_(1.0)
                e0.record(stream)
                dstep()
                e1.record(stream)
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1) * 1e3)
            del scratch
            us_cold = float(np.median(cold))
            # 1000 chained tokens, each with fresh operands (drawn on the device beforehand,
            # with the step workload's distributions), timed as one run
            n_chain = 1000
            cg = torch.Generator(device).manual_seed(500)
            shp_c = (n_chain, sw.batch, sw.dim)
            cu = torch.randn(shp_c, device=device, generator=cg).to(torch.bfloat16)
            cd = torch.nn.functional.softplus(torch.randn(shp_c, device=device, generator=cg) - 2.0).to(torch.bfloat16)
            cz = torch.randn(shp_c, device=device, generator=cg).to(torch.bfloat16)
            cB = torch.randn(n_chain, sw.batch, sw.dstate, device=device, generator=cg).to(torch.bfloat16)
            cC = torch.randn(n_chain, sw.batch, sw.dstate, device=device, generator=cg).to(torch.bfloat16)
            cy = torch.empty_like(cu)
            ch = h5.clone()
            torch.cuda.synchronize()
            e0.record(stream)
            for k in range(n_chain):
                ss.step(ch, cu[k], cd[k], A5, cB[k], cC[k], D=D5, z=cz[k], out=cy[k])
            e1.record(stream)
            torch.cuda.synchronize()
            us_chain = e0.elapsed_time(e1) * 1e3 / n_chain
            del cu, cd, cz, cB, cC, cy, ch
            result["decode_step"] = {"workload": "recurrent step B=256 D=5120 N=16, bf16, state (84 MB) in place",
                                     "us_per_token": us, "elements/s": sw.elements / (us * 1e-6),
                                     "alg_GB/s": sb / (us * 1e-6) / 1e9,
                                     "note": "chained on the same operands, state warm in cache",
                                     "cold_us_per_token": us_cold, "cold_alg_GB/s": sb / (us_cold * 1e-6) / 1e9,
                                     "cold_frac_of_8TB/s": sb / (us_cold * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                     "chained_1000_us_per_token": us_chain,
                                     "chained_1000_alg_GB/s": sb / (us_chain * 1e-6) / 1e9,
                                     "chained_1000_note": "1000 tokens in one run, fresh operands per token"}
            del st, y5, h5

            # single-sequence decode (B=1): launch-bound, so the token loop is captured
            # once in a hipGraph and replayed, against the same loop launched eagerly
            n_tok, gd = 64, 5120
            gi = wl.scan_inputs(1, n_tok, gd, 16, wl.BF16, has_D=True, has_z=True, has_h0=True, seed=77)
            gt = {k: to_dev(v) for k, v in gi.items()}
            gcol = {k: [gt[k][:, s].contiguous() for s in range(n_tok)] for k in ("u", "delta", "B", "C", "z")}
            gh = gt["h0"].clone()
            gy = torch.empty(n_tok, 1, gd, dtype=torch.bfloat16, device=device)

            def gloop():
                for s_ in range(n_tok):
                    ss.step(gh, gcol["u"][s_], gcol["delta"][s_], gt["A"], gcol["B"][s_], gcol["C"][s_], D=gt["D"],
                            z=gcol["z"][s_], out=gy[s_])

            def per_token(fn, reps=10):
                fn()
                torch.cuda.synchronize()
                e0.record(torch.cuda.current_stream())
                for _ in range(reps):
                    fn()
                e1.record(torch.cuda.current_stream())
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / (reps * n_tok)

            us_eager = per_token(gloop)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                gloop()
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                gloop()
            torch.cuda.synchronize()
            us_graph = per_token(graph.replay)
            result["decode_graph"] = {"workload": "recurrent step B=1 D=5120 N=16, bf16, D skip + gate, %d tokens "
                                                  "per hipGraph" % n_tok,
                                      "eager_us_per_token": us_eager, "graph_us_per_token": us_graph}
            del graph, gt, gcol, gy, gh

    # the CPU-baseline leg: the oracle checks the timed output on every channel, and (unless
    # skipped) is timed on this host's cores, all threads and one thread
    import oracle
    host_cores = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = host_cores
    threads = min(16, usable)
    log("parity: the oracle over every channel of the timed output (%d threads)" % threads)
    c0 = time.perf_counter()
    ref = oracle.scan(**inp, threads=threads)["y"]
    parity_s = time.perf_counter() - c0
    yb = y_timed.view(torch.int16).cpu().numpy().view(np.uint16)
    yg = (yb.astype(np.uint32) << 16).view(np.float32)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = 0.0
    for bi in range(w.batch):  # one batch row at a time keeps the temporaries small
        d_ = np.abs(yg[bi].astype(np.float64) - ref[bi]) / np.maximum(np.abs(ref[bi]), rms)
        err = max(err, float(d_.max()))
    del ref, yb, yg
    result["parity"] = {"max_rel_err": err, "tol": 2e-2, "lanes": int(w.batch * w.dim), "all_lanes": True,
                        "oracle_seconds": parity_s, "ok": bool(err <= 2e-2)}
    log("parity: max rel err %.3e over all %d channels" % (err, w.batch * w.dim))
    if not args.no_cpu_baseline:
        lanes = np.arange(w.batch * w.dim, dtype=np.int64)
        log("timing the CPU oracle on %d channels x %d steps, %d threads, for at least %.0f s"
            % (lanes.size, w.seqlen, threads, CPU_ORACLE_SECONDS))
        reps = 0
        c0 = time.perf_counter()
        while reps == 0 or time.perf_counter() - c0 < CPU_ORACLE_SECONDS:
            oracle.scan(**inp, lanes=lanes, threads=threads)
            reps += 1
        cdt = time.perf_counter() - c0
        n_el = lanes.size * w.seqlen * w.dstate
        # one thread on a bounded sample: the first 512 channels of batch row 0
        one = np.arange(512, dtype=np.int64)
        reps1 = 0
        c1 = time.perf_counter()
        while reps1 == 0 or time.perf_counter() - c1 < 3.0:
            oracle.scan(**inp, lanes=one, threads=1)
            reps1 += 1
        cdt1 = time.perf_counter() - c1
        n_el1 = one.size * w.seqlen * w.dstate
        result["cpu_baseline"] = {
            "value": reps * n_el / cdt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": "the whole large-layer workload (%d channels x %d steps x %d states = %d elements), fp64, "
                      "%d threads, %d passes in %.1f s" % (lanes.size, w.seqlen, w.dstate, n_el, threads, reps, cdt),
            "threads": threads, "host_cores": host_cores, "usable_cores": usable, "cpu_model": cpu_model(),
            "single_thread": {"value": reps1 * n_el1 / cdt1, "unit": "elements/s", "threads": 1,
                              "sample": "512 channels of batch row 0 x %d steps x %d states = %d elements, "
                                        "%d passes in %.1f s" % (w.seqlen, w.dstate, n_el1, reps1, cdt1)}}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
