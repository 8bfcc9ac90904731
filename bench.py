#!/usr/bin/env python3
"""Benchmark of the KDA forward operator on one MI355X.

One step is one pass of the whole hot path: a chunked prefill call on the
8K workload (one sequence, T = 8192, H = 32, d_k = d_v = 128, bf16 q/k/v,
fp32 gates and state, h0 = 0) followed by one decode step on the decode
workload (256 sequences x 32 heads, fp32 states of 512 MiB updated in place).
Inputs are synthetic (seeded generators), resident in HBM before timing;
every input set is drawn before the first timed call.

Printed: ONE JSON line. ``value`` is prefill tokens/s (T / mean prefill call
time from HIP events on the caller's stream); decode tokens/s is reported
beside it. ``roofline`` is the prefill call's (the headline path: algorithmic
bytes of the call over its mean duration, with the call's measured HBM
traffic from the committed counter summary), ``decode_roofline`` the decode
step's. ``timing`` gives the median, p10 and p90 of the timed calls and of
prefill calls made with cold inputs (each after a 1 GiB scrub write). After
the timed steps the prefill's kernels are also launched one at a time (phase
entry point) to measure each kernel's own duration (``kernels``).

``long_configs``: the prefill on the long single sequence (T = 131072, strong
decay, nonzero h0) and on the 16-sequence packed batch, each with its own
roofline and traffic. ``sweep_h16``: one sequence of 16 heads at T = 2K ..
64K, the shape of the pages' kernel-speed figure (their times are quoted as
context; the pages do not name the hardware), and at 2^20 tokens.

``extensions`` times the operator's optional paths, each on its own
workload with its own roofline: the fused multi-token recurrent call
(256 sequences x 32 heads x L = 4 and 64 new tokens; the L = 64 batch also
through the chunked path, which is the faster one there), the decode step with a
bf16 state, batch-1 decode (one sequence x 32 heads) launched step by step
and replayed from a HIP graph, the prefill with in-kernel q/k L2Norm, the 8K
prefill continuing a bf16 state in place, the 8K prefill with fp32 I/O, the 8K prefill with decays strong enough that every
chunk takes the exact per-element diagonal blocks, and the RMSNorm x
sigmoid-gate epilogue over the prefill's 8192 x 32 output rows.

``probes`` holds what plain kernels (probes/ceilings.hip) reach on the same
GPU: streaming read, copy, in-place update, bf16 MFMA and fp32 FMA loops.
They are reference rates, not ceilings: a roofline object carries
``frac_achievable`` only where its probe is at least as fast as the kernel.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-long-configs]
                    [--no-sweep] [--only WORKLOAD]

``--only`` times one workload's prefill calls and nothing else (for counter
runs): bench_step, long_T131072, packed_16_sequences.
With KDA_ROCTX=1 each timed call is wrapped in a named roctx range
(kda_chunk_fwd, kda_decode_step) for rocprofv3 --marker-trace.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import numpy as np

METRIC = "KDA prefill tokens/s (H=32,d=128,T=8K) + decode tokens/s; % MFMA/HBM peak"
ROOT = Path(__file__).resolve().parent
PROFILES = ROOT / "profiles"
COPY_BYTES = 1 << 30        # the calibration copy reads and writes 1 GiB
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
D, C = 128, 64

# Algorithmic bytes and FLOPs (bf16 I/O). Per token-head of prefill:
# q, k, v 256 B each, log_alpha 512 B, beta 4 B, o 256 B.
PREFILL_IN_BYTES = 3 * 256 + 512 + 4     # read by the intra-chunk kernel
PREFILL_OUT_BYTES = 256                  # o, written by the carry kernel
PREFILL_BYTES = PREFILL_IN_BYTES + PREFILL_OUT_BYTES   # 1540
STATE_BYTES = D * D * 4
FLOPS_EQ13 = 6 * D * D + 3 * C * D + C * C             # 126976 per token-head
FLOPS_DENSE = 6 * D * D + 10 * C * D                   # 180224 per token-head
# Decode, per (sequence, head): state read + write, q/k/v, log_alpha, beta, o.
TOKEN_BYTES = 3 * 256 + 512 + 4 + 256                      # 1540 per token-head
DECODE_BYTES = 2 * STATE_BYTES + TOKEN_BYTES               # 132612
# Recurrent path, per token-head: S~^T k and S~^T q (2 d^2 each as FMAs),
# the decay a*s (d^2) and the rank-1 correction (2 d^2).
FLOPS_RECURRENT = 7 * D * D                                # 114688
# fp32 vector peak, as published for MI355X: 256 CUs x 256 flops per cycle x
# 2.4 GHz. Plain (unpacked) FMAs reach it too on this chip: a loop of
# independent v_fma_f32 measures about 124 TFLOP/s at the 2.2 GHz the
# shader clock holds under load (the FMA probe reports it per run).
FP32_VALU_TFLOPS = 256 * 256 * 2.4e9 / 1e12                 # 157.3
# Epilogue, per row of 128 channels (bf16): o and gate read, y written.
EPILOGUE_BYTES = 3 * 256


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing on the host cores")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline sample")
    ap.add_argument("--no-extensions", action="store_true",
                    help="skip the timings of the optional paths (shorter counter runs)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the plain-kernel probes of achievable bandwidth and FLOP rate")
    ap.add_argument("--no-long-configs", action="store_true",
                    help="skip the prefill on the long single sequence (T = 131072) and the "
                         "16-sequence packed batch (their inputs take about a minute to draw)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 16-head length sweep")
    ap.add_argument("--only", choices=("bench_step", "long_T131072", "packed_16_sequences"),
                    help="time only this workload's prefill calls (counter runs)")
    ap.add_argument("--workload", default="bench_step",
                    help="workload name written by --summarize-pmc")
    ap.add_argument("--calls", type=int, default=3,
                    help="calls the summarised counter runs made (steps + warmup)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy first (counter scale factor)")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="turn one rocprofv3 --pmc run of the MFMA counters (MFMA_COUNTERS) of "
                         "this script into a table; --durations adds rates")
    ap.add_argument("--durations", metavar="KERNEL=US", nargs="*", default=None,
                    help="traced mean duration per launch, e.g. intra=158.5 carry=131.5")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script with --copy-calibration into the traffic summary text")
    return ap.parse_args()


def sources_hash() -> str:
    """Hash of the kernel sources: counter readings apply only to this code."""
    h = hashlib.sha256()
    for f in sorted((ROOT / "gated_delta_rule_50_amd" / "csrc").glob("*")):
        h.update(f.name.encode())
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def _kernel_key(name):
    """Kernel a counter row belongs to. The counter passes run with --only,
    so the only recurrent-kernel dispatches are the decode step's
    (profilers print these template names mangled or demangled, and not
    always faithfully, so only the base name is matched)."""
    if "recurrent_fwd_kernel" in name:
        return "decode"
    for k in ("intra", "carry", "chunk_map"):
        if k in name:
            return k
    # device-to-device copies (the runtime's blit kernel for torch's copy_)
    return "copy" if "copy" in name.lower() else None


def _pmc_per_call(run_dir, counter, calls):
    """Counter value (KiB) per call of each kernel in one pmc run: the sum
    over the kernel's dispatches divided by the calls the run made (a
    windowed prefill launches its kernels once per window); for 'copy', the
    largest dispatch (the 1 GiB calibration copy)."""
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            k = _kernel_key(row["Kernel_Name"])
            if k is None:
                continue
            per.setdefault(k, {}).setdefault(row["Dispatch_Id"], 0.0)
            per[k][row["Dispatch_Id"]] += float(row["Counter_Value"])
    out = {k: (max(v.values()) if k == "copy" else sum(v.values()) / calls)
           for k, v in per.items()}
    out["_dispatches"] = {k: len(v) for k, v in per.items()}
    return out


def summarize_pmc(fetch_dir, write_dir, workload, calls):
    f = _pmc_per_call(fetch_dir, "FETCH_SIZE", calls)
    w = _pmc_per_call(write_dir, "WRITE_SIZE", calls)
    fr = COPY_BYTES / (f["copy"] * 1024.0)
    wr = COPY_BYTES / (w["copy"] * 1024.0)
    lines = [f"workload = {workload}", f"sources_sha256 = {sources_hash()}",
             f"calls = {calls}", f"copy_read_factor = {fr:.6f}",
             f"copy_write_factor = {wr:.6f}"]
    for k in ("chunk_map", "intra", "carry", "decode"):
        if k in f and k in w:
            lines.append(f"{k}_dispatches = {f['_dispatches'][k]}")
            lines.append(f"{k}_fetch_KiB = {f[k]:.1f}")
            lines.append(f"{k}_write_KiB = {w[k]:.1f}")
    print("\n".join(lines))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F32", "GRBM_GUI_ACTIVE", "MfmaUtil")
N_SIMDS, N_XCDS = 256 * 4, 8


def summarize_mfma(run_dir, durations_us=None):
    """Matrix-core use per launch of each kernel from one rocprofv3 --pmc run
    of MFMA_COUNTERS. The profiler writes one value per dispatch and counter,
    summed over the counter's instances: GRBM_GUI_ACTIVE (one per XCD) is
    therefore divided by the XCD count to give the launch's active cycles.
    MFMA busy is the profiler's own MfmaUtil (summed MFMA-busy cycles over
    active cycles x SIMDs); flops count 512 per MOP. With durations (us per
    launch of each kernel, from a kernel trace) the flops become rates
    against the dense peaks (bf16 2.5 PFLOP/s, fp32 matrix 157.3 TFLOP/s)."""
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            k, c = _kernel_key(row["Kernel_Name"]), row["Counter_Name"]
            if k is None or c not in MFMA_COUNTERS:
                continue
            dd = per.setdefault(k, {}).setdefault(row["Dispatch_Id"], {})
            dd[c] = dd.get(c, 0.0) + float(row["Counter_Value"])
    lines = ["| kernel | dispatches | active cycles per XCD | MfmaUtil (%) | bf16 MFMA flops "
             "| fp32 MFMA flops | bf16 TFLOP/s (of 2500) | fp32 TFLOP/s (of 157.3) |",
             "|---|---|---|---|---|---|---|---|"]
    for k in ("intra", "carry", "decode", "chunk_map"):
        if k not in per:
            continue
        ds = [d for d in per[k].values() if all(c in d for c in MFMA_COUNTERS)]
        mean = {c: float(np.mean([d[c] for d in ds])) for c in MFMA_COUNTERS}
        bf = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        f32 = mean["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512
        rb = rf = "-"
        if durations_us and k in durations_us:
            sec = durations_us[k] * 1e-6
            rb = f"{bf / sec / 1e12:.1f} ({bf / sec / 1e12 / BF16_PEAK_TFLOPS:.3f})"
            rf = f"{f32 / sec / 1e12:.1f} ({f32 / sec / 1e12 / 157.3:.3f})"
        lines.append(f"| {k} | {len(ds)} | {mean['GRBM_GUI_ACTIVE'] / N_XCDS:.0f} | "
                     f"{mean['MfmaUtil']:.2f} | {bf:.4g} | {f32:.4g} | {rb} | {rf} |")
    print("\n".join(lines))


def load_traffic(workload="bench_step"):
    """Scaled HBM bytes per call for each kernel of a workload, from the
    committed counter summary profiles/hbm_traffic_<workload>.txt, or {} if
    there is none or it was taken on other kernel sources."""
    path = PROFILES / f"hbm_traffic_{workload}.txt"
    if not path.exists():
        return {}
    kv = {}
    for line in path.read_text().splitlines():
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = (x.strip() for x in line.split("=", 1))
            kv[key] = val
    if kv.get("sources_sha256") != sources_hash():
        return {}
    fr, wr = float(kv["copy_read_factor"]), float(kv["copy_write_factor"])
    out = {}
    for k in ("chunk_map", "intra", "carry", "decode"):
        if f"{k}_fetch_KiB" in kv:
            out[k] = (float(kv[f"{k}_fetch_KiB"]) * fr + float(kv[f"{k}_write_KiB"]) * wr) * 1024
    return out


def prefill_traffic(traffic):
    """Bytes one prefill call moves (its kernels' counter readings), or None."""
    if "intra" not in traffic or "carry" not in traffic:
        return None
    return sum(traffic.get(k, 0.0) for k in ("chunk_map", "intra", "carry"))


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def copy_calibration(torch):
    """A plain device copy of 1 GiB (reads 1 GiB, writes 1 GiB), three times,
    so hardware byte counters can be scaled against a known transfer."""
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def cpu_baseline(p, seconds):
    """The fp64 oracle, as it stands, on the prefill workload (all heads),
    repeated until at least `seconds` of wall time; plus one decode step of
    the decode workload."""
    from oracle import recurrent
    from gated_delta_rule_50_amd import workloads
    threads = recurrent.host_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, None, p.cu_seqlens,
                          threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    cfg = workloads.config(4)
    S0 = workloads.make_decode_state(cfg.n_seqs, cfg.H, cfg.seed)
    d = workloads.make_decode_step(cfg.n_seqs, cfg.H, cfg.seed, 0, io=cfg.io)
    t1 = time.perf_counter()
    recurrent.decode_step(d.q, d.k, d.v, d.log_alpha, d.beta, S0, threads=threads)
    ddt = time.perf_counter() - t1
    return {"value": reps * p.T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"prefill workload (T={p.T}, H={p.H}, all heads) x {reps}, "
                      f"fp64 recurrence, {dt:.1f} s; decode: one step of "
                      f"{cfg.n_seqs}x{cfg.H} states in {ddt:.2f} s",
            "decode_value": cfg.n_seqs / ddt}


def _time_calls(torch, fn, steps, warmup):
    """Mean duration (us) of fn() from events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = _events(torch, steps + 1)
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])) * 1e3


def _spread(ms):
    """Median, p10 and p90 (us) of per-call durations in ms."""
    us = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median_us": float(np.median(us)), "p10_us": float(np.percentile(us, 10)),
            "p90_us": float(np.percentile(us, 90))}


def cold_prefill(torch, pre, reps):
    """Prefill calls each preceded by writing a 1 GiB scrub buffer, which
    evicts the inputs from the 256 MiB memory-side cache (the 8K workload's
    inputs are 337 MB, so a warm repeat finds part of them there). Returns
    the per-call spread (us) of the prefill alone."""
    scrub = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    ev = [_events(torch, 2) for _ in range(reps)]
    for i in range(reps):
        scrub.fill_(float(i))
        ev[i][0].record()
        pre.run()
        ev[i][1].record()
    torch.cuda.synchronize()
    del scrub
    return _spread([e[0].elapsed_time(e[1]) for e in ev])


def probes(torch):
    """Rates plain kernels reach on this GPU (probes/ceilings.hip): streaming
    read, nontemporal copy and in-place update of 1 GiB buffers, a bf16 MFMA
    loop and an fp32 FMA loop. Median of five launches each, HIP events on
    the launch stream."""
    import ctypes
    from probes.build import LIB as PROBE_LIB
    if not PROBE_LIB.exists():
        raise RuntimeError(f"{PROBE_LIB} is not built; run `python -m probes.build`")
    L = ctypes.CDLL(str(PROBE_LIB))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.kdab_read.argtypes = [vp, i64, vp, i32, vp]
    L.kdab_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    L.kdab_rmw.argtypes = [vp, i64, i32, vp]
    L.kdab_mfma.argtypes = [vp, i64, i32, vp]
    L.kdab_valu.argtypes = [vp, i64, i32, vp]
    nbytes = COPY_BYTES
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a).fill_(0.0)
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    pa, pb, ps = ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), \
        ctypes.c_void_p(sink.data_ptr())

    def med_us(launch, reps=5):
        launch()
        ev = [_events(torch, 2) for _ in range(reps)]
        for e in ev:
            e[0].record()
            rc = launch()
            e[1].record()
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e3

    grids = (1024, 2048, 4096, 8192)   # best over launch sizes
    out = {
        "hbm_read_GBps": max(nbytes / med_us(lambda: L.kdab_read(pa, nbytes, ps, g, st))
                             for g in grids) / 1e3,
        "hbm_copy_GBps": max(2 * nbytes / med_us(lambda: L.kdab_copy(pa, pb, nbytes, 1, g, st))
                             for g in grids) / 1e3,
        "hbm_rmw_GBps": max(2 * nbytes / med_us(lambda: L.kdab_rmw(pa, nbytes, g, st))
                            for g in grids) / 1e3,
    }
    # 2048 workgroups of four waves: eight waves per SIMD
    iters, wg = 4000, 2048
    flops = wg * 4 * 8 * iters * (2 * 16 * 16 * 32)
    out["mfma_bf16_TFLOPs"] = flops / med_us(lambda: L.kdab_mfma(ps, iters, wg, st)) / 1e6
    wg = 4096
    flops = wg * 256 * 32 * iters * 2
    out["valu_fp32_TFLOPs"] = flops / med_us(lambda: L.kdab_valu(ps, iters, wg, st)) / 1e6
    del a, b, sink
    out["note"] = ("rates of plain grid-stride kernels on this GPU, for reference: roofline "
                   "fractions use the published peaks; a roofline carries frac_achievable "
                   "against the probe of its kind only where the probe is at least as fast "
                   "as the kernel (the decode step and the epilogue outrun these probes)")
    return out


def _with_probe(roof, probe, key):
    """Adds the probe rate of the same kind to a roofline object, and the
    fraction of it only when the probe bounds the kernel."""
    if probe and key in probe:
        roof["probe"] = probe[key]
        if roof["achieved"] <= probe[key]:
            roof["frac_achievable"] = roof["achieved"] / probe[key]
        else:
            roof["exceeds_probe"] = True
    return roof


def _hbm(alg_bytes, us, traffic=None):
    gbps = alg_bytes / (us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic}
    if traffic is not None:
        roof["traffic_ratio"] = traffic / alg_bytes
    return roof


def prefill_alg_bytes(T, H, N, io_bytes=2, h0=False):
    """Algorithmic bytes of one prefill call: per token-head q, k, v, o in
    the I/O type, log_alpha fp32 and beta fp32; per (sequence, head) h_final
    (and h0 when given)."""
    per_th = 4 * D * io_bytes + D * 4 + 4
    return T * H * per_th + (2 if h0 else 1) * N * H * STATE_BYTES


def extensions(torch, d, pre_args, steps, warmup, extra=None, us_8k=None):
    """Timings of the optional paths (module docstring), inputs resident.
    extra: device inputs of the fp32 and exact-diagonal 8K prefills."""
    from gated_delta_rule_50_amd import (Decode, Prefill, Recurrent, decode_step, rmsnorm_gate,
                                         workloads)
    bf = torch.bfloat16
    out = {}
    N, H = 256, 32
    for L in (4, 64):
        p = workloads.make_prefill([L] * N, H, seed=2000 + L, io="bf16", h0_std=0.02)
        ins = (d(p.q, bf), d(p.k, bf), d(p.v, bf), d(p.log_alpha), d(p.beta))
        S = d(p.h0)
        rec = Recurrent(*ins, S, None, n_seqs=N, h_final=S)
        us = _time_calls(torch, rec.run, steps, warmup)
        alg = N * H * (2 * STATE_BYTES + L * TOKEN_BYTES)
        tf = N * H * L * FLOPS_RECURRENT / (us * 1e-6) / 1e12
        roof = _hbm(alg, us) if L <= 8 else {
            "bound": "alu", "achieved": tf, "peak": FP32_VALU_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / FP32_VALU_TFLOPS}
        out[f"recurrent_L{L}"] = {
            "workload": f"{N} sequences x {H} heads x {L} new tokens, bf16 q/k/v, fp32 states "
                        f"~N(0,0.02) updated in place", "us": us,
            "tokens_per_s": N * L / (us * 1e-6), "alg_bytes": alg,
            "tflops": tf, "roofline": roof}
        if L == 64:
            # the same batch through the chunked path (its short-sequence
            # carry): from 40 tokens per sequence on the faster of the two
            pre = Prefill(*ins, d(p.h0), d(p.cu_seqlens, torch.int32))
            us = _time_calls(torch, pre.run, steps, warmup)
            out["chunked_L64"] = {
                "workload": f"the L = 64 batch through kda_chunk_fwd (packed, {N} sequences)",
                "us": us, "tokens_per_s": N * L / (us * 1e-6), "alg_bytes": alg,
                "roofline": _hbm(alg, us)}
            del pre
        del p, ins, S, rec
    cfg4 = workloads.config(4)
    ds = workloads.make_decode_step(cfg4.n_seqs, cfg4.H, cfg4.seed, 0, io=cfg4.io)
    Sb = d(workloads.make_decode_state(cfg4.n_seqs, cfg4.H, cfg4.seed), bf)
    rec = Recurrent(d(ds.q, bf), d(ds.k, bf), d(ds.v, bf), d(ds.log_alpha), d(ds.beta), Sb,
                    None, n_seqs=cfg4.n_seqs, state_dtype=bf, h_final=Sb)
    us = _time_calls(torch, rec.run, steps, warmup)
    alg = cfg4.n_seqs * cfg4.H * (STATE_BYTES + TOKEN_BYTES)
    out["decode_bf16_state"] = {
        "workload": f"decode step {cfg4.n_seqs}x{cfg4.H}, bf16 states updated in place",
        "us": us, "tokens_per_s": cfg4.n_seqs / (us * 1e-6), "alg_bytes": alg,
        "roofline": _hbm(alg, us)}
    del Sb, rec
    # batch-1 decode (one sequence x 32 heads) is launch-bound: 64 steps
    # launched one by one, and the same 64 steps replayed from a HIP graph
    N1, steps1 = 1, 64
    S1 = d(workloads.make_decode_state(N1, cfg4.H, cfg4.seed))
    toks = []
    for st in range(steps1):
        t = workloads.make_decode_step(N1, cfg4.H, cfg4.seed, st, io=cfg4.io)
        toks.append((d(t.q, bf), d(t.k, bf), d(t.v, bf), d(t.log_alpha), d(t.beta)))
    o1 = torch.empty((N1, cfg4.H, D), dtype=bf, device="cuda")

    def loop():
        for t in toks:
            decode_step(*t, S1, o=o1)
    us_eager = _time_calls(torch, loop, steps, warmup) / steps1
    # the same steps bound once (Decode): one library call per token
    bound = [Decode(*t, S1, o=o1) for t in toks]

    def loop_bound():
        for b in bound:
            b.run()
    us_bound = _time_calls(torch, loop_bound, steps, warmup) / steps1
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        loop()
    us_graph = _time_calls(torch, graph.replay, steps, warmup) / steps1
    alg = N1 * cfg4.H * DECODE_BYTES
    out["decode_batch1"] = {
        "workload": f"decode, 1 sequence x {cfg4.H} heads, fp32 state, {steps1} steps per "
                    "launch sequence", "us_per_token_eager": us_eager,
        "us_per_token_bound": us_bound,
        "us_per_token_graph": us_graph, "tokens_per_s_graph": 1.0 / (us_graph * 1e-6),
        "alg_bytes": alg, "roofline": _hbm(alg, us_graph)}
    del S1, toks, graph, bound
    pre_n = Prefill(*pre_args, qk_l2norm=True)
    us = _time_calls(torch, pre_n.run, steps, warmup)
    out["prefill_qk_l2norm"] = {
        "workload": "the 8K prefill with KDA_FLAG_QK_L2NORM", "us": us,
        "tokens_per_s": pre_args[0].shape[0] / (us * 1e-6)}
    o = pre_n.o
    # the serving state format: the 8K prefill continuing a bf16 state in
    # place (h0 = h_final, KDA_FLAG_STATE_BF16)
    T8, H8 = pre_args[0].shape[0], pre_args[0].shape[1]
    Sb8 = d(workloads.make_decode_state(1, H8, seed=2100), bf)
    pre_b = Prefill(*pre_args[:5], Sb8, pre_args[6], h_final=Sb8, state_dtype=bf)
    us = _time_calls(torch, pre_b.run, steps, warmup)
    alg = prefill_alg_bytes(T8, H8, 1, 2) - H8 * STATE_BYTES + 2 * H8 * STATE_BYTES // 2
    out["prefill_bf16_state"] = {
        "workload": "the 8K prefill continuing a bf16 state ~N(0,0.02) in place "
                    "(KDA_FLAG_STATE_BF16)", "us": us,
        "tokens_per_s": T8 / (us * 1e-6), "alg_bytes": alg, "roofline": _hbm(alg, us)}
    del pre_b, Sb8
    for name, what in (("fp32_8k", "the 8K x 32-head prefill with fp32 q/k/v/o (fp32 "
                                    "intermediates)"),
                       ("exact_diag_8k", "the 8K x 32-head prefill, bf16, with half the "
                                         "channels decaying by e^-3..e^-4 per token, so every "
                                         "16-token diagonal block is evaluated per element")):
        if not extra or name not in extra:
            continue
        x = extra[name]
        pre_x = Prefill(x["q"], x["k"], x["v"], x["la"], x["beta"], None, None)
        us = _time_calls(torch, pre_x.run, steps, warmup)
        io_b = 4 if x["q"].dtype == torch.float32 else 2
        alg = prefill_alg_bytes(x["T"], x["H"], 1, io_b)
        out["prefill_" + name] = {"workload": what, "us": us,
                                  "tokens_per_s": x["T"] / (us * 1e-6), "alg_bytes": alg,
                                  "roofline": _hbm(alg, us)}
        if us_8k:
            out["prefill_" + name]["time_vs_bf16_8k"] = us / us_8k
        del pre_x
    rows = o.shape[0] * o.shape[1]
    e = workloads.make_epilogue(rows, seed=76, io="bf16")
    gate, w = d(e.gate, bf).view(o.shape), d(e.weight)
    y = torch.empty_like(o)
    us = _time_calls(torch, lambda: rmsnorm_gate(o, gate, w, y=y), steps, warmup)
    alg = rows * EPILOGUE_BYTES + D * 4
    out["epilogue"] = {"workload": f"RMSNorm x sigmoid gate over {rows} rows of 128, bf16",
                       "us": us, "alg_bytes": alg, "roofline": _hbm(alg, us)}
    return out


SWEEP_T = (2048, 4096, 8192, 16384, 32768, 65536)
SWEEP_H = 16


def draw_inputs(names):
    """Host inputs of the extra prefill workloads, drawn concurrently before
    any timing (the generators release the interpreter lock while drawing)."""
    from gated_delta_rule_50_amd import workloads
    makers = {
        "long_T131072": lambda: workloads.config(2).prefill(),
        "packed_16_sequences": lambda: workloads.config(3).prefill(),
        "sweep_h16": lambda: workloads.make_prefill([SWEEP_T[-1]], SWEEP_H, seed=1600,
                                                    io="bf16"),
        "fp32_8k": lambda: workloads.make_prefill([8192], 32, seed=1101, io="f32"),
        "exact_diag_8k": lambda: workloads.make_prefill([8192], 32, seed=1201, io="bf16",
                                                        decay="extreme"),
    }
    if not names:
        return {}
    with ThreadPoolExecutor(max_workers=len(names)) as ex:
        futs = {n: ex.submit(makers[n]) for n in names}
        return {n: f.result() for n, f in futs.items()}


def to_device(torch, d, p):
    """Device copies of a host prefill batch (bf16 or fp32 q/k/v)."""
    dt = torch.bfloat16 if p.io == "bf16" else torch.float32
    return {"q": d(p.q, dt), "k": d(p.k, dt), "v": d(p.v, dt), "la": d(p.log_alpha),
            "beta": d(p.beta), "h0": None if p.h0 is None else d(p.h0),
            "cu": d(p.cu_seqlens, torch.int32), "T": p.T, "H": p.H, "N": p.N,
            "lens": np.diff(p.cu_seqlens)}


def long_config(torch, x, name, steps, warmup):
    """Prefill throughput on the long-context or packed variable-length
    workload (parity cases of their own, timed here for their scaling)."""
    from gated_delta_rule_50_amd import Prefill
    pre = Prefill(x["q"], x["k"], x["v"], x["la"], x["beta"], x["h0"], x["cu"])
    us = _time_calls(torch, pre.run, max(4, steps // 2), max(2, warmup // 2))
    T, H, N, lens = x["T"], x["H"], x["N"], x["lens"]
    alg = prefill_alg_bytes(T, H, N, 2, h0=x["h0"] is not None)
    del pre
    torch.cuda.empty_cache()
    return {"workload": f"{N} sequence(s), lengths {int(lens.min())}..{int(lens.max())}, "
                        f"T={T}, H={H}, bf16 q/k/v, h0 ~N(0,0.02)",
            "us": us, "tokens_per_s": T / (us * 1e-6), "alg_bytes": alg,
            "longest_chain_chunks": int((lens.max() + C - 1) // C),
            "roofline": _hbm(alg, us, prefill_traffic(load_traffic(name)))}


def sweep_h16(torch, x, steps, warmup):
    """One sequence of 16 heads at T = 2K .. 64K (prefixes of one seeded
    64K-token batch): the operator shape of the pages' kernel-speed figure;
    and at 2^20 tokens, the longest context at which the pages report the
    whole model's prefill and decode times."""
    from gated_delta_rule_50_amd import Prefill
    rows = []
    for T in SWEEP_T:
        pre = Prefill(x["q"][:T], x["k"][:T], x["v"][:T], x["la"][:T], x["beta"][:T])
        us = _time_calls(torch, pre.run, steps, warmup)
        alg = prefill_alg_bytes(T, SWEEP_H, 1)
        rows.append({"T": T, "us": us, "tokens_per_s": T / (us * 1e-6),
                     "frac_hbm": alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                     "chunks": (T + C - 1) // C})
        del pre
    # the pages' million-token context: the 64K draw repeated 16 times (the
    # timing does not depend on the values; the workspace stays at its cap)
    reps = (1 << 20) // SWEEP_T[-1]
    big = {n: x[n].repeat(reps, *([1] * (x[n].dim() - 1))) for n in ("q", "k", "v", "la", "beta")}
    T = int(big["k"].shape[0])
    pre = Prefill(big["q"], big["k"], big["v"], big["la"], big["beta"])
    us = _time_calls(torch, pre.run, max(3, steps // 4), max(1, warmup // 2))
    alg = prefill_alg_bytes(T, SWEEP_H, 1)
    rows.append({"T": T, "us": us, "tokens_per_s": T / (us * 1e-6),
                 "frac_hbm": alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                 "chunks": (T + C - 1) // C, "workspace_bytes": int(pre.workspace.numel()),
                 "inputs": f"the {SWEEP_T[-1]}-token draw repeated {reps} times"})
    del pre, big
    torch.cuda.empty_cache()
    return {"workload": f"1 sequence, H={SWEEP_H}, d=128, bf16 q/k/v, h0=0",
            "rows": rows,
            "pages_context": "the pages' kernel-speed figure gives about 2 ms at 2K and about "
                             "32 ms at 64K tokens for this shape (batch 1, 16 heads, head "
                             "dimension 128) without naming the hardware or whether the time "
                             "covers more than the forward pass: context, not a target"}


def only_workload(torch, d, name, steps, warmup):
    """Times one workload's prefill calls and nothing else (counter runs);
    for bench_step, the step's prefill call and decode step."""
    from gated_delta_rule_50_amd import Prefill, decode_step, workloads
    if name == "bench_step":
        x = to_device(torch, d, workloads.config(1).prefill())
        cfg4 = workloads.config(4)
        S = d(workloads.make_decode_state(cfg4.n_seqs, cfg4.H, cfg4.seed))
        ds = workloads.make_decode_step(cfg4.n_seqs, cfg4.H, cfg4.seed, 0, io=cfg4.io)
        bf = torch.bfloat16
        dargs = (d(ds.q, bf), d(ds.k, bf), d(ds.v, bf), d(ds.log_alpha), d(ds.beta), S)
    else:
        x = to_device(torch, d, draw_inputs([name])[name])
        dargs = None
    pre = Prefill(x["q"], x["k"], x["v"], x["la"], x["beta"], x["h0"], x["cu"])

    def call():
        pre.run()
        if dargs is not None:
            decode_step(*dargs)
    us = _time_calls(torch, call, steps, warmup)
    print(json.dumps({"only": name, "us_per_call": us, "calls": steps + warmup}))


def main():
    args = _parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.workload, args.calls)
        return
    if args.summarize_mfma:
        durs = dict((k, float(v)) for k, v in (x.split("=", 1) for x in args.durations or []))
        summarize_mfma(args.summarize_mfma, durs)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world}): the "
              "operator's kernels run on one MI355X (heads and sequences shard across GPUs "
              "with no communication; that path is not implemented). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)

    from gated_delta_rule_50_amd import Prefill, decode_step, lib, workloads
    lib()  # fail loudly if the HIP library is missing
    bf = torch.bfloat16

    def d(x, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dt)

    if args.only:
        only_workload(torch, d, args.only, args.steps, args.warmup)
        return

    # every input set is drawn before the first timed call
    t_gen = time.perf_counter()
    names = []
    if not args.no_long_configs:
        names += ["long_T131072", "packed_16_sequences"]
    if not args.no_sweep:
        names.append("sweep_h16")
    if not args.no_extensions:
        names += ["fp32_8k", "exact_diag_8k"]
    if names:
        print(f"drawing inputs: {', '.join(names)}", file=sys.stderr, flush=True)
    host = draw_inputs(names)
    extra = {}
    for n in list(host):
        extra[n] = to_device(torch, d, host.pop(n))
    gen_s = time.perf_counter() - t_gen

    cfg1 = workloads.config(1)
    p = cfg1.prefill()
    pre_args = (d(p.q, bf), d(p.k, bf), d(p.v, bf), d(p.log_alpha), d(p.beta), None,
                d(p.cu_seqlens, torch.int32))
    pre = Prefill(*pre_args)
    cfg4 = workloads.config(4)
    S = d(workloads.make_decode_state(cfg4.n_seqs, cfg4.H, cfg4.seed))
    ds = workloads.make_decode_step(cfg4.n_seqs, cfg4.H, cfg4.seed, 0, io=cfg4.io)
    dq, dk, dv = d(ds.q, bf), d(ds.k, bf), d(ds.v, bf)
    dla, db = d(ds.log_alpha), d(ds.beta)
    do = torch.empty_like(dv)
    pairs = cfg4.n_seqs * cfg4.H

    # KDA_ROCTX=1: named ranges around the two calls of a step, for
    # rocprofv3 --marker-trace (torch's range markers are roctx on ROCm)
    marks = os.environ.get("KDA_ROCTX") == "1"

    def ranged(name, fn):
        if marks:
            torch.cuda.nvtx.range_push(name)
        fn()
        if marks:
            torch.cuda.nvtx.range_pop()

    def step(ev=None):
        # one prefill call + one decode step
        if ev is not None:
            ev[0].record()
        ranged("kda_chunk_fwd", pre.run)
        if ev is not None:
            ev[1].record()
        ranged("kda_decode_step", lambda: decode_step(dq, dk, dv, dla, db, S, o=do))
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [_events(torch, 3) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prefill_ms = [ev[0].elapsed_time(ev[1]) for ev in evs]
    decode_ms = [ev[1].elapsed_time(ev[2]) for ev in evs]

    # Per-kernel characterisation after the timed steps: the prefill's
    # kernels launched one at a time over all chunks (the phase entry
    # point), so each kernel's own duration is measured on the launch stream.
    for _ in range(args.warmup):
        for ph in range(3):
            pre.run_phase(ph)
    torch.cuda.synchronize()
    pevs = [_events(torch, 4) for _ in range(args.steps)]
    for s_ in range(args.steps):
        pevs[s_][0].record()
        for ph in range(3):
            pre.run_phase(ph)
            pevs[s_][1 + ph].record()
    torch.cuda.synchronize()

    names_k = ["chunk_map", "intra", "carry"]
    dur = {n: [ev[i].elapsed_time(ev[i + 1]) for ev in pevs] for i, n in enumerate(names_k)}
    dur["decode"] = decode_ms
    mean = {n: float(np.mean(v)) for n, v in dur.items()}
    t_pre = float(np.mean(prefill_ms)) * 1e-3
    t_dec = mean["decode"] * 1e-3

    th = p.T * p.H
    nh = p.N * p.H
    kernels = {
        "chunk_map": {"mean_us": mean["chunk_map"] * 1e3},
        "intra": {"mean_us": mean["intra"] * 1e3, "bound": "hbm",
                  "alg_bytes": th * PREFILL_IN_BYTES,
                  "unit_note": "q,k,v,log_alpha,beta per token-head (1284 B)"},
        "carry": {"mean_us": mean["carry"] * 1e3, "bound": "hbm",
                  "alg_bytes": th * PREFILL_OUT_BYTES + nh * STATE_BYTES,
                  "unit_note": "o per token-head (256 B) + h_final per sequence-head"},
        "decode": {"mean_us": mean["decode"] * 1e3, "bound": "hbm",
                   "alg_bytes": pairs * DECODE_BYTES,
                   "unit_note": "132612 B per (sequence, head)"},
    }
    for n, kdesc in kernels.items():
        if "alg_bytes" in kdesc:
            gbps = kdesc["alg_bytes"] / (kdesc["mean_us"] * 1e-6) / 1e9
            kdesc["achieved_GBps"] = gbps
            kdesc["frac"] = gbps / HBM_PEAK_GBPS
    traffic = load_traffic("bench_step")
    for n, b in traffic.items():
        if n in kernels:
            kernels[n]["traffic_bytes"] = b
            if "alg_bytes" in kernels[n]:
                kernels[n]["traffic_ratio"] = b / kernels[n]["alg_bytes"]

    # headline roofline: the prefill call (value is its tokens/s)
    pre_bytes = th * PREFILL_BYTES + nh * STATE_BYTES
    roofline = _hbm(pre_bytes, t_pre * 1e6, prefill_traffic(traffic))
    roofline["kernel"] = "kda_chunk_fwd call (intra_kernel + carry_kernel)"
    roofline["unit_bytes"] = ("1540 B per token-head (q, k, v, o bf16; log_alpha, beta fp32) + "
                              "65536 B per (sequence, head) h_final")
    decode_roofline = _hbm(pairs * DECODE_BYTES, mean["decode"] * 1e3, traffic.get("decode"))
    decode_roofline["kernel"] = "recurrent_fwd_kernel (decode step)"
    decode_roofline["unit_bytes"] = "132612 B per (sequence, head)"

    t_roof = max(pre_bytes / (HBM_PEAK_GBPS * 1e9), th * FLOPS_EQ13 / (BF16_PEAK_TFLOPS * 1e12))
    prefill_path = {
        "time_us": t_pre * 1e6,
        "alg_bytes": pre_bytes,
        "achieved_GBps": pre_bytes / t_pre / 1e9,
        "frac_hbm": pre_bytes / t_pre / 1e9 / HBM_PEAK_GBPS,
        "tflops_eq13": th * FLOPS_EQ13 / t_pre / 1e12,
        "frac_mfma_eq13": th * FLOPS_EQ13 / t_pre / 1e12 / BF16_PEAK_TFLOPS,
        "tflops_dense": th * FLOPS_DENSE / t_pre / 1e12,
        "frac_mfma_dense": th * FLOPS_DENSE / t_pre / 1e12 / BF16_PEAK_TFLOPS,
        "attainable_frac": t_roof / t_pre,
    }
    decode_tps = cfg4.n_seqs / t_dec
    # distribution of the timed calls (the means above give value and
    # roofline), and the prefill with cold inputs
    timing = {"prefill_warm": _spread(prefill_ms), "decode": _spread(decode_ms),
              "prefill_cold": cold_prefill(torch, pre, max(5, args.steps // 2))}

    out = {
        "metric": METRIC,
        "value": p.T / t_pre,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill T={p.T} H={p.H} d=128 chunk=64 bf16 q/k/v, fp32 "
                               f"gates/state, h0=0; + decode step {cfg4.n_seqs}x{cfg4.H} "
                               f"fp32 states", "T": p.T, "H": p.H, "d": D, "chunk": C,
                   "decode_batch": cfg4.n_seqs},
        "decode_tokens_per_s": decode_tps,
        "prefill_phases_us": sum(mean[n] for n in names_k) * 1e3,
        "roofline": roofline,
        "decode_roofline": decode_roofline,
        "prefill_path": prefill_path,
        "timing": timing,
        "kernels": kernels,
        "input_draw_s": gen_s,
    }
    print("8K prefill and decode timed", file=sys.stderr, flush=True)
    if not args.no_long_configs:
        out["long_configs"] = {n: long_config(torch, extra.pop(n), n, args.steps, args.warmup)
                               for n in ("long_T131072", "packed_16_sequences")}
        print("long configs timed", file=sys.stderr, flush=True)
    if not args.no_sweep:
        out["sweep_h16"] = sweep_h16(torch, extra.pop("sweep_h16"), args.steps, args.warmup)
        print("16-head sweep timed", file=sys.stderr, flush=True)
    if not args.no_extensions:
        out["extensions"] = extensions(torch, d, pre_args, args.steps, args.warmup, extra,
                                       t_pre * 1e6)
        print("extensions timed", file=sys.stderr, flush=True)
    extra.clear()
    if not args.no_probes:
        pr = probes(torch)
        out["probes"] = pr
        _with_probe(roofline, pr, "hbm_copy_GBps")
        _with_probe(decode_roofline, pr, "hbm_rmw_GBps")
        kinds = {"recurrent_L4": "hbm_rmw_GBps", "recurrent_L64": "valu_fp32_TFLOPs",
                 "chunked_L64": "hbm_copy_GBps",
                 "decode_bf16_state": "hbm_rmw_GBps", "decode_batch1": "hbm_rmw_GBps",
                 "epilogue": "hbm_copy_GBps"}
        for name, key in kinds.items():
            if name in out.get("extensions", {}):
                _with_probe(out["extensions"][name]["roofline"], pr, key)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
