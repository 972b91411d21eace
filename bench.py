#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

One step = one fa_fwd call over the whole workload (every head, every query
tile: the full hot path). The default workload is the long-context causal
decoder attention the headline metric is quoted on: bf16, B=1, H=32,
N=8192, d=128, causal, 1% of the key rows scaled x8, scale 1/sqrt(128).

Back-to-back launches of this kernel after an idle period run through the
chip's power-management transient for a few dozen launches (per-launch times
swing by up to 30% before they settle). Before the W warm-up steps the step is
therefore launched back to back for --settle-ms of GPU time (200 ms by
default, counted from the first launch's duration; reported as
config.settle_launches), so that the timed steps measure the sustained state
whatever W is.

The K timed launches run back to back between two events on the launch
stream; the p10 / median / p90 of single launches come from a further sample
of launches right after them, each between its own pair of events.

Prints ONE JSON line. `value` is attention TFLOP/s (4*B*H*N^2*d, halved for
causal) over the timed steps with inputs already in HBM; `roofline` prices the
kernel's per-launch average (HIP events on the launch stream) against the
dense bf16 MFMA peak; `cpu_baseline` times the float64 oracle on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MFMA peak, bf16 causal B1 H32 N8192 d128"
# Published dense MI355X peaks (TFLOP/s) per input dtype of the contraction.
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2, "fp32": 157.3}
EXP_PEAK_T = 256 * 4 * 8 * 2.4e9 / 1e12
SPREAD_SAMPLE = 50  # steps timed one by one after the timed region
SETTLE_CHUNK = 10  # steps per chunk of the settle phase
KERNEL_SOURCES = ["exact_io_aware_56_amd/csrc/fa_fwd.hip", "exact_io_aware_56_amd/csrc/fa_api.cpp",
                  "exact_io_aware_56_amd/csrc/fa_internal.h"]


def kernel_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def sq_counters(workload: str):
    """MFMA busy fraction, VALU and LDS instructions per MFMA and the LDS bank
    conflict rate of the kernel from the committed SQ counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_{workload}_sq_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]+)", text)
    if not sha or sha.group(1) != kernel_sha():
        return None
    out = {}
    for key in ("mfma_busy_frac", "valu_per_mfma", "lds_per_mfma", "lds_bank_conflict_rate",
                "valu_mfma_coexec_frac"):
        m = re.search(key + r":\s*([0-9.eE+-]+)", text)
        if m:
            out[key] = float(m.group(1))
    out["source"] = os.path.relpath(path, ROOT)
    return out


def host_cores() -> int:
    """CPUs this process may run on."""
    return len(os.sched_getaffinity(0))


def blas_threads() -> int:
    """Threads for the oracle's BLAS: this process's CPUs, capped by
    OMP_NUM_THREADS when the environment sets it."""
    n = host_cores()
    env = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(env)) if env.isdigit() and int(env) > 0 else n


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != kernel_sha():
        return None
    return float(val.group(1))


def decode_bytes(spec, key_len) -> int:
    """Decode: each batch entry's valid K/V rows read once, Q read once, O and
    LSE written once."""
    e = {"fp16": 2, "bf16": 2}[spec.dtype]
    kl = spec.N * spec.B if key_len is None else int(key_len.sum())
    qo = 2 * e * spec.B * spec.H * spec.Nq * spec.d
    return 2 * e * spec.kv_heads * spec.d * kl + qo + 4 * spec.B * spec.H * spec.Nq


def algorithmic_bytes(spec, rows=None) -> int:
    """Q, K, V read once, O written once, LSE written once (K and V have
    H_kv heads when the workload groups them). `rows`: query rows per head
    (the packed rows of a packed batch; B*N otherwise)."""
    e_in = {"fp32": 4, "fp16": 2, "bf16": 2, "fp8": 1}[spec.dtype]
    e_out = {"fp32": 4, "fp16": 2, "bf16": 2, "fp8": 2}[spec.dtype]
    rows = spec.B * spec.N if rows is None else rows
    return ((e_in + e_out) * spec.H + 2 * e_in * spec.kv_heads) * rows * spec.d + 4 * spec.H * rows


def cpu_baseline_backward(w, budget_s: float):
    """The float64 backward oracle on whole heads until the budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    threads = blas_threads()
    with threadpool_limits(limits=threads):
        return _cpu_baseline_backward(w, budget_s, threads, np, oracle)


def _cpu_baseline_backward(w, budget_s, threads, np, oracle):
    s = w.spec
    q, k, v = w.exact()
    rng = np.random.default_rng(s.seed + 1)
    heads = 0
    t0 = time.perf_counter()
    for b in range(s.B):
        for h in range(s.H):
            g = h // (s.H // s.kv_heads)
            do = rng.standard_normal((1, 1, s.N, s.d))
            oracle.attention_backward(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1],
                                      v[b:b + 1, g:g + 1], do, s.scale, s.causal,
                                      None if w.key_len is None else w.key_len[b:b + 1])
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 2.5 * s.flops() / (s.B * s.H) * heads
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": host_cores(),
            "threads": threads, "kind": "oracle",
            "sample": f"{heads} of {s.B * s.H} heads of the same workload's backward, every "
                      f"query row, float64, {dt:.2f} s wall"}


def cpu_baseline(w, budget_s: float):
    """Time the float64 oracle on whole heads of the workload until the budget
    is spent (at least one head), its BLAS on blas_threads() threads; returns
    the JSON object."""
    from threadpoolctl import threadpool_limits

    threads = blas_threads()
    with threadpool_limits(limits=threads):
        return _cpu_baseline(w, budget_s, threads)


def _cpu_baseline(w, budget_s: float, threads: int):
    import oracle

    s = w.spec
    q, k, v = w.exact()
    kl = w.key_len_or_none()
    if s.packed:
        done, flops = 0, 0.0
        t0 = time.perf_counter()
        for b, n in enumerate(w.lengths):
            for h in range(s.H):
                oracle.attention_varlen_rows(q, k, v, w.cu_seqlens, s.scale, s.causal, b, h,
                                             range(int(n)))
                done += 1
                flops += s.flops([n]) / s.H
                if time.perf_counter() - t0 >= budget_s:
                    break
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": host_cores(),
                "threads": threads, "kind": "oracle",
                "sample": f"{done} of {s.B * s.H} (sequence, head) pairs of the same packed "
                          f"batch, every row, float64, {dt:.2f} s wall"}
    if s.is_decode:
        done = 0
        t0 = time.perf_counter()
        for b in range(s.B):
            oracle.attention_decode(q[b:b + 1], k[b:b + 1], v[b:b + 1], s.scale, s.causal,
                                    None if kl is None else kl[b:b + 1])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": round(s.flops() / s.B * done / dt / 1e12, 6), "unit": "TFLOP/s",
                "cores": host_cores(), "threads": threads, "kind": "oracle",
                "sample": f"{done} of {s.B} sequences of the same workload, every head, "
                          f"float64, {dt:.2f} s wall"}
    heads = 0
    t0 = time.perf_counter()
    for b in range(s.B):
        for h in range(s.H):
            kb = None if kl is None else kl[b:b + 1]
            g = h // (s.H // s.kv_heads)
            oracle.attention_forward(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1],
                                     v[b:b + 1, g:g + 1], s.scale, s.causal, kb,
                                     window=(s.window_left, -1) if s.window_left >= 0 else None)
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = s.flops() / (s.B * s.H) * heads
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": host_cores(),
            "threads": threads, "kind": "oracle",
            "sample": f"{heads} of {s.B * s.H} heads of the same workload, every query row, "
                      f"float64, {dt:.2f} s wall"}


def workload_dtype(name: str) -> str:
    import workloads as W
    return W.SPECS[name].dtype if name in W.SPECS else ""


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="long_causal_bf16")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dQ, dK, dV) of the workload instead of the "
                         "forward; FLOP counted as 2.5x the forward's (five N^2 d products)")
    ap.add_argument("--p8", action="store_true",
                    help="fp8 workloads: time fa_fwd_fp8_p8 (P rounded to e4m3 for the P V "
                         "product, both products on the fp8 matrix cores)")
    ap.add_argument("--N", type=int, default=0,
                    help="override the workload's sequence length (HBM scaling runs); "
                         "such a line is not the headline measurement")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="GPU time of back-to-back steps run before the warm-up steps so that "
                         "the chip's clocks settle (0 disables)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the cpu_baseline leg (0 disables)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times) and exit; "
                         "its HBM counters calibrate FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args(argv)

    if args.p8 and workload_dtype(args.workload) != "fp8":
        print(json.dumps({"error": "--p8 applies to fp8 workloads"}))
        return 2
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; "
                                   "multi-GPU runs are not supported (use --gpus 1)"}))
        return 2

    import torch

    import exact_io_aware_56_amd as fa
    import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 3
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return 0
    spec = W.SPECS[args.workload]
    default_n = args.N in (0, spec.N)
    if not default_n:
        spec = spec.with_shape(N=args.N)
    w = W.draw(spec)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    kl = None if w.key_len is None else torch.from_numpy(w.key_len).to(dev)
    o = torch.empty(q.shape, dtype=fa.out_dtype(q.dtype), device=dev)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    cu = None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens).to(dev)
    stream = torch.cuda.current_stream()
    ws = None
    if spec.is_decode:
        nbytes = fa.decode_workspace_bytes(spec.B, spec.H, spec.kv_heads, spec.Nq, spec.N, spec.d)
        ws = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device=dev)

    if args.backward:
        if spec.is_decode or spec.packed or spec.dtype not in ("bf16", "fp16"):
            print(json.dumps({"error": "the backward covers 16-bit forward workloads"}))
            return 2
        o_f, lse_f = fa.fwd(q, k, v, scale=spec.scale, causal=spec.causal, key_len=kl)
        g = torch.Generator(device="cpu").manual_seed(spec.seed + 1)
        dout = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
        grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        ws = torch.empty((fa.bwd_workspace_bytes(spec.B, spec.H, spec.N) + 15) // 16 * 4,
                         dtype=torch.float32, device=dev)
        o = grads[0]

    def step():
        if args.backward:
            fa.fa_bwd(q, k, v, o_f, dout, lse_f, *grads, ws, spec.scale, spec.causal, kl,
                      stream=stream)
        elif spec.packed:
            fa.fa_fwd_varlen(q, k, v, o, lse, cu, spec.N, spec.scale, spec.causal, stream=stream)
        elif spec.window_left >= 0:
            fa.fa_fwd_window(q, k, v, o, lse, spec.scale, spec.causal, (spec.window_left, -1), kl,
                             *w.descale, stream=stream)
        elif spec.is_decode:
            fa.fa_fwd_decode(q, k, v, o, lse, ws, spec.scale, spec.causal, kl, stream=stream)
        elif spec.kv_heads != spec.H:
            fa.fa_fwd_gqa(q, k, v, o, lse, spec.scale, spec.causal, kl, *w.descale, stream=stream)
        elif spec.dtype == "fp8" and args.p8:
            fa.fa_fwd_fp8_p8(q, k, v, o, lse, spec.scale, spec.causal, kl, *w.descale,
                             stream=stream)
        elif spec.dtype == "fp8":
            fa.fa_fwd_fp8(q, k, v, o, lse, spec.scale, spec.causal, kl, *w.descale, stream=stream)
        else:
            fa.fa_fwd(q, k, v, o, lse, spec.scale, spec.causal, kl, stream=stream)

    def finite() -> bool:
        return bool(torch.isfinite(o.float()).all())

    # The first launch is checked. Then the step runs back to back for at
    # least --settle-ms of GPU time, in chunks whose events are read while the
    # next chunk is already queued (so the GPU never idles), until the chip's
    # clocks have left their power-management transient; then the W warm-up
    # steps and the timed steps follow with only one synchronisation in
    # between: any longer idle spell restarts the transient.
    settle = 0
    if args.warmup > 0 or args.settle_ms > 0:
        step()
        torch.cuda.synchronize()
        if not finite():
            print(json.dumps({"error": "non-finite output"}))
            return 4
    if args.settle_ms > 0:
        done_ms, prev = 0.0, None
        while True:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(SETTLE_CHUNK):
                step()
            b.record(stream)
            settle += SETTLE_CHUNK
            if prev is not None:
                prev[1].synchronize()
                done_ms += prev[0].elapsed_time(prev[1])
                if done_ms >= args.settle_ms or settle >= 20000:
                    break
            prev = (a, b)

    # The timed region is the K steps between two events on the launch stream,
    # with nothing else enqueued between the launches. The spread of single
    # launches comes from a separate sample of steps right after it, each
    # bracketed by its own pair of events (those events add a few microseconds
    # of idle time per launch, so they stay out of the timed region).
    outer0, outer1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_spread = min(SPREAD_SAMPLE, args.steps)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread)]
    for _ in range(args.warmup - (1 if settle == 0 else 0)):
        step()
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    outer0.record(stream)
    for _ in range(args.steps):
        step()
    outer1.record(stream)
    for i in range(n_spread):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    if args.warmup == 0 and not finite():
        print(json.dumps({"error": "non-finite output"}))
        return 4
    total_ms = outer0.elapsed_time(outer1)
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends)) or [total_ms / args.steps]
    ms_per_step = total_ms / args.steps
    avg_launch_ms = ms_per_step  # one step is one launch (decode and backward: their kernels)

    flop = w.flops() * (2.5 if args.backward else 1.0)
    value = flop / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[spec.dtype]
    achieved = flop / (avg_launch_ms * 1e-3) / 1e12
    prof_name = spec.name + ("_p8" if args.p8 else "")
    traffic = measured_traffic(prof_name) if default_n and not args.backward else None
    exps = w.exps()
    if spec.is_decode:
        # HBM-bound: the roofline is bytes moved, the two kernels of a step
        # (split pass and merge) timed together
        alg = decode_bytes(spec, w.key_len)
        gbs = alg / (avg_launch_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                    "frac": round(gbs / 8000.0, 4), "traffic": traffic, "algorithmic_bytes": alg,
                    "kernel_sources_sha256_16": kernel_sha()}
    else:
        roofline = None
    result = {
        "metric": METRIC if spec.name == "long_causal_bf16" and default_n and not args.backward
        else f"attention {'bwd' if args.backward else 'fwd'} TFLOP/s ({spec.name}, N={spec.N})",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape and structure)",
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "config": {
            "workload": spec.name, "B": spec.B, "H": spec.H, "N": spec.N, "d": spec.d,
            "causal": spec.causal, "scale": spec.scale,
            "H_kv": spec.kv_heads, "Nq": spec.q_len, "window_left": spec.window_left,
            "key_len": None if w.key_len is None else "per-batch padding",
            "packed": None if cu is None else {
                "sequences": spec.B, "rows": int(w.q.shape[1]),
                "lengths": "U{%d..%d}" % spec.key_len_range, "max_seqlen": spec.N},
            "outlier_keys_frac": spec.outlier_frac, "seed": spec.seed,
            "p_e4m3": bool(args.p8) if spec.dtype == "fp8" else None,
            "settle_launches": settle,
            "spread_sample_steps": len(per),
            "launch_ms_p10": round(per[len(per) // 10], 5),
            "launch_ms_median": round(per[len(per) // 2], 5),
            "launch_ms_p90": round(per[(9 * len(per)) // 10], 5),
            "host_wall_s_incl_spread": round(wall, 4),
        },
        "roofline": roofline or {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "algorithmic_bytes": algorithmic_bytes(spec, None if cu is None else w.q.shape[1]),
            "kernel_sources_sha256_16": kernel_sha(),
            # Secondary bound: one exp2 per unmasked score on the transcendental
            # unit (256 CUs x 4 SIMDs x 8 lanes per cycle x 2.4 GHz).
            "exp": {"achieved": round(exps / (avg_launch_ms * 1e-3) / 1e12, 4),
                    "peak": EXP_PEAK_T, "unit": "Texp/s",
                    "frac": round(exps / (avg_launch_ms * 1e-3) / 1e12 / EXP_PEAK_T, 4)},
        },
    }
    counters = sq_counters(prof_name) if default_n and not args.backward else None
    if counters is not None:
        result["counters"] = counters
    if w.key_len is not None and (not spec.causal or spec.is_decode):
        eff = spec.flops() * float(w.key_len.sum()) / (spec.B * spec.N)
        result["config"]["effective_tflops"] = round(eff / (ms_per_step * 1e-3) / 1e12, 3)
    if args.backward:
        result["config"]["pass"] = "backward"
        result["roofline"]["exp"] = None
    if args.cpu_budget > 0:
        result["cpu_baseline"] = (cpu_baseline_backward if args.backward else cpu_baseline)(
            w, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
