"""Helpers shared by the GPU tests: run the library on a workload and compare
with the float64 oracle under the stated error bars."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import exact_io_aware_56_amd as fa
import oracle

# Error bars per input dtype: max |dO|, mean |dO|, max |dLSE| (absolute, or
# relative to max(1, |LSE|) when lse_rel is set).
TOL = {
    "bf16": dict(max_o=2e-2, mean_o=2e-3, lse=1e-2, lse_rel=False),
    "fp16": dict(max_o=2e-2, mean_o=2e-3, lse=1e-2, lse_rel=False),
    "fp32": dict(max_o=1e-5, mean_o=1e-6, lse=1e-5, lse_rel=True),
    "fp8": dict(max_o=8e-2, mean_o=8e-3, lse=1e-2, lse_rel=False),
}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(w):
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    kl = None if w.key_len is None else torch.from_numpy(w.key_len).to(dev)
    return q, k, v, kl


def run(w, stream=None):
    """Run the library on workload w; returns (O, LSE) as float64 numpy arrays."""
    q, k, v, kl = to_device(w)
    o, lse = fa.fwd(q, k, v, scale=w.spec.scale, causal=w.spec.causal, key_len=kl,
                    descale=w.descale, stream=stream)
    torch.cuda.synchronize()
    return o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


def errors(o, lse, o_ref, lse_ref, lse_rel):
    d = np.abs(o - o_ref)
    fin = np.isfinite(lse_ref)
    same_inf = np.array_equal(np.isfinite(lse), fin) and np.all(lse[~fin] == lse_ref[~fin])
    if fin.any():
        dl = np.abs(lse[fin] - lse_ref[fin])
        if lse_rel:
            dl = dl / np.maximum(1.0, np.abs(lse_ref[fin]))
        dl = float(dl.max())
    else:
        dl = 0.0
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0, dl, same_inf


def assert_close(o, lse, o_ref, lse_ref, dtype, label=""):
    t = TOL[dtype]
    mx, mean, dl, same_inf = errors(o, lse, o_ref, lse_ref, t["lse_rel"])
    say(f"  {label} max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dLSE|={dl:.3e}")
    assert np.all(np.isfinite(o)), f"{label}: non-finite O"
    assert same_inf, f"{label}: LSE -inf pattern differs"
    assert mx <= t["max_o"], f"{label}: max|dO| {mx} > {t['max_o']}"
    assert mean <= t["mean_o"], f"{label}: mean|dO| {mean} > {t['mean_o']}"
    assert dl <= t["lse"], f"{label}: max|dLSE| {dl} > {t['lse']}"


def full_oracle(w):
    q, k, v = w.exact()
    return oracle.attention_forward(q, k, v, w.spec.scale, w.spec.causal, w.key_len_or_none())


def sampled_rows(spec, rng, per_head=48, extra=None):
    """Query rows to check per (b, h): the edges, tile boundaries and random rows."""
    N = spec.N
    fixed = {0, 1, 2, 31, 32, 63, 64, 127, 128, N // 2, N - 129, N - 65, N - 2, N - 1}
    fixed = {r for r in fixed if 0 <= r < N}
    if extra is not None:
        fixed |= {int(r) for r in extra if 0 <= r < N}
    rnd = rng.choice(N, size=min(N, per_head), replace=False)
    return np.array(sorted(fixed | set(int(r) for r in rnd)), dtype=np.int64)
