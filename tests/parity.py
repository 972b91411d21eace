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


def run(w, stream=None, p8=False):
    """Run the library on workload w (p8: fp8 inputs through fa_fwd_fp8_p8);
    returns (O, LSE) as float64 numpy arrays."""
    q, k, v, kl = to_device(w)
    o, lse = fa.fwd(q, k, v, scale=w.spec.scale, causal=w.spec.causal, key_len=kl,
                    descale=w.descale, stream=stream, p8=p8)
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


def worker_count() -> int:
    """Host threads for oracle work: this process's CPU share, at most 16."""
    import os
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(16, n))


def every_element_errors(w, o, lse, say_every=8):
    """max|dO|, mean|dO| over all B*H*N*d elements and max|dLSE| of the
    library's (o, lse) against the float64 oracle, computed head by head
    (a pool of threads, each head's oracle with one BLAS thread) so that
    memory stays bounded at the full workload sizes."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    s = w.spec
    q, k, v = w.exact()
    kl = w.key_len_or_none()
    pairs = [(b, h) for b in range(s.B) for h in range(s.H)]

    def one(bh):
        b, h = bh
        g = h // (s.H // s.kv_heads)
        o_ref, lse_ref = oracle.attention_forward(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1],
                                                  v[b:b + 1, g:g + 1], s.scale, s.causal,
                                                  None if kl is None else kl[b:b + 1])
        d = np.abs(o[b, h] - o_ref[0, 0])
        fin = np.isfinite(lse_ref[0, 0])
        same_inf = bool(np.array_equal(np.isfinite(lse[b, h]), fin)
                        and np.all(lse[b, h][~fin] == lse_ref[0, 0][~fin]))
        dl = float(np.abs(lse[b, h][fin] - lse_ref[0, 0][fin]).max()) if fin.any() else 0.0
        return float(d.max()), float(d.sum()), d.size, dl, same_inf

    mx, total, count, dl, same = 0.0, 0.0, 0, 0.0, True
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=worker_count()) as ex:
        for i, r in enumerate(ex.map(one, pairs)):
            mx, total, count = max(mx, r[0]), total + r[1], count + r[2]
            dl, same = max(dl, r[3]), same and r[4]
            if (i + 1) % say_every == 0 or i + 1 == len(pairs):
                say(f"  oracle heads {i + 1}/{len(pairs)}: max|dO|={mx:.3e} "
                    f"mean|dO|={total / count:.3e} max|dLSE|={dl:.3e}")
    return mx, total / max(1, count), dl, same
