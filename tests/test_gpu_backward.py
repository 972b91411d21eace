"""GPU parity of fa_bwd (dQ, dK, dV) with the float64 backward oracle.

The kernels recompute P from the forward's LSE and take Delta = rowsum(dO*O)
from the forward's 16-bit O, so they differ from the oracle by the forward's
own rounding as well as their own (16-bit P and dS operands, 16-bit outputs).
Errors are measured relative to the size of each gradient: max|d| over
max(1, max|ref|) and mean|d| over max(1e-3, mean|ref|)."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_56_amd as fa
import oracle
import workloads as W
from parity import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
TOL_MAX = 2.5e-2   # max |d| / max(1, max |ref|)
TOL_MEAN = 1e-2    # mean |d| / max(1e-3, mean |ref|)


def check(name, got, ref, label):
    got = got.double().cpu().numpy()
    d = np.abs(got - ref)
    rel_max = float(d.max()) / max(1.0, float(np.abs(ref).max())) if d.size else 0.0
    rel_mean = float(d.mean()) / max(1e-3, float(np.abs(ref).mean())) if d.size else 0.0
    say(f"  {label} {name}: max|d|={d.max():.3e} (rel {rel_max:.3e}) mean|d|={d.mean():.3e} "
        f"(rel {rel_mean:.3e}) max|ref|={np.abs(ref).max():.3e}")
    assert np.all(np.isfinite(got)), f"{label} {name}: non-finite"
    assert rel_max <= TOL_MAX, f"{label} {name}: max rel {rel_max}"
    assert rel_mean <= TOL_MEAN, f"{label} {name}: mean rel {rel_mean}"


def run_case(dtype, B, H, H_kv, N, d, causal, key_len, seed):
    spec = W.SPECS["decoder_causal_bf16"].with_shape(
        B=B, H=H, H_kv=H_kv, N=N, d=d, dtype=dtype, causal=causal, scale=1.0 / math.sqrt(d),
        key_len_range=None, seed=seed)
    w = W.draw(spec)
    rng = np.random.default_rng(seed + 1)
    do32 = rng.standard_normal((B, H, N, d)).astype(np.float32)
    do = torch.from_numpy(do32).to(W.TORCH_STORAGE[dtype])
    q, k, v, dod = (t.to(DEV) for t in (w.q, w.k, w.v, do))
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32, device=DEV)
    o, lse = fa.fwd(q, k, v, scale=spec.scale, causal=causal, key_len=kl)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dod, scale=spec.scale, causal=causal, key_len=kl)
    torch.cuda.synchronize()
    qe, ke, ve = w.exact()
    ref = oracle.attention_backward(qe, ke, ve, do.double().numpy(), spec.scale, causal,
                                    None if key_len is None else np.asarray(key_len))
    label = f"{dtype} B{B} H{H}/{H_kv} N{N} d{d} causal={causal} kl={key_len}"
    for name, g, r in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
        check(name, g, r, label)


SMALL_N = [1, 31, 33, 100, 257]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small_sweep(dtype, d, causal):
    for i, N in enumerate(SMALL_N):
        for padded in (False, True):
            key_len = [N, max(0, N // 2 - 1)] if padded else None
            seed = 15000 + 31 * i + 7 * padded + d + causal
            say(f"case bwd dtype={dtype} d={d} causal={causal} N={N} padded={padded} seed={seed}")
            run_case(dtype, 2, 2, 2, N, d, causal, key_len, seed)


@pytest.mark.parametrize("H,H_kv,N,causal", [(4, 2, 200, True), (6, 1, 130, False),
                                             (4, 4, 1024, True), (8, 2, 777, False)])
def test_backward_grouped_and_longer(H, H_kv, N, causal):
    seed = 16000 + H * 10 + H_kv + N
    say(f"case bwd grouped H={H} H_kv={H_kv} N={N} causal={causal} seed={seed}")
    run_case("bf16", 1, H, H_kv, N, 128, causal, [N - 5] if N > 300 else None, seed)


def test_backward_rejects_bad_dtype_and_workspace():
    w = W.draw(W.SPECS["single_head_fp32"].with_shape(N=64, d=64))
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o, lse = fa.fwd(q, k, v, scale=0.125)
    ws = torch.empty(1 << 16, dtype=torch.float32, device=DEV)
    g = [torch.empty_like(q) for _ in range(3)]
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, q, lse, *g, ws, 0.125)
    qb, kb, vb = (t.to(torch.bfloat16) for t in (q, k, v))
    ob, lseb = fa.fwd(qb, kb, vb, scale=0.125)
    gb = [torch.full_like(qb, 3.0) for _ in range(3)]
    small = torch.empty(4, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError):
        fa.fa_bwd(qb, kb, vb, ob, qb, lseb, *gb, small, 0.125)
    torch.cuda.synchronize()
    assert all(torch.all(x == 3.0) for x in gb)


def test_backward_full_benched_shape():
    """The shape the benchmark times (B1 H32 N8192 d128 causal bf16, the long
    workload's inputs with its outlier keys): every element of dQ, dK and dV
    against the float64 backward oracle, head by head."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from parity import worker_count

    w = W.draw(W.SPECS["long_causal_bf16"])
    s = w.spec
    say(f"case bwd full shape B{s.B} H{s.H} N{s.N} d{s.d} causal={s.causal} seed={s.seed}")
    rng = np.random.default_rng(s.seed + 1)
    do32 = rng.standard_normal((s.B, s.H, s.N, s.d)).astype(np.float32)
    do = torch.from_numpy(do32).to(torch.bfloat16)
    q, k, v, dod = (t.to(DEV) for t in (w.q, w.k, w.v, do))
    o, lse = fa.fwd(q, k, v, scale=s.scale, causal=s.causal)
    grads = fa.bwd(q, k, v, o, lse, dod, scale=s.scale, causal=s.causal)
    torch.cuda.synchronize()
    got = [g.double().cpu().numpy() for g in grads]
    del grads
    qe, ke, ve = w.exact()
    dod64 = do.double().numpy()

    def one(h):
        ref = oracle.attention_backward(qe[:, h:h + 1], ke[:, h:h + 1], ve[:, h:h + 1],
                                        dod64[:, h:h + 1], s.scale, s.causal)
        out = []
        for g, r in zip(got, ref):
            d = np.abs(g[:, h:h + 1] - r)
            out.append((float(d.max()), float(d.sum()), float(np.abs(r).max()),
                        float(np.abs(r).sum()), d.size))
        return out

    acc = [[0.0, 0.0, 0.0, 0.0, 0] for _ in range(3)]
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=min(8, worker_count())) as ex:
        for i, res in enumerate(ex.map(one, range(s.H))):
            for a, r in zip(acc, res):
                a[0], a[1], a[2], a[3], a[4] = (max(a[0], r[0]), a[1] + r[1], max(a[2], r[2]),
                                                a[3] + r[3], a[4] + r[4])
            if (i + 1) % 8 == 0:
                say(f"  oracle heads {i + 1}/{s.H}")
    for name, (mx, sd, mr, sr, n) in zip(("dQ", "dK", "dV"), acc):
        rel_max = mx / max(1.0, mr)
        rel_mean = (sd / n) / max(1e-3, sr / n)
        say(f"  full shape {name}: max|d|={mx:.3e} (rel {rel_max:.3e}) mean|d|={sd / n:.3e} "
            f"(rel {rel_mean:.3e}) max|ref|={mr:.3e}")
        assert np.isfinite(mx), f"{name}: non-finite"
        assert rel_max <= TOL_MAX, f"{name}: max rel {rel_max}"
        assert rel_mean <= TOL_MEAN, f"{name}: mean rel {rel_mean}"
