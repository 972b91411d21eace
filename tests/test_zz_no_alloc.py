"""fa_fwd_decode_noalloc (partial results in the library's own device scratch)
against fa_fwd_decode (caller's workspace) through the C ABI: two calls in a
row, the second on a smaller input, each compared with the workspace entry
point on the same inputs (bit for bit: the same kernels run on both) and with
the float64 decode oracle under the bf16 / fp16 error bars."""
import numpy as np
import pytest
import torch

import exact_io_aware_56_amd as fa
import oracle
import workloads as W
from exact_io_aware_56_amd import _lib
from parity import TOL, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def case(spec_name, **shape):
    spec = W.SPECS[spec_name].with_shape(**shape) if shape else W.SPECS[spec_name]
    return W.draw(spec)


def run_both(w):
    s = w.spec
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    kl = None if w.key_len is None else torch.from_numpy(w.key_len).to(DEV)
    B, H, Nq, d = q.shape
    o_ws = torch.full_like(q, float("nan"))
    lse_ws = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    o_na = torch.full_like(q, float("nan"))
    lse_na = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    nbytes = fa.decode_workspace_bytes(B, H, k.shape[1], Nq, k.shape[2], d)
    ws = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device=DEV)
    fa.fa_fwd_decode(q, k, v, o_ws, lse_ws, ws, s.scale, s.causal, kl)
    fa.fa_fwd_decode_noalloc(q, k, v, o_na, lse_na, s.scale, s.causal, kl)
    torch.cuda.synchronize()
    return (o_ws, lse_ws), (o_na, lse_na), nbytes


def check(w, label):
    s = w.spec
    (o_ws, lse_ws), (o_na, lse_na), nbytes = run_both(w)
    say(f"  {label}: B{s.B} H{s.H}/{s.kv_heads} Nq{s.q_len} Nk{s.N} d{s.d} causal={s.causal} "
        f"partial results {nbytes} bytes")
    assert nbytes <= 8 << 20
    assert torch.equal(o_na, o_ws), f"{label}: O differs from the workspace entry point"
    assert torch.equal(lse_na, lse_ws), f"{label}: LSE differs from the workspace entry point"
    qe, ke, ve = w.exact()
    o_ref, lse_ref = oracle.attention_decode(qe, ke, ve, s.scale, s.causal, w.key_len_or_none())
    o = o_na.double().cpu().numpy()
    lse = lse_na.double().cpu().numpy()
    t = TOL[s.dtype]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    dmax, dmean = float(np.abs(o - o_ref).max()), float(np.abs(o - o_ref).mean())
    dl = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    say(f"  {label}: max|dO|={dmax:.3e} mean|dO|={dmean:.3e} max|dLSE|={dl:.3e}")
    assert dmax <= t["max_o"] and dmean <= t["mean_o"] and dl <= t["lse"]


def test_noalloc_decode_matches_workspace_entry_point_twice():
    say("case noalloc decode: full decode workload, then a smaller padded causal fp16 input")
    check(case("decode_grouped_bf16"), "first call")
    small = case("decode_grouped_bf16", B=3, H=8, H_kv=2, Nq=4, N=1000, dtype="fp16",
                 key_len_range=(1, 1000), seed=4242)
    check(small, "second call")


def test_noalloc_decode_rejects_oversize_without_touching_outputs():
    q = torch.zeros((64, 32, 64, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((64, 8, 8192, 128), dtype=torch.bfloat16, device=DEV)
    o = torch.full_like(q, 3.0)
    lse = torch.full((64, 32, 64), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_decode_noalloc(q, k, k, o, lse, 0.1, True)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.all(lse == 3.0)
    assert "FA_DECODE_NOALLOC_MAX_BYTES" in _lib.load().fa_last_error().decode()
