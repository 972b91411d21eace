"""GPU parity of fa_fwd_decode (few queries against a key/value cache) with
the float64 oracle's decode definition, on seeded inputs: grouped and plain
K/V heads, one and several queries, several row blocks, ragged and empty
caches, queries with no allowed key, and the full-size decode workload."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_56_amd as fa
import oracle
import workloads as W
from parity import assert_close, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)

CASES = [  # dtype, B, H, H_kv, Nq, Nk, d, causal, key_len
    ("bf16", 2, 8, 2, 1, 1000, 128, True, [1000, 357]),
    ("fp16", 3, 4, 4, 5, 777, 64, True, [777, 10, 3]),    # kl < Nq: rows with no key
    ("bf16", 2, 6, 1, 7, 2000, 128, False, [0, 1999]),    # an empty cache
    ("fp16", 1, 4, 2, 40, 300, 64, True, None),           # 80 rows: three row blocks
    ("bf16", 2, 2, 2, 1, 1, 64, True, None),              # a single key
    ("bf16", 1, 8, 8, 2, 33, 128, False, [33]),           # ragged last tile
    ("fp16", 2, 16, 4, 3, 5000, 128, True, [4999, 2500]),
    ("bf16", 1, 4, 1, 64, 129, 64, True, None),           # Nq near Nk, multi-query
]


def draw(dtype, B, H, H_kv, Nq, Nk, d, causal, key_len, seed):
    spec = W.SPECS["decode_grouped_bf16"].with_shape(
        B=B, H=H, H_kv=H_kv, Nq=Nq, N=Nk, d=d, dtype=dtype, causal=causal,
        scale=1.0 / math.sqrt(d), key_len_range=None, seed=seed)
    w = W.draw(spec)
    kl = None if key_len is None else np.asarray(key_len, dtype=np.int32)
    return w, kl


@pytest.mark.parametrize("case", CASES)
def test_decode_parity(case):
    dtype, B, H, H_kv, Nq, Nk, d, causal, key_len = case
    seed = 12000 + B * 97 + Nq * 13 + Nk
    w, kl = draw(dtype, B, H, H_kv, Nq, Nk, d, causal, key_len, seed)
    say(f"case decode {case} seed={seed}")
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    kl_d = None if kl is None else torch.from_numpy(kl).to(DEV)
    o, lse = fa.decode(q, k, v, scale=w.spec.scale, causal=causal, key_len=kl_d)
    torch.cuda.synchronize()
    qe, ke, ve = w.exact()
    o_ref, lse_ref = oracle.attention_decode(qe, ke, ve, w.spec.scale, causal, kl)
    assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref, dtype,
                 f"decode {case}")


def test_decode_workload_full_size():
    w = W.draw(W.SPECS["decode_grouped_bf16"])
    s = w.spec
    say(f"case decode workload seed={s.seed}")
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    kl = torch.from_numpy(w.key_len).to(DEV)
    o, lse = fa.decode(q, k, v, scale=s.scale, causal=s.causal, key_len=kl)
    torch.cuda.synchronize()
    qe, ke, ve = w.exact()
    o_ref, lse_ref = oracle.attention_decode(qe, ke, ve, s.scale, s.causal, w.key_len_or_none())
    assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref, "bf16",
                 "decode workload")


def test_decode_equals_forward_rows_and_reuses_workspace():
    """Nq = Nk with every key valid is the causal forward; a second call on the
    same workspace with other sizes gives its own correct result."""
    w, _ = draw("bf16", 1, 4, 4, 300, 300, 128, True, None, 12345)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    nbytes = max(fa.decode_workspace_bytes(1, 4, 4, 300, 300, 128),
                 fa.decode_workspace_bytes(2, 8, 2, 1, 4000, 64))
    ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 300), dtype=torch.float32, device=DEV)
    fa.fa_fwd_decode(q, k, v, o, lse, ws, w.spec.scale, True)
    torch.cuda.synchronize()
    qe, ke, ve = w.exact()
    o_ref, lse_ref = oracle.attention_forward(qe, ke, ve, w.spec.scale, True)
    assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref, "bf16",
                 "decode at Nq = Nk")
    w2, kl2 = draw("bf16", 2, 8, 2, 1, 4000, 64, False, [4000, 1234], 12346)
    q2, k2, v2 = (t.to(DEV) for t in (w2.q, w2.k, w2.v))
    o2 = torch.empty_like(q2)
    lse2 = torch.empty((2, 8, 1), dtype=torch.float32, device=DEV)
    fa.fa_fwd_decode(q2, k2, v2, o2, lse2, ws, w2.spec.scale, False, torch.from_numpy(kl2).to(DEV))
    torch.cuda.synchronize()
    qe, ke, ve = w2.exact()
    o_ref, lse_ref = oracle.attention_decode(qe, ke, ve, w2.spec.scale, False, kl2)
    assert_close(o2.double().cpu().numpy(), lse2.double().cpu().numpy(), o_ref, lse_ref, "bf16",
                 "reused workspace")


def test_decode_rejects_small_workspace_without_writing():
    w, _ = draw("bf16", 1, 2, 2, 1, 100, 64, False, None, 3)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 1), 7.0, device=DEV)
    ws = torch.empty(4, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_decode(q, k, v, o, lse, ws, 0.1)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)
