"""The seeded generators follow their stated recipe (no attention arithmetic here)."""
import numpy as np
import torch

import workloads as W


def small(name, **kw):
    return W.SPECS[name].with_shape(**kw)


def test_determinism_and_order():
    s = small("decoder_causal_bf16", B=1, H=2, N=16, d=8)
    a, b = W.draw(s), W.draw(s)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    rng = np.random.default_rng(s.seed)
    q = rng.standard_normal((1, 2, 16, 8)).astype(np.float32)
    assert torch.equal(a.q, torch.from_numpy(q).to(torch.bfloat16))


def test_bf16_is_round_to_nearest_even():
    s = small("decoder_causal_bf16", B=1, H=1, N=64, d=64)
    w = W.draw(s)
    rng = np.random.default_rng(s.seed)
    x = rng.standard_normal((1, 1, 64, 64)).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32).view(np.float32)
    assert np.array_equal(w.q.to(torch.float32).numpy(), r)


def test_outliers_and_key_len():
    s = small("long_causal_bf16", H=3, N=500, d=8)
    w = W.draw(s)
    assert w.outlier_rows.shape == (1, 3, 5)
    for h in range(3):
        assert len(set(w.outlier_rows[0, h].tolist())) == 5
    p = small("encoder_padded_bf16", B=50, H=1, N=512, d=8)
    kl = W.draw(p).key_len
    assert kl.dtype == np.int32 and kl.min() >= 256 and kl.max() <= 512


def test_fp8_quantisation_recipe():
    s = small("long_causal_fp8", H=2, N=64, d=16)
    w = W.draw(s)
    assert w.q.dtype == torch.float8_e4m3fn
    rng = np.random.default_rng(s.seed)
    x = rng.standard_normal((1, 2, 64, 16)).astype(np.float32)
    sq = np.float32(np.abs(x).max()) / np.float32(448)
    assert w.descale[0] == float(sq)
    qf = w.q.to(torch.float32).numpy()
    assert np.abs(qf).max() == 448.0
    deq = w.exact()[0]
    # dequantised values are within half an e4m3 ulp (relative 2^-4) of the draw
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 2.0 ** -6 * sq)
    assert rel.max() <= 2.0 ** -4 + 1e-6


def test_oracle_fixture_does_not_drift():
    """tests/golden/oracle_tiny.json was written by tests/golden/make_oracle_fixture.py."""
    import json
    import os
    import oracle
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    for case in json.load(open(path)):
        spec = W.SPECS[case["name"]].with_shape(**case["shape"])
        w = W.draw(spec)
        q, k, v = w.exact()
        o, lse = oracle.attention_forward(q, k, v, spec.scale, spec.causal, w.key_len_or_none())
        # BLAS summation order may differ between hosts: allow a few ulps
        ref_o = np.array([float.fromhex(x) for x in case["o"]])
        ref_l = np.array([float.fromhex(x) for x in case["lse"]])
        assert np.abs(o.reshape(-1) - ref_o).max() <= 1e-14
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(lse.reshape(-1)), fin)
        assert np.abs(lse.reshape(-1)[fin] - ref_l[fin]).max() <= 1e-14


def test_grouped_workload_shapes():
    s = small("long_causal_grouped_bf16", H=8, H_kv=2, N=100, d=8)
    w = W.draw(s)
    assert tuple(w.q.shape) == (1, 8, 100, 8)
    assert tuple(w.k.shape) == (1, 2, 100, 8) and tuple(w.v.shape) == (1, 2, 100, 8)
    assert w.outlier_rows.shape == (1, 2, 1)
    # an ungrouped spec of the same seed draws the same Q
    u = W.draw(s.with_shape(H_kv=None))
    assert torch.equal(w.q, u.q)
