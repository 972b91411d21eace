"""Pins of the float64 backward oracle: torch autograd through its own fp64
attention (a second library), central finite differences of the pinned
forward, and the special cases the masks create."""
import numpy as np
import pytest
import torch

import oracle


def sdpa_grads(q, k, v, do, scale, causal, key_len):
    B, H, N, d = q.shape
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    j = torch.arange(N)
    mask = torch.ones(B, 1, N, N, dtype=torch.bool)
    if causal:
        mask &= (j[None, :] <= j[:, None])[None, None]
    if key_len is not None:
        mask &= (j[None, None, None, :] < torch.as_tensor(key_len)[:, None, None, None])
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                                         enable_gqa=k.shape[1] != H)
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("H,H_kv,causal,padded", [(2, 2, False, False), (3, 3, True, False),
                                                  (4, 2, True, True), (4, 1, False, True)])
def test_backward_matches_torch_autograd_fp64(H, H_kv, causal, padded):
    rng = np.random.default_rng(300 + 10 * H + H_kv + causal)
    B, N, d = 2, 23, 8
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H_kv, N, d))
    v = rng.standard_normal((B, H_kv, N, d))
    do = rng.standard_normal((B, H, N, d))
    key_len = rng.integers(1, N + 1, size=B) if padded else None
    got = oracle.attention_backward(q, k, v, do, 0.35, causal, key_len)
    ref = sdpa_grads(q, k, v, do, 0.35, causal, key_len)
    for g, r in zip(got, ref):
        assert np.abs(g - r).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    rng = np.random.default_rng(17 + causal)
    B, H, N, d = 1, 2, 5, 3
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    key_len = np.array([4])
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.7, causal, key_len)

    def loss(q_, k_, v_):
        o, _ = oracle.attention_forward(q_, k_, v_, 0.7, causal, key_len)
        return float((o * do).sum())

    h = 1e-6
    for x, g, name in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            a_p = [xp if n == name else a for n, a in zip("qkv", args)]
            a_m = [xm if n == name else a for n, a in zip("qkv", args)]
            num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
        assert np.abs(num - g).max() <= 1e-7, name
    # keys at or beyond key_len get no gradient
    assert np.all(dk[:, :, 4:] == 0.0) and np.all(dv[:, :, 4:] == 0.0)


def test_backward_rows_without_keys_and_delta_identity():
    rng = np.random.default_rng(5)
    B, H, N, d = 2, 2, 12, 4
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    key_len = np.array([0, 12])
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, True, key_len)
    assert np.all(dq[0] == 0.0) and np.all(dk[0] == 0.0) and np.all(dv[0] == 0.0)
    # rowsum(P * dP) == rowsum(dO * O): the fused form of the softmax Jacobian term
    o, _ = oracle.attention_forward(q, k, v, 0.5, True, key_len)
    p = oracle.probabilities(q, k, 0.5, True, key_len, 1, 1)
    dp = do[1, 1] @ v[1, 1].T
    assert np.abs((p * dp).sum(1) - (do[1, 1] * o[1, 1]).sum(1)).max() <= 1e-13
