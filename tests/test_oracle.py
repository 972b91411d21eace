"""Pins for the float64 oracle, checked against things other than itself.

The pages print no worked numeric example, so every pin here is one of:
arbitrary-precision brute force of the naive softmax formula, a second
implementation (pure-Python two-pass loops), a library routine (torch's CPU
scaled_dot_product_attention in float64), closed forms and invariants of the
definition (FlashAttention (ES), "El problema de la atención estándar").
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt

mpmath.mp.dps = 50


def rand_qkv(rng, B, H, N, d, scale_k=1.0):
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) * scale_k
    v = rng.standard_normal((B, H, N, d))
    return q, k, v


def brute_force(q, k, v, scale, causal, key_len):
    """exp(s)/sum(exp(s)) with no max subtraction, 50 significant digits."""
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        kl = N if key_len is None else min(max(int(key_len[b]), 0), N)
        for h in range(H):
            for i in range(N):
                allowed = [j for j in range(N) if j < kl and (not causal or j <= i)]
                if not allowed:
                    L[b, h, i] = -np.inf
                    continue
                w = {}
                for j in allowed:
                    s = mpmath.mpf(0)
                    for t in range(d):
                        s += mpmath.mpf(float(q[b, h, i, t])) * mpmath.mpf(float(k[b, h, j, t]))
                    w[j] = mpmath.exp(mpmath.mpf(scale) * s)
                z = mpmath.fsum(w.values())
                for t in range(d):
                    O[b, h, i, t] = float(mpmath.fsum(w[j] * mpmath.mpf(float(v[b, h, j, t]))
                                                      for j in allowed) / z)
                L[b, h, i] = float(mpmath.log(z))
    return O, L


def lse_close(a, b, tol):
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.all(a[~fin] == b[~fin])
    if fin.any():
        err = np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin]))
        assert err.max() <= tol, err.max()


CASES = [
    # (N, d, causal, key_len mode)
    (1, 1, False, None), (1, 4, True, None), (2, 3, True, None), (3, 8, False, "rand"),
    (5, 2, True, "rand"), (8, 8, False, None), (13, 5, True, "rand"), (16, 8, True, None),
    (16, 8, False, "rand"), (16, 4, True, "edge"),
]


@pytest.mark.parametrize("N,d,causal,klmode", CASES)
def test_oracle_matches_bruteforce(N, d, causal, klmode):
    rng = np.random.default_rng(1000 + N * 31 + d * 7 + causal)
    B, H = 3, 2
    q, k, v = rand_qkv(rng, B, H, N, d)
    scale = 1.0 / math.sqrt(d) * 1.7
    key_len = None
    if klmode == "rand":
        key_len = rng.integers(0, N + 1, size=B)
    elif klmode == "edge":
        key_len = np.array([0, 1, N + 5])  # empty, one key, clamped above N
    O, L = oracle.attention_forward(q, k, v, scale, causal, key_len)
    Ob, Lb = brute_force(q, k, v, scale, causal, key_len)
    assert np.abs(O - Ob).max() <= 1e-13
    lse_close(L, Lb, 1e-13)


def test_fully_masked_rows_are_zero_and_neg_inf():
    rng = np.random.default_rng(5)
    q, k, v = rand_qkv(rng, 2, 2, 7, 3)
    O, L = oracle.attention_forward(q, k, v, 0.5, True, np.array([0, 3]))
    assert np.all(O[0] == 0) and np.all(L[0] == -np.inf)
    assert np.all(np.isfinite(L[1]))


def two_pass_loops(q, k, v, scale, causal, kl):
    """Pure-Python safe softmax: pass 1 the row max, pass 2 exp-sum and normalise."""
    N, d = len(q), len(q[0])
    O = [[0.0] * d for _ in range(N)]
    L = [-math.inf] * N
    for i in range(N):
        s = []
        for j in range(N):
            if j < kl and (not causal or j <= i):
                s.append((j, scale * math.fsum(q[i][t] * k[j][t] for t in range(d))))
        if not s:
            continue
        mx = max(x for _, x in s)
        e = [(j, math.exp(x - mx)) for j, x in s]
        z = math.fsum(x for _, x in e)
        for t in range(d):
            O[i][t] = math.fsum(w * v[j][t] for j, w in e) / z
        L[i] = mx + math.log(z)
    return np.array(O), np.array(L)


@pytest.mark.parametrize("N,causal,kl", [(4, False, 4), (9, True, 9), (16, True, 11),
                                         (16, False, 5), (12, False, 0)])
def test_oracle_matches_two_pass_loops(N, causal, kl):
    rng = np.random.default_rng(77 + N)
    q, k, v = rand_qkv(rng, 1, 1, N, 6)
    O, L = oracle.attention_forward(q, k, v, 0.4, causal, np.array([kl]))
    O2, L2 = two_pass_loops(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.4, causal, kl)
    assert np.abs(O[0, 0] - O2).max() <= 1e-14
    lse_close(L[0, 0], L2, 1e-14)


@pytest.mark.parametrize("N,d,causal,padded", [(33, 16, False, False), (64, 8, True, False),
                                               (50, 32, False, True), (70, 16, True, True)])
def test_oracle_matches_torch_sdpa_fp64(N, d, causal, padded):
    rng = np.random.default_rng(900 + N)
    B, H = 2, 3
    q, k, v = rand_qkv(rng, B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    key_len = rng.integers(1, N + 1, size=B) if padded else None
    O, L = oracle.attention_forward(q, k, v, scale, causal, key_len)
    j = torch.arange(N)
    mask = torch.ones(B, 1, N, N, dtype=torch.bool)
    if causal:
        mask &= (j[None, :] <= j[:, None])[None, None]
    if padded:
        mask &= (j[None, None, None, :] < torch.as_tensor(key_len)[:, None, None, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=scale)
    assert np.abs(O - ref.numpy()).max() <= 1e-12
    # LSE by the library's own logsumexp over the same masked logits
    s = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) * scale
    s = s.masked_fill(~mask, -math.inf)
    lse_close(L, torch.logsumexp(s, dim=-1).numpy(), 1e-13)


def test_probability_rows_sum_to_one_and_mask_is_exact_zero():
    rng = np.random.default_rng(3)
    N = 40
    q, k, _ = rand_qkv(rng, 1, 1, N, 8)
    key_len = np.array([29])
    P = oracle.probabilities(q, k, 0.7, True, key_len, 0, 0)
    assert np.all(P >= 0)
    assert np.abs(P.sum(axis=1) - 1).max() <= 1e-14
    i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
    masked = (j > i) | (j >= 29)
    assert np.all(P[masked] == 0.0)
    assert np.all(P[~masked] > 0.0)


def test_all_equal_keys_give_mean_of_allowed_values():
    rng = np.random.default_rng(11)
    N, d = 37, 5
    q = rng.standard_normal((2, 1, N, d))
    krow = rng.standard_normal(d)
    k = np.broadcast_to(krow, (2, 1, N, d)).copy()
    v = rng.standard_normal((2, 1, N, d))
    scale = 0.3
    key_len = np.array([N, 20])
    O, L = oracle.attention_forward(q, k, v, scale, True, key_len)
    for b, kl in enumerate(key_len):
        for i in range(N):
            n = min(i + 1, kl)
            np.testing.assert_allclose(O[b, 0, i], v[b, 0, :n].mean(axis=0), rtol=0, atol=1e-14)
            s = scale * float(q[b, 0, i] @ krow)
            assert abs(L[b, 0, i] - (s + math.log(n))) <= 1e-13 * max(1, abs(s))


def test_one_dominant_logit_selects_its_value_row():
    rng = np.random.default_rng(12)
    N, d = 64, 16
    q, k, v = rand_qkv(rng, 1, 1, N, d)
    i, jstar, c = 40, 17, 40.0
    k[0, 0, jstar] = c * q[0, 0, i]
    scale = 1.0 / 4.0
    O, _ = oracle.attention_forward(q, k, v, scale, False, None)
    s = scale * (k[0, 0] @ q[0, 0, i])
    bound = 2 * np.abs(v).max() * np.exp(np.delete(s, jstar) - s[jstar]).sum()
    assert bound < 1e-6
    assert np.abs(O[0, 0, i] - v[0, 0, jstar]).max() <= bound


def test_causal_row_zero_and_single_key():
    rng = np.random.default_rng(13)
    q, k, v = rand_qkv(rng, 2, 3, 19, 7)
    O, L = oracle.attention_forward(q, k, v, 0.9, True, None)
    assert np.array_equal(O[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(L[:, :, 0], 0.9 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=1e-15, atol=1e-15)
    q1, k1, v1 = rand_qkv(rng, 2, 2, 1, 9)
    O1, L1 = oracle.attention_forward(q1, k1, v1, 0.2, False, None)
    assert np.array_equal(O1, v1)
    np.testing.assert_allclose(L1[..., 0], 0.2 * np.einsum("bhd,bhd->bh", q1[:, :, 0], k1[:, :, 0]),
                               rtol=1e-15, atol=1e-15)


def test_row_shift_invariance_via_key_offset():
    """K -> K + 1 u^T adds scale*q_i.u to every logit of row i: O unchanged, LSE shifted."""
    rng = np.random.default_rng(14)
    q, k, v = rand_qkv(rng, 2, 2, 45, 8)
    u = rng.standard_normal(8) * 3
    key_len = np.array([45, 30])
    O, L = oracle.attention_forward(q, k, v, 0.35, True, key_len)
    O2, L2 = oracle.attention_forward(q, k + u, v, 0.35, True, key_len)
    assert np.abs(O - O2).max() <= 1e-12
    np.testing.assert_allclose(L2 - L, 0.35 * (q @ u), rtol=0, atol=1e-12)


def test_linearity_in_values_and_constant_values():
    rng = np.random.default_rng(15)
    q, k, v1 = rand_qkv(rng, 1, 2, 30, 6)
    v2 = rng.standard_normal(v1.shape)
    A = rng.standard_normal((6, 6))
    f = lambda v: oracle.attention_forward(q, k, v, 0.5, True, np.array([23]))[0]  # noqa: E731
    assert np.abs(f(v1 + v2) - f(v1) - f(v2)).max() <= 1e-13
    assert np.abs(f(v1 @ A) - f(v1) @ A).max() <= 1e-12
    assert np.abs(f(np.ones_like(v1)) - 1.0).max() <= 1e-15


def test_permutation_equivariance_without_mask():
    rng = np.random.default_rng(16)
    q, k, v = rand_qkv(rng, 1, 1, 25, 4)
    O, L = oracle.attention_forward(q, k, v, 0.6, False, None)
    pk = rng.permutation(25)
    pq = rng.permutation(25)
    O2, L2 = oracle.attention_forward(q[:, :, pq], k[:, :, pk], v[:, :, pk], 0.6, False, None)
    assert np.abs(O2 - O[:, :, pq]).max() <= 1e-14
    assert np.abs(L2 - L[:, :, pq]).max() <= 1e-13


def test_huge_logits_stay_finite_and_exact():
    """Scale 200: exp(s) overflows float64 without the max subtraction."""
    rng = np.random.default_rng(17)
    q, k, v = rand_qkv(rng, 1, 2, 12, 4)
    O, L = oracle.attention_forward(q, k, v, 200.0, True, None)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    Ob, Lb = brute_force(q, k, v, 200.0, True, None)
    assert np.abs(O - Ob).max() <= 1e-13
    lse_close(L, Lb, 1e-14)


def test_rows_api_matches_full():
    rng = np.random.default_rng(18)
    q, k, v = rand_qkv(rng, 2, 2, 90, 8)
    key_len = np.array([90, 47])
    O, L = oracle.attention_forward(q, k, v, 0.25, True, key_len, row_block=16)
    rows = [0, 1, 46, 47, 89]
    o, lse = oracle.attention_rows(q, k, v, 0.25, True, key_len, 1, 1, rows)
    assert np.array_equal(o, O[1, 1, rows])
    assert np.array_equal(lse, L[1, 1, rows])


# --- the pins must catch plausible mistakes planted in the oracle -------------

def _brute_check(monkeypatch_fn=None):
    rng = np.random.default_rng(99)
    q, k, v = rand_qkv(rng, 2, 2, 9, 4)
    key_len = np.array([9, 6])
    Ob, Lb = brute_force(q, k, v, 0.8, True, key_len)
    O, L = oracle.attention_forward(q, k, v, 0.8, True, key_len)
    return np.abs(O - Ob).max() <= 1e-13 and np.allclose(L, Lb, rtol=1e-13, atol=1e-13)


MUTANTS = {
    "strict_causal": lambda rows, N, causal, kl, window=None: (
        (np.arange(N)[None, :] < kl) & (np.arange(N)[None, :] < rows[:, None])),
    "key_len_off_by_one": lambda rows, N, causal, kl, window=None: (
        (np.arange(N)[None, :] <= kl) & (np.arange(N)[None, :] <= rows[:, None])),
    "mask_ignored": lambda rows, N, causal, kl, window=None: np.ones((len(rows), N), bool),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mask_mistakes(monkeypatch, name):
    assert _brute_check()
    monkeypatch.setattr(oatt, "allowed_mask", MUTANTS[name])
    assert not _brute_check()


def test_pins_catch_planted_arithmetic_mistakes(monkeypatch):
    orig = oatt.masked_scores

    def no_scale(q_rows, k, scale, rows, causal, kl, window=None):
        return orig(q_rows, k, 1.0, rows, causal, kl, window)

    def transposed(q_rows, k, scale, rows, causal, kl, window=None):
        s = float(scale) * (np.asarray(k, np.float64) @ np.asarray(q_rows, np.float64).T)
        return np.where(oatt.allowed_mask(rows, k.shape[0], causal, kl), s, -np.inf)

    for bad in (no_scale, transposed):
        monkeypatch.setattr(oatt, "masked_scores", bad)
        assert not _brute_check()
        monkeypatch.setattr(oatt, "masked_scores", orig)

    orig_sm = oatt.softmax_stats

    def log2_lse(s):
        p, m, l = orig_sm(s)
        return p, m, np.exp2(np.log(l))  # LSE would come out in the wrong base

    monkeypatch.setattr(oatt, "softmax_stats", log2_lse)
    assert not _brute_check()


# ---------------------------------------------------------------------------
# Grouped K/V heads (multi-query attention and its grouped form)

@pytest.mark.parametrize("H,H_kv,causal,padded", [(6, 2, False, False), (6, 3, True, False),
                                                  (4, 1, True, True), (8, 4, False, True)])
def test_grouped_oracle_matches_torch_sdpa_gqa_fp64(H, H_kv, causal, padded):
    rng = np.random.default_rng(40 + H * 7 + H_kv)
    B, N, d = 2, 37, 16
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H_kv, N, d))
    v = rng.standard_normal((B, H_kv, N, d))
    scale = 0.3
    key_len = rng.integers(1, N + 1, size=B) if padded else None
    O, L = oracle.attention_forward(q, k, v, scale, causal, key_len)
    j = torch.arange(N)
    mask = torch.ones(B, 1, N, N, dtype=torch.bool)
    if causal:
        mask &= (j[None, :] <= j[:, None])[None, None]
    if padded:
        mask &= (j[None, None, None, :] < torch.as_tensor(key_len)[:, None, None, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=scale,
        enable_gqa=True)
    assert np.abs(O - ref.numpy()).max() <= 1e-12
    # rows of one head through the row entry point agree with the whole-tensor one
    h = H - 1
    o_r, l_r = oracle.attention_rows(q, k, v, scale, causal, key_len, 1, h, [0, 5, N - 1])
    assert np.abs(o_r - O[1, h, [0, 5, N - 1]]).max() == 0.0
    lse_close(l_r, L[1, h, [0, 5, N - 1]], 0.0)


def test_grouped_heads_follow_consecutive_grouping():
    # Query heads 0,1,2 use K/V head 0 and 3,4,5 use head 1: the result equals
    # the ungrouped forward on K/V heads repeated in that order, and differs
    # from the interleaved order (h % H_kv) on the same data.
    rng = np.random.default_rng(77)
    q = rng.standard_normal((1, 6, 20, 8))
    k = rng.standard_normal((1, 2, 20, 8))
    v = rng.standard_normal((1, 2, 20, 8))
    O, L = oracle.attention_forward(q, k, v, 0.5, True)
    O_rep, L_rep = oracle.attention_forward(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1),
                                            0.5, True)
    assert np.abs(O - O_rep).max() == 0.0 and np.abs(L - L_rep).max() == 0.0
    O_int, _ = oracle.attention_forward(q, np.tile(k, (1, 3, 1, 1)), np.tile(v, (1, 3, 1, 1)),
                                        0.5, True)
    assert np.abs(O - O_int).max() > 1e-3


def test_multi_query_with_equal_query_heads_gives_equal_outputs():
    rng = np.random.default_rng(5)
    q1 = rng.standard_normal((1, 1, 24, 8))
    q = np.repeat(q1, 4, axis=1)
    k = rng.standard_normal((1, 1, 24, 8))
    v = rng.standard_normal((1, 1, 24, 8))
    O, L = oracle.attention_forward(q, k, v, 0.4, False)
    O1, L1 = oracle.attention_forward(q1, k, v, 0.4, False)
    for h in range(4):
        assert np.abs(O[0, h] - O1[0, 0]).max() == 0.0
        lse_close(L[0, h], L1[0, 0], 0.0)
    with pytest.raises(ValueError):
        oracle.attention_forward(q, np.zeros((1, 3, 24, 8)), np.zeros((1, 3, 24, 8)), 0.4, False)


# ---------------------------------------------------------------------------
# Decode: the newest Nq queries against a key/value cache of kl_b valid keys

def brute_force_decode(q, k, v, scale, causal, key_len):
    """Decode definition written out with no max subtraction, 50 digits."""
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    O = np.zeros((B, H, Nq, d))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        kl = Nk if key_len is None else min(max(int(key_len[b]), 0), Nk)
        for h in range(H):
            g = h // (H // H_kv)
            for i in range(Nq):
                pos = kl - Nq + i
                allowed = [j for j in range(Nk) if j < kl and (not causal or j <= pos)]
                if not allowed:
                    L[b, h, i] = -np.inf
                    continue
                w = {j: mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(
                    mpmath.mpf(float(q[b, h, i, t])) * mpmath.mpf(float(k[b, g, j, t]))
                    for t in range(d))) for j in allowed}
                z = mpmath.fsum(w.values())
                for t in range(d):
                    O[b, h, i, t] = float(mpmath.fsum(w[j] * mpmath.mpf(float(v[b, g, j, t]))
                                                      for j in allowed) / z)
                L[b, h, i] = float(mpmath.log(z))
    return O, L


@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_brute_force(causal):
    rng = np.random.default_rng(611 + causal)
    B, H, H_kv, Nq, Nk, d = 3, 4, 2, 3, 11, 4
    q = rng.standard_normal((B, H, Nq, d))
    k = rng.standard_normal((B, H_kv, Nk, d))
    v = rng.standard_normal((B, H_kv, Nk, d))
    key_len = np.array([11, 5, 2])  # the last entry leaves query 0 no key when causal
    O, L = oracle.attention_decode(q, k, v, 0.6, causal, key_len)
    O2, L2 = brute_force_decode(q, k, v, 0.6, causal, key_len)
    assert np.abs(O - O2).max() <= 1e-13
    lse_close(L, L2, 1e-13)
    if causal:
        assert np.all(O[2, :, 0] == 0.0) and np.all(L[2, :, 0] == -np.inf)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_with_every_position_is_the_forward(causal):
    rng = np.random.default_rng(44)
    q, k, v = rand_qkv(rng, 2, 3, 29, 8)
    O, L = oracle.attention_decode(q, k, v, 0.3, causal)
    O2, L2 = oracle.attention_forward(q, k, v, 0.3, causal)
    assert np.abs(O - O2).max() == 0.0
    lse_close(L, L2, 0.0)


def test_decode_rows_are_the_causal_forward_rows_at_their_positions():
    # Place the Nq decode queries at positions kl-Nq .. kl-1 of a full query
    # sequence over the first kl keys: the causal forward's rows there are the
    # decode outputs.
    rng = np.random.default_rng(45)
    B, H, Nq, Nk, d = 2, 2, 4, 30, 8
    q = rng.standard_normal((B, H, Nq, d))
    k = rng.standard_normal((B, H, Nk, d))
    v = rng.standard_normal((B, H, Nk, d))
    key_len = np.array([30, 17])
    O, L = oracle.attention_decode(q, k, v, 0.4, True, key_len)
    for b, kl in enumerate(key_len):
        qf = rng.standard_normal((1, H, kl, d))
        qf[0, :, kl - Nq:] = q[b]
        Of, Lf = oracle.attention_forward(qf, k[b:b + 1, :, :kl], v[b:b + 1, :, :kl], 0.4, True)
        assert np.abs(O[b] - Of[0, :, kl - Nq:]).max() <= 1e-14
        lse_close(L[b], Lf[0, :, kl - Nq:], 1e-14)


def test_decode_matches_torch_sdpa_bottom_right_mask():
    rng = np.random.default_rng(46)
    B, H, H_kv, Nq, Nk, d = 3, 6, 3, 5, 40, 16
    q = rng.standard_normal((B, H, Nq, d))
    k = rng.standard_normal((B, H_kv, Nk, d))
    v = rng.standard_normal((B, H_kv, Nk, d))
    key_len = np.array([40, 23, 9])
    O, _ = oracle.attention_decode(q, k, v, 0.25, True, key_len)
    j = torch.arange(Nk)
    i = torch.arange(Nq)
    kl = torch.as_tensor(key_len)
    mask = (j[None, None, :] < kl[:, None, None]) & (
        j[None, None, :] <= (kl[:, None, None] - Nq + i[None, :, None]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask[:, None],
        scale=0.25, enable_gqa=True)
    assert np.abs(O - ref.numpy()).max() <= 1e-12


def test_single_query_decode_sees_every_valid_key():
    rng = np.random.default_rng(47)
    q = rng.standard_normal((2, 2, 1, 8))
    k = rng.standard_normal((2, 2, 25, 8))
    v = rng.standard_normal((2, 2, 25, 8))
    key_len = np.array([25, 7])
    a = oracle.attention_decode(q, k, v, 0.5, True, key_len)
    b = oracle.attention_decode(q, k, v, 0.5, False, key_len)
    assert np.abs(a[0] - b[0]).max() == 0.0


# ---------------------------------------------------------------------------
# Sliding-window (banded) masks

def brute_force_window(q, k, v, scale, causal, key_len, left, right):
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        kl = N if key_len is None else min(max(int(key_len[b]), 0), N)
        for h in range(H):
            for i in range(N):
                allowed = [j for j in range(N) if j < kl and (not causal or j <= i)
                           and (left < 0 or j >= i - left) and (right < 0 or j <= i + right)]
                if not allowed:
                    L[b, h, i] = -np.inf
                    continue
                w = {j: mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(
                    mpmath.mpf(float(q[b, h, i, t])) * mpmath.mpf(float(k[b, h, j, t]))
                    for t in range(d))) for j in allowed}
                z = mpmath.fsum(w.values())
                for t in range(d):
                    O[b, h, i, t] = float(mpmath.fsum(w[j] * mpmath.mpf(float(v[b, h, j, t]))
                                                      for j in allowed) / z)
                L[b, h, i] = float(mpmath.log(z))
    return O, L


@pytest.mark.parametrize("causal,left,right", [(True, 3, -1), (False, 2, 4), (False, -1, 1),
                                               (True, 0, -1)])
def test_window_matches_brute_force(causal, left, right):
    rng = np.random.default_rng(70 + left + 3 * right + causal)
    q, k, v = rand_qkv(rng, 2, 2, 13, 4)
    key_len = np.array([13, 9])
    O, L = oracle.attention_forward(q, k, v, 0.5, causal, key_len, window=(left, right))
    O2, L2 = brute_force_window(q, k, v, 0.5, causal, key_len, left, right)
    assert np.abs(O - O2).max() <= 1e-13
    lse_close(L, L2, 1e-13)


def test_wide_window_is_no_window_and_zero_window_is_self():
    rng = np.random.default_rng(71)
    q, k, v = rand_qkv(rng, 1, 2, 20, 8)
    a = oracle.attention_forward(q, k, v, 0.3, True, window=(19, -1))
    b = oracle.attention_forward(q, k, v, 0.3, True)
    assert np.abs(a[0] - b[0]).max() == 0.0
    O, L = oracle.attention_forward(q, k, v, 0.3, True, window=(0, -1))
    assert np.abs(O - v).max() <= 1e-15
    assert np.abs(L - 0.3 * np.einsum("bhnd,bhnd->bhn", q, k)).max() <= 1e-12


def test_window_matches_torch_sdpa_band_mask():
    rng = np.random.default_rng(72)
    B, H, N, d = 2, 3, 40, 16
    q, k, v = rand_qkv(rng, B, H, N, d)
    key_len = np.array([40, 31])
    O, _ = oracle.attention_forward(q, k, v, 0.25, False, key_len, window=(5, 7))
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    band = (j >= i - 5) & (j <= i + 7)
    mask = band[None, None] & (j[None, None] < torch.as_tensor(key_len)[:, None, None, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.25)
    assert np.abs(O - ref.numpy()).max() <= 1e-12


# ---------------------------------------------------------------------------
# Packed variable-length batches

def segment_ids(cu, T):
    """Sequence index of every packed row (-1 for rows in no sequence)."""
    seg = np.full(T, -1)
    for b in range(len(cu) - 1):
        seg[cu[b]:cu[b + 1]] = b
    return seg


def brute_force_packed(q, k, v, cu, scale, causal):
    """Naive exp(s)/sum(exp(s)) over the whole packed row axis, 50 digits:
    packed row i sees packed row j iff both lie in one sequence (and j <= i
    when causal)."""
    H, T, d = q.shape
    group = H // k.shape[0]
    seg = segment_ids(cu, T)
    O = np.full((H, T, d), np.nan)
    L = np.full((H, T), np.nan)
    for h in range(H):
        g = h // group
        for i in range(T):
            if seg[i] < 0:
                continue
            allowed = [j for j in range(T) if seg[j] == seg[i] and (not causal or j <= i)]
            w = {j: mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(
                mpmath.mpf(float(q[h, i, t])) * mpmath.mpf(float(k[g, j, t])) for t in range(d)))
                for j in allowed}
            z = mpmath.fsum(w.values())
            for t in range(d):
                O[h, i, t] = float(mpmath.fsum(w[j] * mpmath.mpf(float(v[g, j, t]))
                                               for j in allowed) / z)
            L[h, i] = float(mpmath.log(z))
    return O, L


PACKED = [([0, 5, 5, 6, 14], 2, 1), ([0, 16], 1, 1), ([0, 3, 9, 12], 4, 2), ([2, 7, 13], 2, 2)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cu,H,H_kv", PACKED)
def test_packed_matches_brute_force(cu, H, H_kv, causal):
    rng = np.random.default_rng(80 + len(cu) + H + causal)
    T, d = 16, 4
    q = rng.standard_normal((H, T, d))
    k = rng.standard_normal((H_kv, T, d))
    v = rng.standard_normal((H_kv, T, d))
    O, L = oracle.attention_varlen(q, k, v, cu, 0.5, causal)
    O2, L2 = brute_force_packed(q, k, v, cu, 0.5, causal)
    assert np.array_equal(np.isnan(O), np.isnan(O2)) and np.array_equal(np.isnan(L), np.isnan(L2))
    ok = ~np.isnan(L2)
    assert np.abs(O[~np.isnan(O2)] - O2[~np.isnan(O2)]).max() <= 1e-13
    assert np.abs(L[ok] - L2[ok]).max() <= 1e-13


def test_packed_matches_torch_sdpa_block_diagonal_mask():
    rng = np.random.default_rng(83)
    cu = [0, 37, 38, 100, 161]
    H, H_kv, T, d = 4, 2, 161, 16
    q = rng.standard_normal((H, T, d))
    k = rng.standard_normal((H_kv, T, d))
    v = rng.standard_normal((H_kv, T, d))
    seg = torch.as_tensor(segment_ids(cu, T))
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    for causal in (False, True):
        O, L = oracle.attention_varlen(q, k, v, cu, 0.3, causal)
        mask = (seg[:, None] == seg[None, :]) & ((j <= i) if causal else True)
        kk = torch.from_numpy(np.repeat(k, 2, axis=0))
        vv = torch.from_numpy(np.repeat(v, 2, axis=0))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], kk[None], vv[None], attn_mask=mask, scale=0.3)[0]
        assert np.abs(O - ref.numpy()).max() <= 1e-12


def test_packed_equals_padded_batch_with_key_lengths():
    # The same sequences laid out padded ([B, H, n_max, d], garbage past each
    # length, key_len = lengths) through the padded forward: the valid rows agree.
    rng = np.random.default_rng(84)
    lens = [9, 1, 30, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, T, d, n_max = 3, int(cu[-1]), 8, max(lens)
    q = rng.standard_normal((H, T, d))
    k = rng.standard_normal((H, T, d))
    v = rng.standard_normal((H, T, d))
    for causal in (False, True):
        O, L = oracle.attention_varlen(q, k, v, cu, 0.4, causal)
        pad = [rng.standard_normal((len(lens), H, n_max, d)) * 50 for _ in range(3)]
        for b, n in enumerate(lens):
            for x, y in zip(pad, (q, k, v)):
                x[b, :, :n] = y[:, cu[b]:cu[b] + n]
        Op, Lp = oracle.attention_forward(*pad, 0.4, causal, key_len=np.array(lens))
        for b, n in enumerate(lens):
            assert np.abs(O[:, cu[b]:cu[b] + n] - Op[b, :, :n]).max() <= 1e-13
            assert np.abs(L[:, cu[b]:cu[b] + n] - Lp[b, :, :n]).max() <= 1e-13


def test_packed_uncovered_rows_clamping_and_max_seqlen():
    rng = np.random.default_rng(85)
    q, k, v = (rng.standard_normal((2, 12, 4)) for _ in range(3))
    O, L = oracle.attention_varlen(q, k, v, [1, 4, 4, 9], 0.5, True)
    assert np.isnan(L[:, [0, 9, 10, 11]]).all() and not np.isnan(L[:, 1:9]).any()
    # causal first row of a sequence sees only itself
    assert np.abs(O[:, 1] - v[:, 1]).max() <= 1e-15 and np.abs(O[:, 4] - v[:, 4]).max() <= 1e-15
    # bounds past T are clamped, a decreasing end gives an empty sequence
    assert oracle.packed_segments([0, 5, 3, 40], 12) == [(0, 5), (5, 0), (3, 9)]
    # max_seqlen cuts a sequence to its first rows, which keep their values
    O2, L2 = oracle.attention_varlen(q, k, v, [1, 4, 4, 9], 0.5, True, max_seqlen=3)
    assert np.isnan(L2[:, 7:9]).all()
    assert np.array_equal(O2[:, 4:7], O[:, 4:7]) and np.array_equal(L2[:, 1:7], L[:, 1:7])


def test_packed_rows_api_matches_full():
    rng = np.random.default_rng(86)
    cu = [0, 20, 57]
    q = rng.standard_normal((4, 57, 8))
    k, v = (rng.standard_normal((2, 57, 8)) for _ in range(2))
    O, L = oracle.attention_varlen(q, k, v, cu, 0.5, True)
    rows = [0, 5, 36]
    o, lse = oracle.attention_varlen_rows(q, k, v, cu, 0.5, True, 1, 3, rows)
    assert np.array_equal(o, O[3, 20 + np.array(rows)]) and np.array_equal(lse, L[3, 20 + np.array(rows)])


def test_pins_catch_planted_segment_mistake(monkeypatch):
    # A sequence that reaches one row past its end must fail the brute force.
    orig = oatt.packed_segments
    monkeypatch.setattr(oatt, "packed_segments",
                        lambda cu, T, m=None: [(s, min(n + 1, T - s)) for s, n in orig(cu, T, m)])
    rng = np.random.default_rng(87)
    q, k, v = (rng.standard_normal((1, 16, 4)) for _ in range(3))
    cu = [0, 3, 9, 16]
    O, _ = oracle.attention_varlen(q, k, v, cu, 0.5, False)
    O2, _ = brute_force_packed(q, k, v, cu, 0.5, False)
    assert np.abs(O - O2).max() > 1e-3
