"""fa_fwd_fp8_p8 -- fp8 e4m3 inputs with P rounded to e4m3 for the P V product
(both products on the fp8 matrix cores, the FP8 form of FlashAttention (ES),
"FlashAttention-3 (2024)") -- against the float64 oracle on the dequantised
inputs.

Unit-variance inputs (the distribution the fp8 bounds are stated for) are held
to max|dO| 8e-2, mean|dO| 8e-3, max|dLSE| 1e-2: small and ragged shapes, both
head sizes, causal and padding masks, degenerate key lengths, and sequences
that stream many key tiles. With 5% outlier keys (x8) a row's weight can sit on
two or three keys; rounding each weight to e4m3 moves it by at most u = 2^-4
relative, and since the row sum adds the same rounded values, O moves by at
most 2u / (1 - u) * sum_j w_j |V[j, c] - O[c]| in column c. Those cases are
held to 8e-2 plus that term, computed from the oracle's exact weights.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from parity import assert_close, full_oracle, run, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -4  # e4m3 unit roundoff (3 mantissa bits)


def spec_of(d, N, causal, padded, B=2, H=3, seed=0, outliers=False):
    s = W.SPECS["long_causal_fp8"]
    return s.with_shape(B=B, H=H, N=N, d=d, dtype="fp8", causal=causal, scale=1.0 / math.sqrt(d),
                        key_len_range=(max(0, N // 3), N) if padded else None,
                        outlier_frac=0.05 if outliers else 0.0, seed=seed)


SWEEP_N = [1, 2, 15, 17, 33, 63, 64, 65, 127, 129, 257, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_p8_small_shape_sweep(d, causal):
    for i, N in enumerate(SWEEP_N):
        for padded in (False, True):
            spec = spec_of(d, N, causal, padded, seed=7400 + 17 * i + padded)
            say(f"case p8 d={d} causal={causal} N={N} padded={padded} seed={spec.seed}")
            w = W.draw(spec)
            o, lse = run(w, p8=True)
            o_ref, lse_ref = full_oracle(w)
            assert_close(o, lse, o_ref, lse_ref, "fp8", f"p8 N={N} padded={padded}")


@pytest.mark.parametrize("N,causal,padded,B,H", [(4096, False, False, 1, 2), (4160, True, True, 2, 1),
                                                 (4417, True, False, 1, 1)])
def test_p8_long_sequences(N, causal, padded, B, H):
    spec = spec_of(128, N, causal, padded, B=B, H=H, seed=7500 + N)
    say(f"case p8 long N={N} causal={causal} padded={padded} seed={spec.seed}")
    w = W.draw(spec)
    o, lse = run(w, p8=True)
    o_ref, lse_ref = full_oracle(w)
    assert_close(o, lse, o_ref, lse_ref, "fp8", f"p8 long N={N}")


def test_p8_degenerate_key_lengths():
    spec = spec_of(128, 300, True, False, B=5, H=2, seed=7600)
    w = W.draw(spec)
    w.key_len = np.array([0, 1, -7, 10000, 257], dtype=np.int32)
    say("case p8 degenerate key_len")
    o, lse = run(w, p8=True)
    o_ref, lse_ref = full_oracle(w)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf) and np.all(lse[2] == -np.inf)
    assert_close(o, lse, o_ref, lse_ref, "fp8", "p8 degenerate")


def rounding_term(w, o_ref, lse_ref):
    """2u/(1-u) * sum_j w_j |V[j, c] - O[c]| per (b, h, row, c), from the exact
    inputs and the oracle's O and LSE (w_j = exp(s_j - LSE), 0 where masked)."""
    s = w.spec
    q, k, v = w.exact()
    kl = w.key_len_or_none()
    out = np.zeros_like(o_ref)
    N = s.N
    j = np.arange(N)
    for b in range(s.B):
        n_keys = N if kl is None else int(min(max(kl[b], 0), N))
        for h in range(s.H):
            for r0 in range(0, N, 64):
                r = np.arange(r0, min(N, r0 + 64))
                logit = (q[b, h, r] @ k[b, h].T) * s.scale
                ok = (j[None, :] < n_keys) & (~s.causal | (j[None, :] <= r[:, None]))
                fin = np.isfinite(lse_ref[b, h, r])
                wt = np.where(ok & fin[:, None], np.exp(logit - np.where(fin, lse_ref[b, h, r], 0)[:, None]), 0.0)
                dev = np.abs(v[b, h][None, :, :] - o_ref[b, h, r][:, None, :])
                out[b, h, r] = np.einsum("rj,rjc->rc", wt, dev)
    return 2 * U / (1 - U) * out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_p8_outlier_keys_within_the_rounding_bound(d, causal):
    for i, N in enumerate([48, 127, 300]):
        spec = spec_of(d, N, causal, False, seed=7700 + 31 * i + d + causal, outliers=True)
        say(f"case p8 outliers d={d} causal={causal} N={N} seed={spec.seed}")
        w = W.draw(spec)
        o, lse = run(w, p8=True)
        o_ref, lse_ref = full_oracle(w)
        bound = 8e-2 + rounding_term(w, o_ref, lse_ref)
        err = np.abs(o - o_ref)
        worst = float((err - bound).max())
        say(f"  max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} "
            f"max(|dO| - bound)={worst:.3e} max|dLSE|={np.abs(lse - lse_ref)[np.isfinite(lse_ref)].max():.3e}")
        assert np.all(np.isfinite(o))
        assert worst <= 0.0, f"N={N}: |dO| exceeds 8e-2 + the e4m3 rounding term by {worst}"
        assert err.mean() <= 8e-3
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.abs(lse - lse_ref)[fin].max() <= 1e-2
