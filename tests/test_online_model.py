"""The tiled online-softmax method reproduces the plain definition exactly.

The pages claim the block-by-block softmax with a running maximum and running
sum of exponentials gives the exact result (FlashAttention (ES), "Cálculo de
Softmax en línea"). This checks that claim in float64 for the block shapes,
masks and skip rules the kernel uses, before any kernel is involved.
"""
import math

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("N,d,causal,padded,bq,bk", [
    (1, 8, False, False, 64, 64), (17, 8, True, False, 16, 16), (100, 16, True, True, 32, 64),
    (129, 16, False, True, 128, 64), (257, 32, True, False, 128, 64), (200, 8, True, True, 64, 128),
    (65, 4, False, False, 32, 32),
])
def test_online_equals_oracle(N, d, causal, padded, bq, bk):
    rng = np.random.default_rng(400 + N + bq)
    B, H = 2, 2
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    # outlier keys that arrive late force the running max to grow mid-row
    k[:, :, rng.choice(N, max(1, N // 50), replace=False)] *= 8
    key_len = rng.integers(0, N + 1, size=B) if padded else None
    scale = 1.0 / math.sqrt(d)
    O, L = oracle.attention_forward(q, k, v, scale, causal, key_len)
    O2, L2 = oracle.online_forward(q, k, v, scale, causal, key_len, bq, bk)
    assert np.abs(O - O2).max() <= 1e-12
    fin = np.isfinite(L)
    assert np.array_equal(fin, np.isfinite(L2))
    assert np.abs(L[fin] - L2[fin]).max() <= 1e-12


def test_online_with_large_scale_needs_rescaling():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, 96, 8))
    k = np.sort(rng.standard_normal((1, 1, 96, 8)), axis=2)  # logits grow along the row
    v = rng.standard_normal((1, 1, 96, 8))
    O, L = oracle.attention_forward(q, k, v, 30.0, False, None)
    O2, L2 = oracle.online_forward(q, k, v, 30.0, False, None, 32, 16)
    assert np.abs(O - O2).max() <= 1e-12
    assert np.abs(L - L2).max() <= 1e-11


@pytest.mark.parametrize("bound", [2.0 ** 15, 2.0 ** 64])
@pytest.mark.parametrize("growth", [1.0, 40.0])
def test_lazy_reference_is_exact(bound, growth):
    """A stale reference maximum, moved only when a block's exponentials would
    sum past a bound (or overflow), still gives the exact softmax: O and the
    running sum share every scale factor. Keys grow along the row (up to
    `growth` times) so the reference is stale on most blocks and still has to
    move on some."""
    rng = np.random.default_rng(77 + int(growth))
    B, H, N, d = 2, 2, 300, 16
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) * np.linspace(0.2, growth, N)[None, None, :, None]
    v = rng.standard_normal((B, H, N, d))
    key_len = np.array([N, 173])
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        O, L = oracle.attention_forward(q, k, v, scale, causal, key_len)
        O2, L2 = oracle.online_forward(q, k, v, scale, causal, key_len, 64, 32, move_bound=bound)
        assert np.abs(O - O2).max() <= 1e-12
        fin = np.isfinite(L)
        assert np.array_equal(fin, np.isfinite(L2))
        assert np.abs(L[fin] - L2[fin]).max() <= 1e-11 * max(1.0, np.abs(L[fin]).max())


def test_lazy_reference_kept_for_the_whole_row():
    """Logits that never grow by 64 (base 2) past the first block's maximum:
    with a bound of 2^64 that maximum stays the reference for the whole row,
    and the result is still exact."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 128, 8))
    k = rng.standard_normal((1, 1, 128, 8))
    v = rng.standard_normal((1, 1, 128, 8))
    O, L = oracle.attention_forward(q, k, v, 0.5, False, None)
    O2, L2 = oracle.online_forward(q, k, v, 0.5, False, None, 128, 32, move_bound=2.0 ** 64)
    assert np.abs(O - O2).max() <= 1e-12 and np.abs(L - L2).max() <= 1e-12
