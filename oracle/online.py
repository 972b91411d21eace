"""float64 model of the tiled online-softmax method.

TEST INFRASTRUCTURE ONLY (like the rest of this package).

This is not the reference; it is a CPU model of the *method* the pages
describe, used to check that the method itself is exact before any kernel is
trusted:

* Q, K and V are split into blocks that are processed one at a time
  (FlashAttention (ES), "Tiling y procesamiento por bloques");
* each query row keeps two running values, the current maximum and the sum of
  exponentials, that are corrected as every new key block arrives, so the
  final result equals the full softmax (FlashAttention (ES), "Cálculo de
  Softmax en línea");
* only the final normalised output is produced (FlashAttention (ES),
  "Fusión de operaciones en un único kernel").

Scores are kept in base 2 with ``scale * log2(e)`` folded into one factor,
blocks that a causal or padding mask leaves empty are skipped, and the output
accumulator is rescaled only when a row's running maximum grows. All of that is
an implementation choice that the tests check leaves the result unchanged.

``move_bound`` models a lazier reference: a row's reference maximum is moved
(to the running maximum) only when the block's exponentials, taken against the
current reference, sum to more than ``move_bound`` or to inf/NaN; otherwise the
stale reference is kept and the exponentials may exceed 1. The output and the
sum share every scale factor, so the result is the same softmax for any
reference; the tests check that too.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


def online_forward(q, k, v, scale: float, causal: bool = False, key_len=None,
                   block_q: int = 64, block_k: int = 64, move_bound=None):
    """(O, LSE) of the tiled online-softmax algorithm, float64, inputs [B,H,N,d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, _ = q.shape
    dv = v.shape[-1]
    c = float(scale) * LOG2E
    out = np.zeros((B, H, N, dv))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        kl = N if key_len is None else min(max(int(key_len[b]), 0), N)
        for h in range(H):
            for i0 in range(0, N, block_q):
                i1 = min(N, i0 + block_q)
                rows = np.arange(i0, i1)
                m = np.full(i1 - i0, -np.inf)  # running max, base-2 units
                l = np.zeros(i1 - i0)  # running sum of exponentials
                acc = np.zeros((i1 - i0, dv))
                kv_end = min(kl, i1) if causal else kl
                for j0 in range(0, kv_end, block_k):
                    j1 = min(kv_end, j0 + block_k)
                    cols = np.arange(j0, j1)
                    t = (q[b, h, i0:i1] @ k[b, h, j0:j1].T) * c
                    ok = cols[None, :] < kl
                    if causal:
                        ok = ok & (cols[None, :] <= rows[:, None])
                    t = np.where(ok, t, -np.inf)
                    m_new = np.maximum(m, t.max(axis=1))
                    if move_bound is not None:
                        # keep the stale reference where its exponentials stay in range
                        with np.errstate(invalid="ignore", over="ignore"):
                            s_old = np.exp2(t - m[:, None]).sum(axis=1)
                        keep = np.isfinite(m) & (s_old <= move_bound)
                        m_new = np.where(keep, m, m_new)
                    live = np.isfinite(m_new)
                    base = np.where(live, m_new, 0.0)
                    grew = m_new > m
                    alpha = np.where(grew, np.exp2(np.where(np.isfinite(m), m, -np.inf) - base), 1.0)
                    p = np.exp2(t - base[:, None])
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, h, j0:j1]
                    m = m_new
                done = l > 0
                out[b, h, i0:i1] = np.where(done[:, None], acc / np.where(done, l, 1.0)[:, None], 0.0)
                with np.errstate(divide="ignore"):
                    lse[b, h, i0:i1] = np.where(done, (m + np.log2(np.where(done, l, 1.0))) / LOG2E,
                                                -np.inf)
    return out, lse
