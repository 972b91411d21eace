"""Plain float64 gradients of the exact attention forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module; only the tests and the benchmark's CPU-baseline leg do.

The pages report training speedups (FlashAttention (ES), "Resultados
empíricos": BERT-large, GPT-2, Long-Range Arena), which need the gradients of
the attention output, but they do not write the backward pass out. What is
computed here is the calculus of the definition the oracle's forward uses
(FlashAttention (ES), "El problema de la atención estándar", with the masks of
attention.py): for O = P V with P = softmax(S), S = scale * Q K^T + mask, and an
upstream gradient dO,

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))          (softmax Jacobian, row by row)
    dQ = scale * dS K,     dK = scale * dS^T Q

Masked entries have P = 0 and so no gradient; a row with no allowed key has
P = 0 everywhere and contributes nothing. rowsum(P * dP) equals
rowsum(dO * O), the form a fused backward uses because O is already stored.
K/V heads may be grouped as in attention.py: a K/V head's gradient is the sum
over the query heads that share it.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import allowed_mask, clamp_key_len, kv_head, softmax_stats


def attention_backward(q, k, v, do, scale: float, causal: bool = False,
                       key_len: Optional[Sequence[int]] = None):
    """(dQ, dK, dV) float64 for q, do [B,H,N,d] and k, v [B,H_kv,N,d]."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(N)
    for b in range(B):
        ok = allowed_mask(rows, N, causal, clamp_key_len(key_len, b, N))
        for h in range(H):
            g = kv_head(h, H, H_kv)
            s = np.where(ok, float(scale) * (q[b, h] @ k[b, g].T), -np.inf)
            p = softmax_stats(s)[0]
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = float(scale) * (ds @ k[b, g])
            dk[b, g] += float(scale) * (ds.T @ q[b, h])
    return dq, dk, dv
