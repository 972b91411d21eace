"""Plain float64 reference for the exact attention forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.

What it computes is the textbook definition the FlashAttention pages start
from (FlashAttention (ES), section "El problema de la atención estándar";
the same formula in FlashAttention (PT)): softmax(scale * Q K^T) V, with the
full N x N score matrix S and probability matrix P materialised, here in
float64. The pages list masking among the operations the fused kernel
performs (FlashAttention (ES), "Fusión de operaciones en un único kernel") but
do not say which masks; this reference takes the additive -inf reading:

    s_ij    = scale * sum_k Q[i,k] K[j,k]
    allowed = (j < key_len[b]) and (not causal or j <= i)
    s_ij    = -inf where not allowed
    m_i     = max_j s_ij,  e_ij = exp(s_ij - m_i),  l_i = sum_j e_ij
    P_ij    = e_ij / l_i,  O_i = sum_j P_ij V_j,  LSE_i = m_i + log(l_i)

Grouped K/V heads: FlashAttention (ES), "Evolución y desarrollos posteriores",
lists multi-query attention (one K/V head for all query heads) among
FlashAttention-2's additions. K and V may therefore carry H_kv heads with H_kv
dividing H; query head h then takes K/V head h // (H // H_kv) (consecutive
query heads form a group; H_kv = 1 is multi-query, H_kv = H the plain case).

Sliding windows: richer masks are named in the pages only through a title in
the bibliography of FlashAttention (ES) ("FlashMask"). The banded (local)
mask is read as: with window = (left, right), key j is also required to
satisfy j >= i - left and j <= i + right (a negative bound means unbounded);
it combines with the causal and padding masks by AND.

A row with no allowed key gets O_i = 0 and LSE_i = -inf. key_len is clamped to
[0, N]; None means every key is valid. LSE is the natural-log log-sum-exp of
the allowed scaled logits, i.e. the running maximum and running sum of
exponentials that the online softmax keeps (FlashAttention (ES), "Cálculo de
Softmax en línea") folded into one number.

Rows are processed in blocks of at most ``row_block`` full-width rows only to
bound memory; each row's softmax still sees its whole row, so this is the
plain definition and not a tiled algorithm.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def allowed_mask(rows: np.ndarray, N: int, causal: bool, kl: int, window=None) -> np.ndarray:
    """Boolean [len(rows), N]: which keys each query row may attend to."""
    j = np.arange(N)[None, :]
    ok = j < kl
    if causal:
        ok = ok & (j <= rows[:, None])
    if window is not None:
        left, right = window
        if left >= 0:
            ok = ok & (j >= rows[:, None] - left)
        if right >= 0:
            ok = ok & (j <= rows[:, None] + right)
    return ok


def clamp_key_len(key_len, b: int, N: int) -> int:
    if key_len is None:
        return N
    return int(min(max(int(key_len[b]), 0), N))


def masked_scores(q_rows: np.ndarray, k: np.ndarray, scale: float, rows: np.ndarray,
                  causal: bool, kl: int, window=None) -> np.ndarray:
    """scale * q_rows @ k.T with -inf where the mask forbids the pair (float64)."""
    s = float(scale) * (_as64(q_rows) @ _as64(k).T)
    ok = allowed_mask(rows, k.shape[0], causal, kl, window)
    return np.where(ok, s, -np.inf)


def softmax_stats(s: np.ndarray):
    """Row softmax of masked scores. Returns (P, m, l); fully masked rows give P=0."""
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 at masked entries
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, l)[:, None])
    return p, m, l


def _rows_forward(q_rows, k, v, scale, rows, causal, kl, window=None):
    s = masked_scores(q_rows, k, scale, rows, causal, kl, window)
    p, m, l = softmax_stats(s)
    o = p @ _as64(v)
    with np.errstate(divide="ignore"):
        lse = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def kv_head(h: int, H: int, H_kv: int) -> int:
    """The K/V head that query head h of H attends with, for H_kv K/V heads."""
    if H_kv < 1 or H % H_kv:
        raise ValueError("H_kv must divide H")
    return h // (H // H_kv)


def attention_forward(q, k, v, scale: float, causal: bool = False,
                      key_len: Optional[Sequence[int]] = None, row_block: int = 2048,
                      window=None):
    """O [B,H,N,d] and LSE [B,H,N] (float64) for q [B,H,N,d] and k, v [B,H_kv,N,d]."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    o = np.zeros((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        kl = clamp_key_len(key_len, b, N)
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                g = kv_head(h, H, H_kv)
                o[b, h, rows], lse[b, h, rows] = _rows_forward(
                    q[b, h, rows], k[b, g], v[b, g], scale, rows, causal, kl, window)
    return o, lse


def attention_rows(q, k, v, scale: float, causal: bool, key_len, b: int, h: int,
                   rows: Sequence[int], window=None):
    """O and LSE of selected query rows of one (b, h), each row against its full row."""
    rows = np.asarray(rows, dtype=np.int64)
    N = q.shape[2]
    kl = clamp_key_len(key_len, b, N)
    g = kv_head(h, q.shape[1], k.shape[1])
    return _rows_forward(_as64(q[b, h, rows]), _as64(k[b, g]), _as64(v[b, g]), scale, rows,
                         causal, kl, window)


def attention_decode(q, k, v, scale: float, causal: bool = False,
                     key_len: Optional[Sequence[int]] = None):
    """O [B,H,Nq,d] and LSE [B,H,Nq] (float64) for the newest Nq queries of each
    batch entry against its key/value cache: q [B,H,Nq,d], k, v [B,H_kv,Nk,d].

    FlashAttention (ES), "Soluciones especializadas", names attention over the
    KV cache of streaming generation (FlashInfer) as a use of the method, and
    its bibliography lists FlashDecoding++; neither is defined there. Reading:
    batch entry b holds kl_b = clamp(key_len[b], 0, Nk) valid keys (Nk when
    key_len is None), and its Nq queries are the last Nq positions of that
    sequence, so query i sits at position kl_b - Nq + i. Key j is allowed iff
    j < kl_b and, when causal, j <= kl_b - Nq + i. With Nq = Nk and every key
    valid this is attention_forward's mask; a query with no allowed key gets
    O = 0 and LSE = -inf. K/V heads are grouped as in attention_forward.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, H, Nq, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    i = np.arange(Nq)
    j = np.arange(Nk)
    for b in range(B):
        kl = clamp_key_len(key_len, b, Nk)
        ok = np.broadcast_to(j[None, :] < kl, (Nq, Nk))
        if causal:
            ok = ok & (j[None, :] <= (kl - Nq + i)[:, None])
        for h in range(H):
            g = kv_head(h, H, H_kv)
            s = np.where(ok, float(scale) * (q[b, h] @ k[b, g].T), -np.inf)
            p, m, l = softmax_stats(s)
            o[b, h] = p @ v[b, g]
            with np.errstate(divide="ignore"):
                lse[b, h] = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def packed_segments(cu_seqlens, T: int, max_seqlen: Optional[int] = None):
    """(start, length) of each sequence of a packed batch of T rows.

    Sequence b holds rows [cu[b], cu[b+1]); bounds are clamped to [0, T] with the
    end no earlier than the start, and a length above max_seqlen (when given) is
    cut to max_seqlen.
    """
    cu = [int(x) for x in cu_seqlens]
    out = []
    for b in range(len(cu) - 1):
        s0 = min(max(cu[b], 0), T)
        s1 = min(max(cu[b + 1], s0), T)
        n = s1 - s0 if max_seqlen is None else min(s1 - s0, int(max_seqlen))
        out.append((s0, n))
    return out


def attention_varlen(q, k, v, cu_seqlens, scale: float, causal: bool = False,
                     max_seqlen: Optional[int] = None, row_block: int = 2048):
    """O [H,T,d] and LSE [H,T] (float64) of a packed variable-length batch.

    Packed batches of sequences of unequal length are among the richer masks
    named through the FlashMask title in the bibliography of FlashAttention
    (ES); the pages do not define them further. Reading: q is [H, T, d] and k, v
    are [H_kv, T, d]; the sequences are concatenated along the row axis, sequence
    b occupying rows [cu[b], cu[b+1]) of every head (packed_segments), and each
    sequence is attended on its own: row i of sequence b sees exactly the keys of
    sequence b (and, when causal, only those at or before its own position).
    That is the plain forward applied to each sequence as one batch entry, which
    is how it is computed here. K/V heads are grouped as in attention_forward.
    Rows that belong to no sequence are not defined and come back as NaN.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    H, T, d = q.shape
    H_kv = k.shape[0]
    o = np.full((H, T, v.shape[-1]), np.nan)
    lse = np.full((H, T), np.nan)
    for s0, n in packed_segments(cu_seqlens, T, max_seqlen):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            for r0 in range(0, n, row_block):
                rows = np.arange(r0, min(n, r0 + row_block))
                o[h, s0 + rows], lse[h, s0 + rows] = _rows_forward(
                    q[h, s0 + rows], k[g, s0:s0 + n], v[g, s0:s0 + n], scale, rows, causal, n)
    return o, lse


def attention_varlen_rows(q, k, v, cu_seqlens, scale: float, causal: bool, b: int, h: int,
                          rows: Sequence[int], max_seqlen: Optional[int] = None):
    """O and LSE of selected rows (positions within sequence b) of query head h
    of a packed batch, each against its whole sequence."""
    rows = np.asarray(rows, dtype=np.int64)
    s0, n = packed_segments(cu_seqlens, q.shape[1], max_seqlen)[b]
    g = kv_head(h, q.shape[0], k.shape[0])
    return _rows_forward(_as64(q[h, s0 + rows]), _as64(k[g, s0:s0 + n]), _as64(v[g, s0:s0 + n]),
                         scale, rows, causal, n)


def probabilities(q, k, scale: float, causal: bool, key_len, b: int, h: int):
    """The full N x N probability matrix P of one (b, h), for checks on P itself."""
    N = q.shape[2]
    rows = np.arange(N)
    s = masked_scores(q[b, h], k[b, h], scale, rows, causal, clamp_key_len(key_len, b, N))
    return softmax_stats(s)[0]
