"""Seeded synthetic attention workloads.

This module only draws random inputs and casts them to the storage dtype the
kernel reads. It holds none of the attention arithmetic, so both the GPU path
and the CPU oracle can consume its output without sharing any of the method.

Recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64); draw ``standard_normal`` in
  float64 in the order Q, K, V, Q of shape ``[B, H, Nq, d]`` and K, V of shape
  ``[B, H_kv, N, d]`` (H_kv = H unless the workload groups K/V heads; Nq = N
  except for decode workloads, whose Nq queries meet a cache of N keys), then
  cast each to float32.
* Outlier keys (the long-context decoder workloads): for every (b, K/V head),
  in that order, ``rng.choice(N, round(frac * N), replace=False)`` picks distinct key
  rows that are multiplied by ``outlier_scale`` (in float32, exact).
* Key padding: ``key_len[b] = rng.integers(lo, hi + 1)`` for each batch entry,
  drawn after the outliers; shared by all heads of that batch entry.
* Storage cast: bf16 / fp16 by round-to-nearest-even (torch's ``Tensor.to``);
  fp32 unchanged; fp8 e4m3 (OCP "fn" variant) by per-tensor quantisation with
  ``s = amax(|x|) / 448`` (float32) and ``x_q = e4m3(RNE(clamp(x / s, ±448)))``.
* Packed variable-length batches: the B sequence lengths
  ``rng.integers(lo, hi + 1, size=B)`` are drawn first, then Q of shape
  ``[H, T, d]`` and K, V of shape ``[H_kv, T, d]`` (T = the sum of the lengths;
  the sequences are concatenated along the row axis, ``cu_seqlens`` holds their
  bounds), then the outliers per K/V head over all T rows, then the cast.

``Workload.exact()`` returns the float64 values the stored tensors represent
(for fp8: ``float64(x_q) * float64(s)``); that is what the oracle must consume.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

FP8_MAX = 448.0

DTYPES = ("fp32", "fp16", "bf16", "fp8")
TORCH_STORAGE = {
    "fp32": torch.float32,
    "fp16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8": torch.float8_e4m3fn,
}


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and structure of one attention workload."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    scale: float
    key_len_range: Optional[Tuple[int, int]] = None  # inclusive [lo, hi]
    outlier_frac: float = 0.0
    outlier_scale: float = 8.0
    seed: int = 0
    H_kv: Optional[int] = None  # K/V heads (None: H, no grouping)
    Nq: Optional[int] = None    # decode: queries per head against N cached keys
    window_left: int = -1       # causal sliding window: keys j >= i - window_left
    packed: bool = False        # B sequences of lengths in key_len_range, concatenated

    @property
    def is_decode(self) -> bool:
        return self.Nq is not None

    @property
    def q_len(self) -> int:
        return self.N if self.Nq is None else self.Nq

    @property
    def kv_heads(self) -> int:
        return self.H if self.H_kv is None else self.H_kv

    def flops(self, lengths=None) -> float:
        """Nominal attention FLOP: 4*B*H*N^2*d, halved when causal; decode:
        4*B*H*Nq*N*d (every query against the whole cache); packed batches:
        4*H*d*sum(n_b^2) over the drawn sequence lengths, halved when causal."""
        if self.packed:
            f = 4.0 * self.H * self.d * float(np.sum(np.asarray(lengths, np.float64) ** 2))
            return f / 2 if self.causal else f
        if self.is_decode:
            return 4.0 * self.B * self.H * self.Nq * self.N * self.d
        if self.window_left >= 0 and self.causal:
            return 4.0 * self.B * self.H * self.d * self._band_pairs()
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def exps(self, lengths=None) -> float:
        """Nominal exponentials (one per score): B*H*N^2, halved when causal."""
        if self.packed:
            e = float(self.H) * float(np.sum(np.asarray(lengths, np.float64) ** 2))
            return e / 2 if self.causal else e
        if self.is_decode:
            return float(self.B) * self.H * self.Nq * self.N
        if self.window_left >= 0 and self.causal:
            return float(self.B) * self.H * self._band_pairs()
        e = float(self.B) * self.H * self.N * self.N
        return e / 2 if self.causal else e

    def _band_pairs(self) -> float:
        """(query, key) pairs of a causal band of width window_left + 1."""
        w, n = self.window_left + 1, self.N
        if w >= n:
            return n * (n + 1) / 2.0
        return w * (w + 1) / 2.0 + (n - w) * float(w)

    def with_shape(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


# The five workloads the method is measured on. Seeds are 20260000 + index.
SPECS = {
    "single_head_fp32": Spec("single_head_fp32", 1, 1, 128, 64, "fp32", False,
                             1.0 / math.sqrt(64), seed=20260001),
    "encoder_padded_bf16": Spec("encoder_padded_bf16", 8, 16, 512, 64, "bf16", False,
                                1.0 / 8.0, key_len_range=(256, 512), seed=20260002),
    "decoder_causal_bf16": Spec("decoder_causal_bf16", 8, 12, 1024, 64, "bf16", True,
                                1.0 / 8.0, seed=20260003),
    "long_causal_bf16": Spec("long_causal_bf16", 1, 32, 8192, 128, "bf16", True,
                             1.0 / math.sqrt(128), outlier_frac=0.01, seed=20260004),
    "long_causal_fp8": Spec("long_causal_fp8", 1, 32, 16384, 128, "fp8", True,
                            1.0 / math.sqrt(128), seed=20260005),
    # The long causal decoder shape with 8 K/V heads, each shared by 4 query
    # heads (grouped multi-query attention).
    "long_causal_grouped_bf16": Spec("long_causal_grouped_bf16", 1, 32, 8192, 128, "bf16", True,
                                     1.0 / math.sqrt(128), outlier_frac=0.01, seed=20260006,
                                     H_kv=8),
    # Head dimension 256 at the long causal decoder's FLOP count (half the heads).
    "long_causal_d256_bf16": Spec("long_causal_d256_bf16", 1, 16, 8192, 256, "bf16", True,
                                  1.0 / math.sqrt(256), outlier_frac=0.01, seed=20260008),
    # The long causal decoder shape with a 1024-key sliding window.
    "long_causal_window_bf16": Spec("long_causal_window_bf16", 1, 32, 8192, 128, "bf16", True,
                                    1.0 / math.sqrt(128), outlier_frac=0.01, seed=20260009,
                                    window_left=1023),
    # A packed training batch of the long causal decoder's heads: 16 sequences of
    # 256..8192 tokens concatenated along the row axis (49,314 rows).
    "packed_causal_bf16": Spec("packed_causal_bf16", 16, 32, 8192, 128, "bf16", True,
                               1.0 / math.sqrt(128), key_len_range=(256, 8192),
                               outlier_frac=0.01, seed=20260010, packed=True),
    # One new token per sequence against a 16K-key cache: 16 sequences whose
    # caches hold 8K..16K valid keys, 32 query heads over 8 K/V heads.
    "decode_grouped_bf16": Spec("decode_grouped_bf16", 16, 32, 16384, 128, "bf16", True,
                                1.0 / math.sqrt(128), key_len_range=(8192, 16384),
                                seed=20260007, H_kv=8, Nq=1),
}
ORDER = list(SPECS)


@dataclasses.dataclass
class Workload:
    spec: Spec
    q: torch.Tensor  # CPU, storage dtype, [B,H,N,d] contiguous
    k: torch.Tensor
    v: torch.Tensor
    key_len: Optional[np.ndarray]  # int32 [B] or None
    descale: Tuple[float, float, float]  # (q, k, v); 1.0 unless fp8
    outlier_rows: Optional[np.ndarray] = None  # int64 [B,H_kv,n_out]
    cu_seqlens: Optional[np.ndarray] = None  # packed: int32 [B+1] sequence bounds

    @property
    def lengths(self) -> Optional[np.ndarray]:
        return None if self.cu_seqlens is None else np.diff(self.cu_seqlens)

    def flops(self) -> float:
        return self.spec.flops(self.lengths)

    def exps(self) -> float:
        return self.spec.exps(self.lengths)

    def exact(self):
        """float64 arrays (q, k, v) holding exactly the values the storage represents."""
        out = []
        for t, s in zip((self.q, self.k, self.v), self.descale):
            x = t.to(torch.float64).numpy()
            if self.spec.dtype == "fp8":
                x = x * np.float64(np.float32(s))
            out.append(x)
        return tuple(out)

    def key_len_or_none(self):
        return None if self.key_len is None else self.key_len.copy()


def _quantise_fp8(x: np.ndarray):
    amax = np.float32(np.abs(x).max())
    s = np.float32(amax / np.float32(FP8_MAX)) if amax > 0 else np.float32(1.0)
    y = np.clip(x / s, -FP8_MAX, FP8_MAX).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn), float(s)


def draw(spec: Spec, seed: Optional[int] = None) -> Workload:
    """Generate the workload for ``spec`` (seed defaults to the spec's own)."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    if spec.packed:
        return _draw_packed(spec, rng)
    shape = (spec.B, spec.H, spec.q_len, spec.d)
    kv_shape = (spec.B, spec.kv_heads, spec.N, spec.d)
    q = rng.standard_normal(shape).astype(np.float32)
    k = rng.standard_normal(kv_shape).astype(np.float32)
    v = rng.standard_normal(kv_shape).astype(np.float32)
    rows = None
    if spec.outlier_frac > 0:
        n_out = int(round(spec.outlier_frac * spec.N))
        rows = np.zeros((spec.B, spec.kv_heads, n_out), dtype=np.int64)
        for b in range(spec.B):
            for h in range(spec.kv_heads):
                idx = rng.choice(spec.N, n_out, replace=False)
                rows[b, h] = idx
                k[b, h, idx, :] *= np.float32(spec.outlier_scale)
    key_len = None
    if spec.key_len_range is not None:
        lo, hi = spec.key_len_range
        key_len = rng.integers(lo, hi + 1, size=spec.B).astype(np.int32)
    if spec.dtype == "fp8":
        (qt, sq), (kt, sk), (vt, sv) = (_quantise_fp8(x) for x in (q, k, v))
        descale = (sq, sk, sv)
    else:
        tdt = TORCH_STORAGE[spec.dtype]
        qt, kt, vt = (torch.from_numpy(x).to(tdt) for x in (q, k, v))
        descale = (1.0, 1.0, 1.0)
    return Workload(spec, qt.contiguous(), kt.contiguous(), vt.contiguous(), key_len,
                    descale, rows)


def _draw_packed(spec: Spec, rng) -> Workload:
    lo, hi = spec.key_len_range
    lens = rng.integers(lo, hi + 1, size=spec.B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((spec.H, T, spec.d)).astype(np.float32)
    k = rng.standard_normal((spec.kv_heads, T, spec.d)).astype(np.float32)
    v = rng.standard_normal((spec.kv_heads, T, spec.d)).astype(np.float32)
    rows = None
    if spec.outlier_frac > 0:
        n_out = int(round(spec.outlier_frac * T))
        rows = np.zeros((1, spec.kv_heads, n_out), dtype=np.int64)
        for h in range(spec.kv_heads):
            idx = rng.choice(T, n_out, replace=False)
            rows[0, h] = idx
            k[h, idx, :] *= np.float32(spec.outlier_scale)
    if spec.dtype not in ("bf16", "fp16"):
        raise ValueError("packed workloads are 16-bit")
    tdt = TORCH_STORAGE[spec.dtype]
    qt, kt, vt = (torch.from_numpy(x).to(tdt).contiguous() for x in (q, k, v))
    return Workload(spec, qt, kt, vt, None, (1.0, 1.0, 1.0), rows, cu)


def spec(name: str) -> Spec:
    return SPECS[name]
