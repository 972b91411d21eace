"""Exact IO-aware attention forward for AMD Instinct MI355X (gfx950).

Python face of libfa (include/fa.h). ``fa_fwd`` / ``fa_fwd_fp8`` / ``fa_fwd_gqa`` /
``fa_fwd_window`` / ``fa_fwd_varlen`` / ``fa_fwd_decode`` / ``fa_fwd_decode_noalloc`` / ``fa_bwd`` marshal torch tensors' device pointers and the current stream
into the C entry points of the same names; ``fwd`` (and its positional twin ``forward``) additionally
allocates O and LSE. Nothing here computes any part of the attention.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (FaError, abi_version, bwd_workspace_bytes, decode_workspace_bytes,  # noqa: F401
                   load, status_name)

_DTYPE = {
    torch.float32: _lib.FA_DTYPE_FP32,
    torch.float16: _lib.FA_DTYPE_FP16,
    torch.bfloat16: _lib.FA_DTYPE_BF16,
    torch.float8_e4m3fn: _lib.FA_DTYPE_FP8_E4M3,
}


def out_dtype(in_dtype: torch.dtype) -> torch.dtype:
    return torch.bfloat16 if in_dtype == torch.float8_e4m3fn else in_dtype


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check_inputs(q, k, v, o, lse, key_len, grouped=False):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, k, v must be [B, H, N, d] tensors and k, v of one shape")
    if grouped:
        B, H, N, d = q.shape
        if (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d) or H % k.shape[1] != 0:
            raise ValueError("k, v must be [B, H_kv, N, d] with H_kv dividing q's H")
    elif k.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype or q.dtype not in _DTYPE:
        raise ValueError(f"unsupported or mixed dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    if o.shape != q.shape or o.dtype != out_dtype(q.dtype):
        raise ValueError("o must be [B, H, N, d] of the output dtype")
    if lse.shape != q.shape[:3] or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    if key_len is not None:
        if (not key_len.is_cuda or key_len.dtype != torch.int32 or key_len.shape != (q.shape[0],)
                or not key_len.is_contiguous()):
            raise ValueError("key_len must be a contiguous device int32 tensor of shape [B]")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool = False,
           key_len: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue fa_fwd on `stream` (default: torch's current stream)."""
    _check_inputs(q, k, v, o, lse, key_len)
    B, H, N, d = q.shape
    _lib._check(_lib.fa_fwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, scale,
                                causal, _ptr(key_len), _DTYPE[q.dtype], _stream(stream)))


def fa_fwd_fp8(q8, k8, v8, o, lse, scale: float, causal: bool = False,
               key_len: Optional[torch.Tensor] = None, q_descale: float = 1.0,
               k_descale: float = 1.0, v_descale: float = 1.0, stream=None) -> None:
    """Enqueue fa_fwd_fp8 (per-tensor descaled fp8 e4m3 inputs, bf16 O)."""
    if q8.dtype != torch.float8_e4m3fn:
        raise ValueError("fa_fwd_fp8 takes float8_e4m3fn inputs")
    _check_inputs(q8, k8, v8, o, lse, key_len)
    B, H, N, d = q8.shape
    _lib._check(_lib.fa_fwd_fp8_raw(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, H, N, d,
                                    scale, causal, _ptr(key_len), q_descale, k_descale, v_descale,
                                    _stream(stream)))


def fa_fwd_fp8_p8(q8, k8, v8, o, lse, scale: float, causal: bool = False,
                  key_len: Optional[torch.Tensor] = None, q_descale: float = 1.0,
                  k_descale: float = 1.0, v_descale: float = 1.0, stream=None) -> None:
    """Enqueue fa_fwd_fp8_p8 (as fa_fwd_fp8, with P rounded to e4m3 for P V)."""
    if q8.dtype != torch.float8_e4m3fn:
        raise ValueError("fa_fwd_fp8_p8 takes float8_e4m3fn inputs")
    _check_inputs(q8, k8, v8, o, lse, key_len)
    B, H, N, d = q8.shape
    _lib._check(_lib.fa_fwd_fp8_p8_raw(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, H, N,
                                       d, scale, causal, _ptr(key_len), q_descale, k_descale,
                                       v_descale, _stream(stream)))


def fa_fwd_gqa(q, k, v, o, lse, scale: float, causal: bool = False,
               key_len: Optional[torch.Tensor] = None, q_descale: float = 1.0,
               k_descale: float = 1.0, v_descale: float = 1.0, stream=None) -> None:
    """Enqueue fa_fwd_gqa: k, v of shape [B, H_kv, N, d], query head h using
    K/V head h // (H // H_kv); descales as fa_fwd_fp8, for every dtype."""
    _check_inputs(q, k, v, o, lse, key_len, grouped=True)
    B, H, N, d = q.shape
    _lib._check(_lib.fa_fwd_gqa_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                                    k.shape[1], N, d, scale, causal, _ptr(key_len),
                                    _DTYPE[q.dtype], q_descale, k_descale, v_descale,
                                    _stream(stream)))


def fa_fwd_window(q, k, v, o, lse, scale: float, causal: bool = False, window=(-1, -1),
                  key_len: Optional[torch.Tensor] = None, q_descale: float = 1.0,
                  k_descale: float = 1.0, v_descale: float = 1.0, stream=None) -> None:
    """Enqueue fa_fwd_window: the grouped forward with a (left, right) band."""
    _check_inputs(q, k, v, o, lse, key_len, grouped=True)
    B, H, N, d = q.shape
    _lib._check(_lib.fa_fwd_window_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                                       k.shape[1], N, d, scale, causal, window[0], window[1],
                                       _ptr(key_len), _DTYPE[q.dtype], q_descale, k_descale,
                                       v_descale, _stream(stream)))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen: int, scale: float,
                  causal: bool = False, stream=None) -> None:
    """Enqueue fa_fwd_varlen: a packed batch, q [H, total, d], k, v [H_kv, total, d],
    o like q, lse float32 [H, total], cu_seqlens device int32 [B + 1]."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse),
                    ("cu_seqlens", cu_seqlens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [H, total, d] and k, v one [H_kv, total, d] shape")
    H, total, d = q.shape
    if k.shape[1:] != (total, d) or H % k.shape[0] != 0:
        raise ValueError("k, v must be [H_kv, total, d] with H_kv dividing q's H")
    if k.dtype != q.dtype or v.dtype != q.dtype or q.dtype not in _DTYPE:
        raise ValueError(f"unsupported or mixed dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    if o.shape != q.shape or o.dtype != out_dtype(q.dtype):
        raise ValueError("o must be [H, total, d] of the output dtype")
    if lse.shape != (H, total) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [H, total]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 2:
        raise ValueError("cu_seqlens must be int32 [B + 1] with B >= 1")
    _lib._check(_lib.fa_fwd_varlen_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       _ptr(cu_seqlens), cu_seqlens.shape[0] - 1, H, k.shape[0],
                                       total, max_seqlen, d, scale, causal, _DTYPE[q.dtype],
                                       _stream(stream)))


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, *, scale: float, causal: bool = False,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(O, LSE) of a packed batch of sequences (see fa_fwd_varlen). O and LSE are
    allocated here; rows outside every sequence are left as allocated (zero)."""
    H, total, d = q.shape
    o = torch.zeros((H, total, d), dtype=out_dtype(q.dtype), device=q.device)
    lse = torch.zeros((H, total), dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen, scale, causal, stream=stream)
    return o, lse


def forward(q, k, v, scale: float, causal: bool = False, key_len=None,
            descale: Tuple[float, float, float] = (1.0, 1.0, 1.0),
            stream=None, window=None, p8: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Allocate O and LSE on q's device and run the forward; returns (O, LSE).
    k and v with fewer heads than q take the grouped entry point; p8 (fp8
    inputs only) takes fa_fwd_fp8_p8."""
    if p8 and (q.dtype != torch.float8_e4m3fn or window is not None or k.shape[1] != q.shape[1]):
        raise ValueError("p8 takes fp8 inputs with one K/V head per query head and no window")
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), dtype=out_dtype(q.dtype), device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if window is not None:
        fa_fwd_window(q, k, v, o, lse, scale, causal, window, key_len, *descale, stream=stream)
    elif k.dim() == 4 and k.shape[1] != H:
        fa_fwd_gqa(q, k, v, o, lse, scale, causal, key_len, *descale, stream=stream)
    elif p8:
        fa_fwd_fp8_p8(q, k, v, o, lse, scale, causal, key_len, *descale, stream=stream)
    elif q.dtype == torch.float8_e4m3fn:
        fa_fwd_fp8(q, k, v, o, lse, scale, causal, key_len, *descale, stream=stream)
    else:
        fa_fwd(q, k, v, o, lse, scale, causal, key_len, stream=stream)
    return o, lse


def fwd(q, k, v, *, scale: float, causal: bool = False, key_len=None,
        descale: Tuple[float, float, float] = (1.0, 1.0, 1.0),
        stream=None, window=None, p8: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """softmax(scale * Q K^T + mask) V and its row log-sum-exp, as (O, LSE).

    Keyword-only form of ``forward``. q, k, v: contiguous device tensors
    [B, H, N, d] of one dtype (float32, float16, bfloat16 or float8_e4m3fn),
    or k, v of [B, H_kv, N, d] with H_kv dividing H (grouped K/V heads);
    key_len: optional device int32 [B] of valid key counts. O has q's dtype
    (bfloat16 for fp8 inputs); LSE is float32 [B, H, N], natural log.
    p8: fp8 inputs with P rounded to e4m3 for the P V product.
    """
    return forward(q, k, v, scale, causal, key_len, descale, stream, window, p8)


def _check_decode(q, k, v, o, lse, key_len, tensors):
    for name, t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q [B, H, Nq, d] and k, v [B, H_kv, Nk, d] expected")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or H % k.shape[1] != 0:
        raise ValueError("k, v must be [B, H_kv, Nk, d] with H_kv dividing H")
    if k.dtype != q.dtype or v.dtype != q.dtype or q.dtype not in _DTYPE:
        raise ValueError(f"unsupported or mixed dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must be [B, H, Nq, d] of q's dtype")
    if lse.shape != q.shape[:3] or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, Nq]")
    if key_len is not None and (not key_len.is_cuda or key_len.dtype != torch.int32
                                or key_len.shape != (B,) or not key_len.is_contiguous()):
        raise ValueError("key_len must be a contiguous device int32 tensor of shape [B]")
    return B, H, Nq, d


def fa_fwd_decode(q, k, v, o, lse, workspace, scale: float, causal: bool = False,
                  key_len: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue fa_fwd_decode: q [B, H, Nq, d], k, v [B, H_kv, Nk, d] (16-bit),
    o like q, lse float32 [B, H, Nq], workspace a contiguous device tensor of at
    least decode_workspace_bytes(...) bytes."""
    B, H, Nq, d = _check_decode(q, k, v, o, lse, key_len,
                                (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse),
                                 ("workspace", workspace)))
    nbytes = workspace.numel() * workspace.element_size()
    _lib._check(_lib.fa_fwd_decode_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                                       k.shape[1], Nq, k.shape[2], d, scale, causal,
                                       _ptr(key_len), _DTYPE[q.dtype], _ptr(workspace), nbytes,
                                       _stream(stream)))


def fa_fwd_decode_noalloc(q, k, v, o, lse, scale: float, causal: bool = False,
                          key_len: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue fa_fwd_decode_noalloc: fa_fwd_decode with the partial results in
    the library's own device scratch (no workspace argument)."""
    B, H, Nq, d = _check_decode(q, k, v, o, lse, key_len,
                                (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)))
    _lib._check(_lib.fa_fwd_decode_noalloc_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B,
                                               H, k.shape[1], Nq, k.shape[2], d, scale, causal,
                                               _ptr(key_len), _DTYPE[q.dtype], _stream(stream)))


def decode(q, k, v, *, scale: float, causal: bool = False, key_len=None,
           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode against a key/value cache, allocating O, LSE and the workspace;
    returns (O, LSE). See fa_fwd_decode for the layouts and the mask."""
    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nbytes = decode_workspace_bytes(B, H, k.shape[1], Nq, k.shape[2], d)
    if nbytes == 0:
        raise ValueError("invalid decode sizes")
    ws = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    fa_fwd_decode(q, k, v, o, lse, ws, scale, causal, key_len, stream=stream)
    return o, lse


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, workspace, scale: float, causal: bool = False,
           key_len: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue fa_bwd: q, o, do, dq [B, H, N, d]; k, v, dk, dv [B, H_kv, N, d]
    (16-bit); lse float32 [B, H, N]; workspace of bwd_workspace_bytes(B, H, N)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("lse", lse),
                    ("dq", dq), ("dk", dk), ("dv", dv), ("workspace", workspace)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    B, H, N, d = q.shape
    if k.dim() != 4 or (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d) or H % k.shape[1]:
        raise ValueError("k, v must be [B, H_kv, N, d] with H_kv dividing H")
    for name, t, shape in (("v", v, k.shape), ("o", o, q.shape), ("do", do, q.shape),
                           ("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, k.shape)):
        if t.shape != shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must have shape {tuple(shape)} and q's dtype")
    if q.dtype not in (torch.bfloat16, torch.float16) or k.dtype != q.dtype:
        raise ValueError("the backward takes bfloat16 or float16 tensors")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    if key_len is not None and (not key_len.is_cuda or key_len.dtype != torch.int32
                                or key_len.shape != (B,) or not key_len.is_contiguous()):
        raise ValueError("key_len must be a contiguous device int32 tensor of shape [B]")
    nbytes = workspace.numel() * workspace.element_size()
    _lib._check(_lib.fa_bwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                _ptr(dk), _ptr(dv), B, H, k.shape[1], N, d, scale, causal,
                                _ptr(key_len), _DTYPE[q.dtype], _ptr(workspace), nbytes,
                                _stream(stream)))


def bwd(q, k, v, o, lse, do, *, scale: float, causal: bool = False, key_len=None,
        stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dQ, dK, dV) of the forward that returned (o, lse) for these
    inputs, given the upstream gradient do; allocates outputs and workspace."""
    B, H, N, d = q.shape
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    nbytes = bwd_workspace_bytes(B, H, N)
    ws = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale, causal, key_len, stream=stream)
    return dq, dk, dv
