"""ctypes binding of libfa.so: argument marshalling only.

Every step of the attention forward runs inside libfa's HIP kernels; torch is
used here only to own device memory and to name the stream. If the library is
not built, every call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_DTYPE_FP32, FA_DTYPE_FP16, FA_DTYPE_BF16, FA_DTYPE_FP8_E4M3 = 0, 1, 2, 3
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, -1, -2, -3

EXPORTED = ("fa_fwd", "fa_fwd_fp8", "fa_fwd_fp8_p8", "fa_fwd_gqa", "fa_fwd_decode", "fa_decode_workspace_bytes",
            "fa_fwd_decode_noalloc",
            "fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd_window", "fa_fwd_varlen", "fa_status_str",
            "fa_abi_version", "fa_last_error")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{status_name(status)}: {detail}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is missing; build it with `python -m exact_io_aware_56_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, f, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_fp8_p8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, f, f, vp]
    lib.fa_fwd_fp8_p8.restype = i
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, f, f, f, vp]
    lib.fa_fwd_gqa.restype = i
    sz = ctypes.c_size_t
    lib.fa_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, vp, sz, vp]
    lib.fa_fwd_decode.restype = i
    lib.fa_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, vp]
    lib.fa_fwd_decode_noalloc.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, i, f, f, f, vp]
    lib.fa_fwd_window.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_status_str.argtypes = [i]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return load().fa_status_str(int(status)).decode()


def abi_version() -> int:
    return load().fa_abi_version()


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, load().fa_last_error().decode())


def fa_fwd_raw(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, dtype, stream) -> int:
    """The C call with plain integers as pointers; returns the fa_status code."""
    return load().fa_fwd(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), key_len,
                         int(dtype), stream)


def fa_fwd_fp8_raw(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, qd, kd, vd,
                   stream) -> int:
    return load().fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), key_len,
                             float(qd), float(kd), float(vd), stream)


def fa_fwd_fp8_p8_raw(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, qd, kd, vd,
                      stream) -> int:
    return load().fa_fwd_fp8_p8(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), key_len,
                                float(qd), float(kd), float(vd), stream)


def fa_fwd_gqa_raw(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, key_len, dtype, qd, kd, vd,
                   stream) -> int:
    return load().fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, float(scale), int(causal),
                             key_len, int(dtype), float(qd), float(kd), float(vd), stream)


def decode_workspace_bytes(B, H, H_kv, Nq, Nk, d) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d))


def fa_fwd_decode_raw(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, key_len, dtype,
                      workspace, workspace_bytes, stream) -> int:
    return load().fa_fwd_decode(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, float(scale),
                                int(causal), key_len, int(dtype), workspace,
                                int(workspace_bytes), stream)


def fa_fwd_decode_noalloc_raw(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, key_len,
                              dtype, stream) -> int:
    return load().fa_fwd_decode_noalloc(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, float(scale),
                                        int(causal), key_len, int(dtype), stream)


def bwd_workspace_bytes(B, H, N) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, N))


def fa_bwd_raw(q, k, v, o, do, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, key_len, dtype,
               workspace, workspace_bytes, stream) -> int:
    return load().fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, H_kv, N, d, float(scale),
                         int(causal), key_len, int(dtype), workspace, int(workspace_bytes), stream)


def fa_fwd_window_raw(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, wl, wr, key_len, dtype,
                      qd, kd, vd, stream) -> int:
    return load().fa_fwd_window(q, k, v, o, lse, B, H, H_kv, N, d, float(scale), int(causal),
                                int(wl), int(wr), key_len, int(dtype), float(qd), float(kd),
                                float(vd), stream)


def fa_fwd_varlen_raw(q, k, v, o, lse, cu_seqlens, B, H, H_kv, total, max_seqlen, d, scale,
                      causal, dtype, stream) -> int:
    return load().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, int(B), int(H), int(H_kv),
                                int(total), int(max_seqlen), int(d), float(scale), int(causal),
                                int(dtype), stream)
