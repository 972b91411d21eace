// Host entry points of libfa: argument validation and dispatch.
//
// Every check runs on the host before any HIP call, so a rejected call
// enqueues nothing and touches no buffer. The library allocates nothing and
// keeps no state besides a per-thread description of the last error.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* what) {
  snprintf(g_last_error, sizeof g_last_error, "%s", what);
  return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool positive_finite(float x) { return isfinite(x) && x > 0.0f; }

int forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
            int H_kv, int N, int d, float scale, int causal, const int32_t* key_len, int dtype,
            float qd, float kd, float vd, void* stream, int win_left = -1, int win_right = -1,
            bool p8 = false) {
  g_last_error[0] = '\0';
  if (!Q || !K || !V || !O || !LSE) return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (B < 1 || H < 1 || N < 1 || d < 1) return fail(FA_ERR_INVALID_ARG, "B, H, N and d must be >= 1");
  if (H_kv < 1 || H % H_kv != 0) return fail(FA_ERR_INVALID_ARG, "H_kv must be >= 1 and divide H");
  if (dtype < FA_DTYPE_FP32 || dtype > FA_DTYPE_FP8_E4M3)
    return fail(FA_ERR_INVALID_ARG, "dtype is not a fa_dtype value");
  if (!positive_finite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!positive_finite(qd) || !positive_finite(kd) || !positive_finite(vd))
    return fail(FA_ERR_INVALID_ARG, "descales must be finite and > 0");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(FA_ERR_INVALID_ARG, "Q, K, V and O must be 16-byte aligned");
  if (!aligned(LSE, 4) || (key_len && !aligned(key_len, 4)))
    return fail(FA_ERR_INVALID_ARG, "LSE and key_len must be 4-byte aligned");
  // B*H*N*d elements, and the same count in bytes for fp32, must fit in int64.
  const __int128 elems = (__int128)B * H * N * d;
  if (elems * 4 > (__int128)INT64_MAX) return fail(FA_ERR_INVALID_ARG, "B*H*N*d overflows");
  if (d != 64 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dimension must be 64, 128 or 256");
  if (d == 256 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16)
    return fail(FA_ERR_UNSUPPORTED, "head dimension 256 takes bfloat16 or float16 inputs");
  const bool window = win_left >= 0 || win_right >= 0;
  if (window && ((dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) || d == 256))
    return fail(FA_ERR_UNSUPPORTED, "sliding windows take bfloat16 or float16 inputs with d 64 or 128");
  // Kernels address one head's K and V through 32-bit byte offsets.
  const long long head_bytes = (long long)N * d * (dtype == FA_DTYPE_FP32 ? 4 : dtype == FA_DTYPE_FP8_E4M3 ? 1 : 2);
  if (head_bytes >= (1LL << 30)) return fail(FA_ERR_UNSUPPORTED, "one head's N x d tensor must be under 1 GiB");

  const fa::Kind kind = p8 ? fa::Kind::FP8_P8 : static_cast<fa::Kind>(dtype);
  const int rows = fa::rows_per_block(kind, d, N, causal != 0, window);
  fa::Params p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.key_len = key_len;
  p.B = B;
  p.H = H;
  p.kv_group = H / H_kv;
  p.N = N;
  p.n_qt = (N + rows - 1) / rows;
  const long long grid = (long long)B * H * p.n_qt;
  if (grid > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "B*H*ceil(N/rows) exceeds the grid limit");
  p.scale_eff = scale * qd * kd;
  if (!positive_finite(p.scale_eff)) return fail(FA_ERR_INVALID_ARG, "scale*q_descale*k_descale is not finite and > 0");
  p.c = (float)((double)p.scale_eff * 1.4426950408889634);
  p.o_scale = vd;
  p.win_left = win_left < 0 ? -1 : win_left;
  p.win_right = win_right < 0 ? -1 : win_right;
  p.cu_seqlens = nullptr;
  p.total = 0;

  const hipError_t e = fa::launch_forward(kind, d, causal != 0, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    snprintf(g_last_error, sizeof g_last_error, "kernel launch failed: %s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

int varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
           const int32_t* cu_seqlens, int B, int H, int H_kv, int total, int max_seqlen, int d,
           float scale, int causal, int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (!Q || !K || !V || !O || !LSE || !cu_seqlens)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer or cu_seqlens is NULL");
  if (B < 1 || H < 1 || total < 1 || max_seqlen < 1 || d < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H, total, max_seqlen and d must be >= 1");
  if (H_kv < 1 || H % H_kv != 0) return fail(FA_ERR_INVALID_ARG, "H_kv must be >= 1 and divide H");
  if (dtype < FA_DTYPE_FP32 || dtype > FA_DTYPE_FP8_E4M3)
    return fail(FA_ERR_INVALID_ARG, "dtype is not a fa_dtype value");
  if (!positive_finite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(FA_ERR_INVALID_ARG, "Q, K, V and O must be 16-byte aligned");
  if (!aligned(LSE, 4) || !aligned(cu_seqlens, 4))
    return fail(FA_ERR_INVALID_ARG, "LSE and cu_seqlens must be 4-byte aligned");
  if ((__int128)H * total * d * 4 > (__int128)INT64_MAX)
    return fail(FA_ERR_INVALID_ARG, "H*total*d overflows");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16)
    return fail(FA_ERR_UNSUPPORTED, "packed batches take bfloat16 or float16 inputs");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
  // No sequence is longer than the packed rows themselves.
  const int n_max = max_seqlen < total ? max_seqlen : total;
  if ((long long)n_max * d * 2 >= (1LL << 30))
    return fail(FA_ERR_UNSUPPORTED, "one sequence's rows x d must be under 1 GiB");
  const int rows = fa::varlen_rows_per_block(n_max, causal != 0);
  fa::Params p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.key_len = nullptr;
  p.B = B;
  p.H = H;
  p.kv_group = H / H_kv;
  p.N = n_max;
  p.n_qt = (n_max + rows - 1) / rows;
  if ((long long)B * H * p.n_qt > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARG, "B*H*ceil(max_seqlen/rows) exceeds the grid limit");
  p.scale_eff = scale;
  p.c = (float)((double)scale * 1.4426950408889634);
  p.o_scale = 1.0f;
  p.win_left = p.win_right = -1;
  p.cu_seqlens = cu_seqlens;
  p.total = total;
  const hipError_t e =
      fa::launch_forward_varlen(static_cast<fa::Kind>(dtype), d, causal != 0, p,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    snprintf(g_last_error, sizeof g_last_error, "kernel launch failed: %s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// Rows per K/V head, 32-row blocks, key chunks and tiles per chunk of a
// decode call, and the workspace bytes it needs; false if the sizes are out
// of range.
struct DecodeShape {
  int R, n_rb, S, chunk_tiles;
  long long units, ws_bytes;
};

bool decode_shape(int B, int H, int H_kv, int Nq, int Nk, int d, DecodeShape& sh) {
  if (B < 1 || H < 1 || H_kv < 1 || Nq < 1 || Nk < 1 || d < 1 || H % H_kv != 0) return false;
  const long long R = (long long)(H / H_kv) * Nq;
  if (R > 0x7fffffffLL - 31) return false;
  sh.R = (int)R;
  sh.n_rb = (int)((R + 31) / 32);
  const long long base = (long long)B * H_kv * sh.n_rb;
  if (base > 0x7fffffffLL) return false;
  sh.S = fa::decode_splits((int)base, Nk, &sh.chunk_tiles);
  sh.units = base * sh.S;
  const __int128 rows = (__int128)B * H * Nq;
  const __int128 bytes = rows * sh.S * (d + 1) * 4 + 256;
  if (sh.units > 0x7fffffffLL || rows > 0x7fffffff || bytes > (__int128)INT64_MAX) return false;
  sh.ws_bytes = (long long)bytes;
  return true;
}

// own_scratch: the partial results go to the library's device scratch
// (fa_fwd_decode_noalloc) instead of the caller's workspace, which is then
// ignored.
int decode(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
           int H_kv, int Nq, int Nk, int d, float scale, int causal, const int32_t* key_len,
           int dtype, void* workspace, size_t workspace_bytes, void* stream,
           bool own_scratch = false) {
  g_last_error[0] = '\0';
  if (!Q || !K || !V || !O || !LSE) return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!own_scratch && !workspace) return fail(FA_ERR_INVALID_ARG, "workspace is NULL");
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H, Nq, Nk and d must be >= 1");
  if (H_kv < 1 || H % H_kv != 0) return fail(FA_ERR_INVALID_ARG, "H_kv must be >= 1 and divide H");
  if (dtype < FA_DTYPE_FP32 || dtype > FA_DTYPE_FP8_E4M3)
    return fail(FA_ERR_INVALID_ARG, "dtype is not a fa_dtype value");
  if (!positive_finite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      (!own_scratch && !aligned(workspace, 16)))
    return fail(FA_ERR_INVALID_ARG, "Q, K, V, O and the workspace must be 16-byte aligned");
  if (!aligned(LSE, 4) || (key_len && !aligned(key_len, 4)))
    return fail(FA_ERR_INVALID_ARG, "LSE and key_len must be 4-byte aligned");
  if ((__int128)B * H * Nq * d * 4 > (__int128)INT64_MAX ||
      (__int128)B * H_kv * Nk * d * 4 > (__int128)INT64_MAX)
    return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  DecodeShape sh;
  if (!decode_shape(B, H, H_kv, Nq, Nk, d, sh)) return fail(FA_ERR_INVALID_ARG, "sizes out of range");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16)
    return fail(FA_ERR_UNSUPPORTED, "decode takes bfloat16 or float16 inputs");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
  if ((long long)Nk * d * 2 >= (1LL << 30))
    return fail(FA_ERR_UNSUPPORTED, "one head's Nk x d tensor must be under 1 GiB");
  if (own_scratch) {
    if (sh.ws_bytes > (long long)FA_DECODE_NOALLOC_MAX_BYTES)
      return fail(FA_ERR_UNSUPPORTED,
                  "decode partial results exceed the library's 8 MiB device scratch "
                  "(fa_decode_workspace_bytes() > FA_DECODE_NOALLOC_MAX_BYTES); use fa_fwd_decode");
    const hipError_t e = fa::decode_scratch(&workspace);
    if (e != hipSuccess) {
      snprintf(g_last_error, sizeof g_last_error, "device scratch lookup failed: %s",
               hipGetErrorString(e));
      return FA_ERR_HIP;
    }
  } else if ((long long)workspace_bytes < sh.ws_bytes) {
    return fail(FA_ERR_INVALID_ARG, "workspace smaller than fa_decode_workspace_bytes()");
  }

  fa::DecodeParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.key_len = key_len;
  const long long rows = (long long)B * H * Nq;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_lse = p.ws_o + rows * sh.S * d;
  p.B = B;
  p.H = H;
  p.H_kv = H_kv;
  p.group = H / H_kv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.R = sh.R;
  p.n_rb = sh.n_rb;
  p.S = sh.S;
  p.chunk_tiles = sh.chunk_tiles;
  p.units = (int)sh.units;
  p.scale_eff = scale;
  p.c = (float)((double)scale * 1.4426950408889634);
  p.o_scale = 1.0f;
  const hipError_t e = fa::launch_decode(static_cast<fa::Kind>(dtype), d, causal != 0, p,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    snprintf(g_last_error, sizeof g_last_error, "kernel launch failed: %s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

long long bwd_workspace(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  const __int128 rows = (__int128)B * H * N;
  if (rows * 8 + 256 > (__int128)INT64_MAX) return 0;
  return (long long)(rows * 8 + 256);
}

int backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int H_kv, int N, int d,
             float scale, int causal, const int32_t* key_len, int dtype, void* workspace,
             size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV)
    return fail(FA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!workspace) return fail(FA_ERR_INVALID_ARG, "workspace is NULL");
  if (B < 1 || H < 1 || N < 1 || d < 1) return fail(FA_ERR_INVALID_ARG, "B, H, N and d must be >= 1");
  if (H_kv < 1 || H % H_kv != 0) return fail(FA_ERR_INVALID_ARG, "H_kv must be >= 1 and divide H");
  if (dtype < FA_DTYPE_FP32 || dtype > FA_DTYPE_FP8_E4M3)
    return fail(FA_ERR_INVALID_ARG, "dtype is not a fa_dtype value");
  if (!positive_finite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  const void* al16[] = {Q, K, V, O, dO, dQ, dK, dV, workspace};
  for (const void* x : al16)
    if (!aligned(x, 16)) return fail(FA_ERR_INVALID_ARG, "tensors and the workspace must be 16-byte aligned");
  if (!aligned(LSE, 4) || (key_len && !aligned(key_len, 4)))
    return fail(FA_ERR_INVALID_ARG, "LSE and key_len must be 4-byte aligned");
  if ((__int128)B * H * N * d * 4 > (__int128)INT64_MAX) return fail(FA_ERR_INVALID_ARG, "B*H*N*d overflows");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16)
    return fail(FA_ERR_UNSUPPORTED, "the backward takes bfloat16 or float16 tensors");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
  if ((long long)N * d * 2 >= (1LL << 30)) return fail(FA_ERR_UNSUPPORTED, "one head's N x d tensor must be under 1 GiB");
  const long long need = bwd_workspace(B, H, N);
  if (need == 0 || (long long)workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARG, "workspace smaller than fa_bwd_workspace_bytes()");
  const int bwd_rows = fa::bwd_rows_per_block();
  const long long tiles = (N + bwd_rows - 1) / bwd_rows;
  if ((long long)B * H * tiles > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "grid too large");

  fa::BwdParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.dout = dO;
  p.lse = LSE;
  p.dq = dQ;
  p.dk = dK;
  p.dv = dV;
  p.key_len = key_len;
  p.delta = static_cast<float*>(workspace);
  p.lse2 = p.delta + (long long)B * H * N;
  p.B = B;
  p.H = H;
  p.H_kv = H_kv;
  p.group = H / H_kv;
  p.N = N;
  p.n_qt = (int)tiles;
  p.n_kt = (int)tiles;
  p.scale = scale;
  p.c = (float)((double)scale * 1.4426950408889634);
  const hipError_t e = fa::launch_backward(static_cast<fa::Kind>(dtype), d, causal != 0, p,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    snprintf(g_last_error, sizeof g_last_error, "kernel launch failed: %s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N,
           int d, float scale, int causal, const int32_t* key_len, int dtype, void* stream) {
  return forward(Q, K, V, O, LSE, B, H, H, N, d, scale, causal, key_len, dtype, 1.0f, 1.0f, 1.0f,
                 stream);
}

int fa_fwd_fp8(const void* Q8, const void* K8, const void* V8, void* O_bf16, float* LSE, int B,
               int H, int N, int d, float scale, int causal, const int32_t* key_len,
               float q_descale, float k_descale, float v_descale, void* stream) {
  return forward(Q8, K8, V8, O_bf16, LSE, B, H, H, N, d, scale, causal, key_len, FA_DTYPE_FP8_E4M3,
                 q_descale, k_descale, v_descale, stream);
}

int fa_fwd_fp8_p8(const void* Q8, const void* K8, const void* V8, void* O_bf16, float* LSE, int B,
                  int H, int N, int d, float scale, int causal, const int32_t* key_len,
                  float q_descale, float k_descale, float v_descale, void* stream) {
  return forward(Q8, K8, V8, O_bf16, LSE, B, H, H, N, d, scale, causal, key_len, FA_DTYPE_FP8_E4M3,
                 q_descale, k_descale, v_descale, stream, -1, -1, true);
}

int fa_fwd_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
               int H_kv, int N, int d, float scale, int causal, const int32_t* key_len, int dtype,
               float q_descale, float k_descale, float v_descale, void* stream) {
  return forward(Q, K, V, O, LSE, B, H, H_kv, N, d, scale, causal, key_len, dtype, q_descale,
                 k_descale, v_descale, stream);
}

size_t fa_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d) {
  DecodeShape sh;
  if (!decode_shape(B, H, H_kv, Nq, Nk, d, sh)) return 0;
  return (size_t)sh.ws_bytes;
}

int fa_fwd_decode(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                  int H_kv, int Nq, int Nk, int d, float scale, int causal,
                  const int32_t* key_len, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return decode(Q, K, V, O, LSE, B, H, H_kv, Nq, Nk, d, scale, causal, key_len, dtype, workspace,
                workspace_bytes, stream);
}

int fa_fwd_decode_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                          int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                          const int32_t* key_len, int dtype, void* stream) {
  static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_MAX_BYTES, "scratch size");
  return decode(Q, K, V, O, LSE, B, H, H_kv, Nq, Nk, d, scale, causal, key_len, dtype, nullptr, 0,
                stream, true);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) { return (size_t)bwd_workspace(B, H, N); }

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int H_kv, int N, int d,
           float scale, int causal, const int32_t* key_len, int dtype, void* workspace,
           size_t workspace_bytes, void* stream) {
  return backward(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, H_kv, N, d, scale, causal, key_len, dtype,
                  workspace, workspace_bytes, stream);
}

int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                  int H_kv, int N, int d, float scale, int causal, int window_left,
                  int window_right, const int32_t* key_len, int dtype, float q_descale,
                  float k_descale, float v_descale, void* stream) {
  return forward(Q, K, V, O, LSE, B, H, H_kv, N, d, scale, causal, key_len, dtype, q_descale,
                 k_descale, v_descale, stream, window_left, window_right);
}

int fa_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  const int32_t* cu_seqlens, int B, int H, int H_kv, int total, int max_seqlen,
                  int d, float scale, int causal, int dtype, void* stream) {
  return varlen(Q, K, V, O, LSE, cu_seqlens, B, H, H_kv, total, max_seqlen, d, scale, causal,
                dtype, stream);
}

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_last_error(void) { return g_last_error; }

}  // extern "C"
