// Internal interface between the host entry points (fa_api.cpp) and the
// kernel launchers (fa_fwd.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a kernel needs, passed by value as its only argument.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* key_len;  // NULL: every key valid
  int B, H, N;
  int kv_group;     // query heads per K/V head (H / H_kv; 1 without grouping)
  int n_qt;         // query tiles per head = ceil(N / rows per workgroup)
  float c;          // scale_eff * log2(e): multiplies raw scores before exp2
  float scale_eff;  // scale * q_descale * k_descale
  float o_scale;    // v_descale
  int win_left;     // sliding window: keys j >= i - win_left (negative: unbounded)
  int win_right;    // and j <= i + win_right (negative: unbounded)
  // Packed batch (NULL otherwise): B sequences concatenated along the rows of
  // every head's [total, D] block, sequence b at rows [cu_seqlens[b],
  // cu_seqlens[b+1]); N is then the longest length the grid covers.
  const int32_t* cu_seqlens;
  int total;
};

// Decode (few queries against a key/value cache), split over keys.
struct DecodeParams {
  const void* q;  // [B, H, Nq, D]
  const void* k;  // [B, H_kv, Nk, D]
  const void* v;
  void* o;        // [B, H, Nq, D]
  float* lse;     // [B, H, Nq]
  const int32_t* key_len;
  float* ws_o;    // workspace: [B*H*Nq][S][D] normalised partial O
  float* ws_lse;  // workspace: [B*H*Nq][S] partial LSE
  int B, H, H_kv, group, Nq, Nk;
  int R;            // rows per K/V head: group * Nq
  int n_rb;         // 32-row blocks per K/V head
  int S;            // key chunks
  int chunk_tiles;  // 32-key tiles per chunk
  int units;        // B * H_kv * n_rb * S waves of work
  float c, scale_eff, o_scale;
};

// Backward: gradients of the forward with respect to Q, K and V.
struct BwdParams {
  const void* q;     // [B, H, N, D]
  const void* k;     // [B, H_kv, N, D]
  const void* v;
  const void* o;     // forward output [B, H, N, D]
  const void* dout;  // upstream gradient dO [B, H, N, D]
  const float* lse;  // forward LSE [B, H, N]
  void* dq;          // [B, H, N, D]
  void* dk;          // [B, H_kv, N, D]
  void* dv;
  const int32_t* key_len;
  float* delta;      // workspace [B*H*N]: rowsum(dO * O)
  float* lse2;       // workspace [B*H*N]: LSE * log2(e), +inf for rows without keys
  int B, H, H_kv, group, N;
  int n_qt;          // 128-query tiles per head (dQ pass)
  int n_kt;          // 128-key tiles per K/V head (dK/dV pass)
  float c;           // scale * log2(e)
  float scale;
};

// FP8_P8: fp8 inputs with P rounded to e4m3 for the P V product (not a
// public dtype value; fa_fwd_fp8_p8 selects it).
enum class Kind { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3, FP8_P8 = 4 };

// Rows of Q owned by one workgroup for a problem's kind, d, N and mask; 0 if
// d is unsupported. Must agree with the kernel launch_forward picks.
int rows_per_block(Kind kind, int d, int N, bool causal, bool window = false);

// Enqueue the forward on `stream`. Arguments are already validated and
// p.n_qt filled in. Returns the launch's hipError_t.
hipError_t launch_forward(Kind kind, int d, bool causal, const Params& p, hipStream_t stream);

// Rows of Q per workgroup of the packed-batch forward (16-bit kinds, d 64 / 128)
// whose longest sequence has max_seqlen rows.
int varlen_rows_per_block(int max_seqlen, bool causal);

// Enqueue the packed-batch forward (p.cu_seqlens set, p.n_qt over p.N).
hipError_t launch_forward_varlen(Kind kind, int d, bool causal, const Params& p,
                                 hipStream_t stream);

// Key chunks S (and 32-key tiles per chunk) for `units_base` = B*H_kv*n_rb
// (K/V head, row block) pairs over Nk keys. Deterministic in its arguments:
// the workspace size and the launch both use it.
int decode_splits(int units_base, int Nk, int* chunk_tiles);

// Query rows (dQ pass) and keys (dK/dV pass) per backward workgroup.
int bwd_rows_per_block();

// Enqueue the backward's three passes on `stream` (16-bit kinds only).
hipError_t launch_backward(Kind kind, int d, bool causal, const BwdParams& p, hipStream_t stream);

// Enqueue the split pass and the merge on `stream` (16-bit kinds only).
hipError_t launch_decode(Kind kind, int d, bool causal, const DecodeParams& p, hipStream_t stream);

// Bytes of the device scratch behind fa_fwd_decode_noalloc.
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;

// The current device's address of that scratch (looked up once per device).
hipError_t decode_scratch(void** out);

}  // namespace fa
