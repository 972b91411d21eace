// Fused exact attention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup owns a tile of query rows of one (batch, head) and streams the
// key/value tiles of that head through double-buffered LDS, keeping for every
// query row a running maximum and a running sum of exponentials that are
// corrected as each key tile arrives (FlashAttention (ES), "Tiling y
// procesamiento por bloques" and "Cálculo de Softmax en línea"). QK^T, the
// mask, the softmax and the product with V happen in this one kernel and only
// O and the per-row log-sum-exp are written ("Fusión de operaciones en un
// único kernel"). No N x N buffer exists.
//
// Matrix-core mapping (wave64, v_mfma_f32_32x32x16_{bf16,f16},
// v_mfma_scale_f32_32x32x64_f8f6f4 and v_mfma_f32_32x32x2_f32):
//
//   Each wave owns 32 query rows and computes the transposed products
//       S^T = K Q^T      (M = keys, N = queries, K = head dim)
//       O^T += V^T P^T   (M = head dim, N = queries, K = keys)
//   In the 32x32 accumulator layout lane l holds column l%32 and rows
//   8*(i/4) + 4*(l/32) + i%4 of its 16 values, so with the queries as the
//   column index every lane owns ONE query row: its 16 scores per 32-key
//   block are that row's, the row maximum needs one exchange with lane
//   l^32 (v_permlane32_swap), the rescale of O is a per-lane scalar, and
//   the score accumulators feed P^T to the second product without leaving
//   registers. The keys' order inside a 16-key reduction step is permuted by
//   that layout; the V^T operand is read from LDS in the same permuted order
//   with the gfx950 transposing LDS read (ds_read_b64_tr_b16), so no
//   transposed copy of V is ever stored.
//
// Scores stay raw (unscaled) in registers; scale*log2(e) is folded into one
// FMA ahead of v_exp_f32 (exp2), so exp(scale*s - m) = exp2(c*s - c*m).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// Build-time tuning knobs (the defaults are the measured best on MI355X).
#ifndef FA_K_SKEW
#define FA_K_SKEW 8  // extra 16-bit elements per K row in LDS
#endif
#ifndef FA_V_SKEW
#define FA_V_SKEW 32  // extra 16-bit elements per V row in LDS
#endif
#ifndef FA_RESCALE_LOG2
#define FA_RESCALE_LOG2 8.0f
#endif
#ifndef FA_WAVES
#define FA_WAVES 4  // waves (of 32 query rows each) per workgroup
#endif
#ifndef FA_KEY_TILE
#define FA_KEY_TILE 64  // keys per LDS tile for the 16-bit and fp8 kernels
#endif
#ifndef FA_WAVES_PER_EU
#define FA_WAVES_PER_EU 2
#endif
#ifndef FA_PIPE_MIN_N
#define FA_PIPE_MIN_N 4096  // causal 16-bit sequences from this length take the pipelined kernel
#endif
#ifndef FA_DMA_WAVES
#define FA_DMA_WAVES 4  // waves per workgroup of the direct-to-LDS kernel
#endif
#ifndef FA_WIDE_WAVES
#define FA_WIDE_WAVES 8  // waves per workgroup of the pipelined kernel
#endif
#ifndef FA_PIPE_LOOKAHEAD
#define FA_PIPE_LOOKAHEAD 0  // pipelined kernels: LDS operand reads issued this many MFMAs ahead
                             // (0: two for head dim 128 over whole V rows, else one)
#endif
#ifndef FA_PIPE_IGLP
#define FA_PIPE_IGLP 3  // pipelined kernel: the compiler's MFMA/exp interleave for each half-step (-1: none)
#endif
#ifndef FA_LOOKAHEAD
#define FA_LOOKAHEAD 2  // LDS operand reads issued this many MFMAs ahead
#endif

// ---------------------------------------------------------------------------
// Small wave-level helpers
// ---------------------------------------------------------------------------

// max / sum of x over lanes l and l^32 (the two halves hold the same query row)
__device__ __forceinline__ float max_halves(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Scheduling fence that only vector ALU, scalar, global-memory and
// transcendental instructions may cross: LDS operand reads and matrix products
// keep their program order, so a read issued ahead of the product before the
// one that takes it stays there (the scheduler otherwise sinks each read onto
// its product and every product waits out a whole LDS latency).
__device__ __forceinline__ void operand_fence() { __builtin_amdgcn_sched_barrier(0x2 | 0x4 | 0x10 | 0x400); }

// Returns x unchanged, but through an asm statement the optimizer cannot look
// into or move. Used inside the rarely taken O-rescale branches: without it
// the compiler hoists the (speculatable) multiplies of O above the branch and
// executes them on every tile.
__device__ __forceinline__ float pinned(float x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}
// The lane index computed by two vector instructions the compiler can neither
// hoist nor merge: lane-derived values built from it are recomputed per work
// item instead of living across the whole kernel (where they are spilled).
__device__ __forceinline__ int fresh_lane() {
  int x;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}
__device__ __forceinline__ int pinned_int(int x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Raw buffer resource (gfx9 descriptor word 3) over `bytes` bytes at `base`.
// Loads at offsets >= bytes return zeros without touching memory, which is how
// ragged tails and padded keys are zero-filled with no branches.
// Both arguments must be wave-uniform; readfirstlane states that to the
// compiler so the descriptor lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// Resource over key rows [j*BC, j*BC + BC) of one head, cut at row `limit`.
// A tile wholly past the limit gets an empty range (and the head's base).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* head, int j, int BC,
                                                            int limit, int row_bytes) {
  const int rows = max(0, min(BC, limit - j * BC));
  const char* base = (const char*)head + (rows > 0 ? (size_t)j * BC * row_bytes : 0);
  return buffer_rsrc(base, rows * row_bytes);
}

__device__ __forceinline__ i32x4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Workgroup -> (batch*head, query tile). Workgroups are handed to the XCDs
// round-robin by id, so id % 8 names the XCD. When B*H is a multiple of 8,
// each XCD owns B*H/8 whole heads, so the workgroups that run together on one
// XCD read those heads' K/V through that XCD's L2, and within an XCD the
// workgroups are issued query-tile-major over its heads: for causal attention
// the last (longest) query tiles of every head first, the shortest last, so
// that the short ones fill the tail of the launch whatever the run-time
// spread of the long ones. Otherwise tiles are issued head by head, causal
// ones longest first, in contiguous runs per XCD when the grid divides.
__device__ __forceinline__ void map_block(int n_qt, bool causal, int& bh, int& qt) {
  const int bid = blockIdx.x, total = gridDim.x;
  int r;
  if (total % (kXcds * n_qt) == 0) {
    const int hx = total / (kXcds * n_qt);  // heads per XCD
    const int i = bid / kXcds;              // issue rank within the XCD
    bh = (bid % kXcds) * hx + i % hx;
    r = i / hx;
  } else {
    int logical = bid;  // contiguous runs of tiles per XCD when possible
    if (total % kXcds == 0) logical = (bid % kXcds) * (total / kXcds) + bid / kXcds;
    bh = logical / n_qt;
    r = logical - bh * n_qt;
  }
  qt = causal ? (n_qt - 1 - r) : r;
}

struct RowRange {
  int bh, kv_bh, b, q_wg0, qw0, qrow, kl, nt, wnt, wfull;
};

// Which key tiles the workgroup streams (nt) and which of them this wave
// multiplies (wnt): keys at or beyond key_len, and for causal keys beyond the
// last row of the workgroup / wave, can only be masked, so those tiles are
// skipped altogether.
template <int BR, int BC, bool CAUSAL, int WR = 32>
__device__ __forceinline__ RowRange row_range_at(const Params& p, int bh, int qt, int wave,
                                                 int l32) {
  RowRange r;
  r.bh = bh;
  // Query heads [g * kv_group, (g + 1) * kv_group) of a batch entry share K/V
  // head g, so the K/V head of query head bh = b * H + h is bh / kv_group.
  r.kv_bh = p.kv_group == 1 ? bh : bh / p.kv_group;
  r.b = r.bh / p.H;
  const int N = p.N;
  int kl = N;
  if (p.key_len != nullptr) {
    const int x = p.key_len[r.b];
    kl = x < 0 ? 0 : (x > N ? N : x);
  }
  // Loaded from memory, so the compiler cannot see it is the same in every
  // lane; without this every branch on the tile range is divergent (both
  // sides executed under an exec mask) instead of a scalar branch.
  r.kl = kl = __builtin_amdgcn_readfirstlane(kl);
  r.q_wg0 = qt * BR;
  r.qw0 = r.q_wg0 + wave * WR;
  r.qrow = r.qw0 + l32;
  int kv_end = kl;
  if (CAUSAL) kv_end = min(kv_end, min(N, r.q_wg0 + BR));
  r.nt = (kv_end + BC - 1) / BC;
  int w_end = kv_end;
  if (CAUSAL) w_end = min(w_end, r.qw0 + WR);
  if (r.qw0 >= N) w_end = 0;
  r.wnt = (w_end + BC - 1) / BC;
  // Tiles [0, wfull) need no mask for any row of this wave: every key is below
  // key_len and (causal) at or below the wave's first row.
  int full = kl / BC;
  if (CAUSAL) full = min(full, (r.qw0 + 1) / BC);
  r.wfull = min(full, r.wnt);
  return r;
}

template <int BR, int BC, bool CAUSAL, int WR = 32>
__device__ __forceinline__ RowRange row_range(const Params& p, int wave, int l32) {
  int bh, qt;
  map_block(p.n_qt, CAUSAL, bh, qt);
  return row_range_at<BR, BC, CAUSAL, WR>(p, bh, qt, wave, l32);
}

// Packed batch: workgroup -> (sequence * H + head, unit), heads fastest.
// Workgroups go to the XCDs round-robin by id, so consecutive ids (the heads
// of one unit of one sequence) spread every sequence evenly over the XCDs,
// whatever the mix of lengths; contiguous runs of whole heads per XCD would
// leave the XCDs that own the longest sequences with most of the work.
__device__ __forceinline__ void varlen_item(int H, int units, int& bh, int& u) {
  const int bid = blockIdx.x;
  const int h = bid % H, r = bid / H;
  u = r % units;
  bh = (r / units) * H + h;
}

// Packed batch: narrows p to the sequence and head of work item bh = b * H + h,
// so that the kernel then runs as on one head of one batch entry: the Q, K, V,
// O and LSE pointers move to the sequence's first row of the head's block and
// N becomes the sequence's length. Bounds are clamped to [0, total] (an end
// before its start gives an empty sequence) and the length is cut to the grid's
// p.N. Returns false, the same in every lane, when query row q0 lies past the
// sequence's end.
template <class TIn, class TOut, int D>
__device__ __forceinline__ bool enter_segment(Params& p, int bh, int q0) {
  const int b = bh / p.H, h = bh - b * p.H, T = p.total;
  int s0 = min(max(p.cu_seqlens[b], 0), T);
  const int s1 = min(max(p.cu_seqlens[b + 1], s0), T);
  const int n = __builtin_amdgcn_readfirstlane(min(s1 - s0, p.N));
  s0 = __builtin_amdgcn_readfirstlane(s0);
  if (q0 >= n) return false;
  const size_t qrow = (size_t)h * T + s0, kvrow = (size_t)(h / p.kv_group) * T + s0;
  p.q = (const TIn*)p.q + qrow * D;
  p.k = (const TIn*)p.k + kvrow * D;
  p.v = (const TIn*)p.v + kvrow * D;
  p.o = (TOut*)p.o + qrow * D;
  p.lse += qrow;
  p.N = n;
  p.key_len = nullptr;
  p.B = p.H = p.kv_group = 1;
  return true;
}

// ---------------------------------------------------------------------------
// 16-bit element policies
// ---------------------------------------------------------------------------
struct Bf16 {
  using T = __bf16;
  using v8 = bf16x8;
  using v4 = bf16x4;
  // Largest P the pipelined kernel lets a stale reference maximum produce:
  // bf16 has fp32's exponent range, and O and l accumulate in fp32.
  static constexpr float kPBound = 0x1p64f;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4 tr4(const T* lds) {
    return __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)lds));
  }
  static __device__ __forceinline__ T cvt(float x) { return (T)x; }
  // acc + a + b (already rounded values), fp32 accumulation
  static __device__ __forceinline__ float sum2(T a, T b, float acc) {
    const bf16x2 one = {(T)1.0f, (T)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a, b}, one, acc, false);
  }
  // acc + sum of the 8 (already rounded) values, fp32 accumulation
  static __device__ __forceinline__ float sum8(v8 x, float acc) {
    const bf16x2 one = {(T)1.0f, (T)1.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[2 * k], x[2 * k + 1]}, one, acc, false);
    return acc;
  }
};

struct F16 {
  using T = _Float16;
  using v8 = f16x8;
  using v4 = f16x4;
  static constexpr float kPBound = 0x1p15f;  // below fp16's largest finite value
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4 tr4(const T* lds) {
    return __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)lds));
  }
  static __device__ __forceinline__ T cvt(float x) { return (T)x; }
  static __device__ __forceinline__ float sum2(T a, T b, float acc) {
    const f16x2 one = {(T)1.0f, (T)1.0f};
    return __builtin_amdgcn_fdot2(f16x2{a, b}, one, acc, false);
  }
  static __device__ __forceinline__ float sum8(v8 x, float acc) {
    const f16x2 one = {(T)1.0f, (T)1.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc = __builtin_amdgcn_fdot2(f16x2{x[2 * k], x[2 * k + 1]}, one, acc, false);
    return acc;
  }
};

// Shared by the 16-bit and fp8 kernels: online-softmax update of one key
// tile for this lane's query row, producing P^T operands in 16-bit.
//   s[SB]  raw scores (masked entries already -inf)
//   m, l   reference maximum (raw units) and this lane's partial running sum
//   o[DB]  output accumulators, rescaled here when the reference moves
//   thr    kRescaleLog2 / c: how far (raw units) a row's maximum may exceed
//          its reference before the reference is moved
//
// The reference maximum only moves when a row's tile maximum exceeds it by
// more than 2^kRescaleLog2 in the exponent; otherwise P = exp2(c*s - c*m) may
// reach 2^kRescaleLog2, which bf16/fp16 and the fp32 sums hold without loss.
// O and l are always scaled by the same factors, so O / l is unchanged: the
// result is the same exact softmax, the threshold only saves the O rescale
// (DB*16 multiplies) on most tiles.
constexpr float kRescaleLog2 = FA_RESCALE_LOG2;

template <class E, int SB, int DB>
__device__ __forceinline__ void online_softmax(f32x16 (&s)[SB], float c, float thr, float& m,
                                               float& l, f32x16 (&o)[DB],
                                               typename E::v8 (&pf)[SB * 2]) {
  float mx = s[0][0];
#pragma unroll
  for (int sb = 0; sb < SB; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
  mx = max_halves(mx);
  const bool move = mx > m + thr;  // true on the first live tile (m = -inf)
  if (__builtin_amdgcn_ballot_w64(move) != 0) {
    const float alpha = pinned(move ? fast_exp2((m - mx) * c) : 1.0f);  // exp2(-inf) = 0
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    m = move ? mx : m;
  }
  const float base = (m == -INFINITY) ? 0.0f : -m * c;
  // The running sum adds the same rounded P values that multiply V, so the
  // weights applied to V's rows sum to one up to fp32 accumulation.
  float rs = 0.0f;
#pragma unroll
  for (int ps = 0; ps < SB * 2; ++ps) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pf[ps][e] = E::cvt(fast_exp2(fmaf(s[ps >> 1][(ps & 1) * 8 + e], c, base)));
    rs = E::sum8(pf[ps], rs);
  }
  l += rs;
}

// The same update with a lazy reference maximum (no row maximum per tile):
// P = exp2(c*s + base), base = -m*c, is formed against the row's current
// reference m, and the row sum of P that l needs anyway tells whether a score
// got too far above m. If a lane's partial sum exceeds E::kPBound, or is
// inf / NaN (the first live tile, while m = -inf and base = +inf), a rarely
// taken branch takes the tile's true row maximum, moves m there, rescales O
// and l and recomputes P. Otherwise every P is at most E::kPBound, which the
// 16-bit P and the fp32 accumulators hold without loss; O / l is the same
// exact softmax for any reference.
template <class E, int SB, int DB>
__device__ __forceinline__ void lazy_softmax(f32x16 (&s)[SB], float c, float& m, float& base,
                                             float& l, f32x16 (&o)[DB],
                                             typename E::v8 (&pf)[SB * 2]) {
  float rs = 0.0f;
#pragma unroll
  for (int ps = 0; ps < SB * 2; ++ps) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pf[ps][e] = E::cvt(fast_exp2(fmaf(s[ps >> 1][(ps & 1) * 8 + e], c, base)));
    rs = E::sum8(pf[ps], rs);
  }
  if (__builtin_amdgcn_ballot_w64(!(rs <= E::kPBound)) != 0) {
    float x = s[0][0];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i) x = fmaxf(x, s[sb][i]);
    const float mn = fmaxf(m, max_halves(x));
    const float alpha = pinned(mn == m ? 1.0f : fast_exp2((m - mn) * c));  // exp2(-inf) = 0
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    m = mn;
    base = -mn * c;
    const float bu = mn == -INFINITY ? 0.0f : base;  // a row with no live key yet: P = 0
    rs = 0.0f;
#pragma unroll
    for (int ps = 0; ps < SB * 2; ++ps) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[ps][e] = E::cvt(fast_exp2(fmaf(s[ps >> 1][(ps & 1) * 8 + e], c, bu)));
      rs = E::sum8(pf[ps], rs);
    }
  }
  l += rs;
}

// Key index of accumulator element i of 32-key block sb for this lane half.
__device__ __forceinline__ int acc_row(int sb, int i, int hi) {
  return 32 * sb + 8 * (i >> 2) + 4 * hi + (i & 3);
}

template <int SB, bool CAUSAL>
__device__ __forceinline__ void apply_mask(f32x16 (&s)[SB], int k0, int kl, int qrow, int hi) {
  // Element i of block sb holds key k0 + 4*hi + c with the compile-time
  // c = 32*sb + 8*(i/4) + i%4; it is allowed iff c < lim.
  int lim = kl - k0 - 4 * hi;
  if (CAUSAL) lim = min(lim, qrow - k0 - 4 * hi + 1);
#pragma unroll
  for (int sb = 0; sb < SB; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 32 * sb + 8 * (i >> 2) + (i & 3);
      s[sb][i] = c < lim ? s[sb][i] : -INFINITY;
    }
}

// The banded mask on top of apply_mask's: keys below qrow - win_left or above
// qrow + win_right (a negative bound is no bound) become -inf as well.
template <int SB, bool CAUSAL>
__device__ __forceinline__ void apply_mask_window(f32x16 (&s)[SB], int k0, int kl, int qrow, int hi,
                                                  int win_left, int win_right) {
  int lim = kl - k0 - 4 * hi;
  if (CAUSAL) lim = min(lim, qrow - k0 - 4 * hi + 1);
  if (win_right >= 0) lim = min(lim, qrow + win_right - k0 - 4 * hi + 1);
  const int lo = win_left >= 0 ? qrow - win_left - k0 - 4 * hi : INT_MIN / 2;
#pragma unroll
  for (int sb = 0; sb < SB; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 32 * sb + 8 * (i >> 2) + (i & 3);
      s[sb][i] = (c < lim && c >= lo) ? s[sb][i] : -INFINITY;
    }
}

// O^T += V^T P^T for one key tile. V sits in LDS row-major [BC][VST] (16-bit);
// the transposing read gives every lane 4 consecutive keys of one head-dim
// column, matching the key order of the P^T operand (see acc_row).
template <class E, int SB, int DB, int VST>
__device__ __forceinline__ void pv_product(const typename E::T* vt, int lane,
                                           const typename E::v8 (&pf)[SB * 2],
                                           f32x16 (&o)[DB]) {
  using v4 = typename E::v4;
  using v8 = typename E::v8;
  const int hi = lane >> 5;
  const int row = 4 * hi + ((lane & 15) >> 2);
  const int col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int ps = 0; ps < SB * 2; ++ps) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const typename E::T* base = vt + (16 * ps + row) * VST + 32 * db + col;
      const v4 a0 = E::tr4(base);
      const v4 a1 = E::tr4(base + 8 * VST);
      const v8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = E::mma(a, pf[ps], o[db]);
    }
  }
}

// Final normalisation and the single write of O (16-bit) and LSE.
template <class OutT, int D, int DB>
__device__ __forceinline__ void epilogue_row(const Params& p, int bh, int qrow, int hi, float m,
                                             float l, const f32x16 (&o)[DB]) {
  typedef OutT v4 __attribute__((ext_vector_type(4)));
  const float lt = sum_halves(l);
  const bool live = lt > 0.0f;
  const float inv = live ? p.o_scale / lt : 0.0f;
  if (qrow < p.N) {
    OutT* orow = (OutT*)p.o + ((size_t)bh * p.N + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (OutT)(o[db][4 * g + e] * inv);
        *(v4*)(orow + 32 * db + 8 * g + 4 * hi) = out;
      }
    if (hi == 0)
      p.lse[(size_t)bh * p.N + qrow] = live ? m * p.scale_eff + logf(lt) : -INFINITY;
  }
}

template <class OutT, int D, int DB>
__device__ __forceinline__ void epilogue(const Params& p, const RowRange& rr, int hi, float m,
                                         float l, const f32x16 (&o)[DB]) {
  epilogue_row<OutT, D, DB>(p, rr.bh, rr.qrow, hi, m, l, o);
}

// The same for the 32 rows [row0, row0 + 32) of one wave, with O staged
// through `stage` (32 * D 16-bit elements of LDS owned by this wave) so that
// each global store covers whole rows. Written straight from the accumulator
// layout a row leaves a lane pair as 8-byte pieces, and lines that L2 evicts
// half written cost extra memory writes.
// D: columns this call writes (one row of the stage); DO: elements per row of
// O in memory, the columns starting at col0 (a column slice when DO > D); LSE
// is written only when lse is set, from l_lse (a lane-partial sum like l)
// when that is given instead of l.
template <class OutT, int D, int DB, int DO = D>
__device__ __forceinline__ void epilogue_staged(const Params& p, int bh, int row0, int lane,
                                                float m, float l, const f32x16 (&o)[DB],
                                                unsigned char* stage, int col0 = 0,
                                                bool lse = true, float l_lse = -1.0f) {
  typedef OutT v4 __attribute__((ext_vector_type(4)));
  constexpr int RB = D * 2, CPR = D / 8;  // bytes and 16-byte slots per row
  // Addresses come from an opaque copy of the lane index: computed here, not
  // hoisted to the kernel's start and kept live (or spilled) meanwhile.
  lane = pinned_int(lane);
  const int l32 = lane & 31, hi = lane >> 5;
  const float lt = sum_halves(l);
  const bool live = lt > 0.0f;
  const float inv = live ? p.o_scale / lt : 0.0f;
  // Slot c of row r is stored at slot c ^ (r % CPR): the 32 rows a store
  // instruction touches then spread over the banks.
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (OutT)(o[db][4 * g + e] * inv);
      const int c = 4 * db + g;
      *(FA_LDS v4*)(stage + l32 * RB + ((c ^ (l32 % CPR)) << 4) + 8 * hi) = out;
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int r = k * RPI + lane / CPR, c = lane % CPR;
    const i32x4 v = *(FA_LDS const i32x4*)(stage + r * RB + ((c ^ (r % CPR)) << 4));
    if (row0 + r < p.N) *(i32x4*)((OutT*)p.o + ((size_t)bh * p.N + row0 + r) * DO + col0 + 8 * c) = v;
  }
  if (lse) {
    // l_lse >= 0: the log-sum-exp takes that (lane-partial) sum instead of l
    const float ll = l_lse >= 0.0f ? sum_halves(l_lse) : lt;
    if (hi == 0 && row0 + l32 < p.N)
      p.lse[(size_t)bh * p.N + row0 + l32] = live ? m * p.scale_eff + logf(ll) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Head dimension 256 (bf16 / fp16): each query tile is handled by two
// workgroups, one per 128-column half of V and O. Both compute the whole S
// (Q and K over all 256 dimensions, in the same order), so both arrive at the
// same running maximum and sum without talking to each other; the first also
// writes LSE. S is computed twice, so the launch executes 1.5x the nominal
// FLOPs, but a wave keeps 128 O accumulators instead of 256 and two of these
// workgroups fit on a CU.
// ---------------------------------------------------------------------------
template <class E, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_d256(Params p) {
  using T = typename E::T;
  using v8 = typename E::v8;
  typedef T v4t __attribute__((ext_vector_type(4)));
  constexpr int D = 256, DV = 128;      // Q/K width, V/O columns per workgroup
  constexpr int BR = NW * 32, BC = 32;
  constexpr int KS = D / 16, DB = DV / 32;
  constexpr int KST = D + FA_K_SKEW, VST = DV + FA_V_SKEW;
  constexpr int NT = NW * 64;
  constexpr int KCPR = D / 8, VCPR = DV / 8;  // 16-byte pieces per K / V row
  constexpr int KCH = BC * KCPR / NT, VCH = BC * VCPR / NT;
  static_assert(BC * KCPR % NT == 0 && BC * VCPR % NT == 0, "tile pieces per thread");

  __shared__ __attribute__((aligned(16))) T ks[2][BC * KST];
  __shared__ __attribute__((aligned(16))) T vs[2][BC * VST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int half = blockIdx.x & 1;
  const int logical = blockIdx.x >> 1;
  const int bh0 = logical / p.n_qt;
  const int qt = CAUSAL ? p.n_qt - 1 - (logical - bh0 * p.n_qt) : logical - bh0 * p.n_qt;
  const RowRange rr = row_range_at<BR, BC, CAUSAL>(p, bh0, qt, wave, l32);
  const int N = p.N;
  const size_t head = (size_t)rr.bh * N * D, kv_head = (size_t)rr.kv_bh * N * D;
  const T* Kh = (const T*)p.k + kv_head;
  const T* Vh = (const T*)p.v + kv_head + half * DV;

  v8 qf[KS];
  {
    const auto rq = tile_rsrc((const T*)p.q + head, rr.q_wg0 / BR, BR, N, D * 2);
    const int off = ((rr.qrow - rr.q_wg0) * D + 8 * hi) * 2;
#pragma unroll
    for (int st = 0; st < KS; ++st) qf[st] = __builtin_bit_cast(v8, load16(rq, off + 32 * st));
  }
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.0f;
  const float thr = fminf(kRescaleLog2 / p.c, 1e30f);

  const int kv_lim = rr.kl;
  i32x4 kreg[KCH], vreg[VCH];
  auto gload = [&](int j) __attribute__((always_inline)) {
    const auto rk = tile_rsrc(Kh, j, BC, kv_lim, D * 2);
    // V rows keep their full 512-byte stride; the resource starts at this
    // workgroup's column half and ends within the last row's half.
    const int rows = max(0, min(BC, kv_lim - j * BC));
    const auto rv = buffer_rsrc(Vh + (rows > 0 ? (size_t)j * BC * D : 0),
                                rows > 0 ? ((rows - 1) * D + DV) * 2 : 0);
#pragma unroll
    for (int cc = 0; cc < KCH; ++cc) {
      const int piece = tid + cc * NT;
      kreg[cc] = load16(rk, ((piece / KCPR) * D + (piece % KCPR) * 8) * 2);
    }
#pragma unroll
    for (int cc = 0; cc < VCH; ++cc) {
      const int piece = tid + cc * NT;
      vreg[cc] = load16(rv, ((piece / VCPR) * D + (piece % VCPR) * 8) * 2);
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < KCH; ++cc) {
      const int piece = tid + cc * NT;
      *(i32x4*)(&ks[buf][(piece / KCPR) * KST + (piece % KCPR) * 8]) = kreg[cc];
    }
#pragma unroll
    for (int cc = 0; cc < VCH; ++cc) {
      const int piece = tid + cc * NT;
      *(i32x4*)(&vs[buf][(piece / VCPR) * VST + (piece % VCPR) * 8]) = vreg[cc];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int j = 0; j < rr.nt; ++j) {
    const int buf = j & 1;
    gload(j + 1);
    auto tile = [&](auto masked) __attribute__((always_inline)) {
      f32x16 sc[1] = {f32x16{}};
      {
        // operand reads held one product ahead (operand_fence)
        v8 ring[2];
#pragma unroll
        for (int t = 0; t <= KS; ++t) {
          if (t < KS) {
            ring[t & 1] = *(const v8*)(ks[buf] + l32 * KST + 16 * t + 8 * hi);
            operand_fence();
          }
          if (t > 0) {
            sc[0] = E::mma(ring[(t - 1) & 1], qf[t - 1], sc[0]);
            operand_fence();
          }
        }
      }
      if constexpr (decltype(masked)::value) apply_mask<1, CAUSAL>(sc, j * BC, rr.kl, rr.qrow, hi);
      v8 pf[2];
      online_softmax<E, 1, DB>(sc, p.c, thr, m, l, o, pf);
      {
        // O^T += V^T P^T as pv_product computes it, reads one product ahead
        const int row = 4 * hi + ((lane & 15) >> 2);
        const int col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        auto vread = [&](int u) __attribute__((always_inline)) {
          const T* b = vs[buf] + (16 * (u / DB) + row) * VST + 32 * (u % DB) + col;
          const auto a0 = E::tr4(b);
          const auto a1 = E::tr4(b + 8 * VST);
          return __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        v8 ring[2];
#pragma unroll
        for (int t = 0; t <= 2 * DB; ++t) {
          if (t < 2 * DB) {
            ring[t & 1] = vread(t);
            operand_fence();
          }
          if (t > 0) {
            const int u = t - 1;
            o[u % DB] = E::mma(ring[u & 1], pf[u / DB], o[u % DB]);
            operand_fence();
          }
        }
      }
    };
    if (j < rr.wfull) tile(std::false_type{});
    else if (j < rr.wnt) tile(std::true_type{});
    sstore(buf ^ 1);
    __syncthreads();
  }

  const float lt = sum_halves(l);
  const bool live = lt > 0.0f;
  const float inv = live ? p.o_scale / lt : 0.0f;
  if (rr.qrow < N) {
    T* orow = (T*)p.o + ((size_t)rr.bh * N + rr.qrow) * D + half * DV;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v4t out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (T)(o[db][4 * g + e] * inv);
        *(v4t*)(orow + 32 * db + 8 * g + 4 * hi) = out;
      }
    if (half == 0 && hi == 0)
      p.lse[(size_t)rr.bh * N + rr.qrow] = live ? m * p.scale_eff + logf(lt) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS tile copies (gfx950 buffer_load_dwordx4 ... lds, 16 bytes per
// lane): no staging registers and no LDS write instructions. Rows are stored
// unpadded and the 16-byte slots of each row are XOR-permuted so that the
// operand reads of the kernels below are free of bank conflicts.
// ---------------------------------------------------------------------------

// Slot permutations (16-byte slots, row = D*2 bytes). k_swz keeps the 16 rows
// a quarter-wave reads at one logical slot on 16 distinct 16-byte bank
// groups: with 256-byte or longer rows every row starts at bank 0, so the
// slots themselves must differ (r mod D/8); with 128-byte rows (d = 64) odd
// rows start half-way round the banks, so rows r and r ^ 1 may share a slot
// and the permutation takes r / 2. v_swz keeps the 8 rows x 64 bytes of one
// transposing read on distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D == 64) return (r >> 1) & 7;
  return r & (D / 8 - 1);
}
// fp8 K rows (D bytes, D/16 slots): the 16 rows a quarter-wave reads at one
// logical slot land on 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int k8_swz(int r) {
  if constexpr (D == 128) return (r >> 1) & 7;
  return (r >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  if constexpr (D == 128) return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0);
  return (r & 3) << 1;
}

// Four e4m3 codes -> four bf16, exact: every e4m3 value (4 significant bits,
// exponents 2^-9 .. 2^8) is a bf16 value; two codes per convert, scale 1.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(unsigned w) {
  u32x2 r;
  r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// 16 bytes per lane from a buffer straight into LDS at dst + 16 * lane (dst is
// wave-uniform). Kept as a function of its own: used directly inside a lambda
// of the kernel, the host compilation pass silently drops the kernel's handle.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rs, unsigned char* dst,
                                           int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)dst, 16, byte_off, 0, 0, 0);
}

// The same for one dword per lane (lane i lands at dst + 4 i).
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t rs, unsigned char* dst, int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)dst, 4, byte_off, 0, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// s_waitcnt vmcnt(N): all but the N most recent vector-memory loads are done
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt / lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// bf16 / fp16 kernel (the default for 16-bit inputs)
//
// NW waves per workgroup (32 query rows each), two workgroups per CU at
// NW = 4. K and V tiles reach LDS through the direct-to-LDS copies above, two
// buffers deep: the copy of tile j + 1 lands while tile j is used. Within a
// tile every MFMA's LDS operand is read FA_LOOKAHEAD MFMAs ahead through a
// small ring of registers (held there by scheduling fences), and the first V
// operands of O += P V are read before the softmax arithmetic so that it
// hides their latency. Used for short causal sequences (the pipelined kernel
// below takes the rest), sliding windows and packed batches of short
// sequences.
// ---------------------------------------------------------------------------
template <class E, int D, int BC, int NW, bool CAUSAL, bool WIN = false, bool VL = false>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_16bit_dma(Params p) {
  using T = typename E::T;
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  constexpr int BR = NW * 32;
  constexpr int KS = D / 16;
  constexpr int SB = BC / 32;
  constexpr int DB = D / 32;
  constexpr int PS = BC / 16;
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int TB = BC * RB;
  constexpr int NDMA = TB / (1024 * NW);
  constexpr int NS = SB * KS, NPV = PS * DB;
  constexpr int LA = FA_LOOKAHEAD;
  static_assert(TB % (1024 * NW) == 0, "tile must split into 1 KB copies per wave");

  // One named array per buffer (not one 2-D array): distinct objects let the
  // compiler see that an in-flight copy into one buffer cannot alias operand
  // reads from another, so it does not wait for the copy before them.
  __shared__ __attribute__((aligned(1024))) unsigned char k0s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char k1s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char v0s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char v1s[TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  RowRange rr;
  if constexpr (VL) {
    // Packed batch: the item's sequence becomes a one-head problem.
    int bh, r;
    varlen_item(p.H, p.n_qt, bh, r);
    const int qt = CAUSAL ? p.n_qt - 1 - r : r;  // longest query tiles first
    if (!enter_segment<T, T, D>(p, bh, qt * BR)) return;
    rr = row_range_at<BR, BC, CAUSAL>(p, 0, qt, wave, l32);
  } else {
    rr = row_range<BR, BC, CAUSAL>(p, wave, l32);
  }
  const int N = p.N;
  // Sliding window: the workgroup streams tiles [t0, nt); this wave computes
  // [wt0, wnt) of them, of which [whead, wfull) need no mask.
  int t0 = 0, wt0 = 0, whead = 0;
  if constexpr (WIN) {
    const int wl = p.win_left, wr = p.win_right;
    const int qw0 = rr.q_wg0 + 32 * wave;
    if (wl >= 0) {
      t0 = max(0, rr.q_wg0 - wl) / BC;
      wt0 = max(0, qw0 - wl) / BC;
      whead = (max(0, qw0 + 31 - wl) + BC - 1) / BC;
    }
    if (wr >= 0) {
      rr.nt = min(rr.nt, (min(rr.kl, rr.q_wg0 + BR + wr) + BC - 1) / BC);
      rr.wnt = min(rr.wnt, (max(0, min(rr.kl, qw0 + 32 + wr)) + BC - 1) / BC);
      rr.wfull = min(rr.wfull, max(0, qw0 + wr + 1) / BC);
    }
    t0 = __builtin_amdgcn_readfirstlane(t0);
  }
  const size_t head = (size_t)rr.bh * N * D, kv_head = (size_t)rr.kv_bh * N * D;
  const T* Kh = (const T*)p.k + kv_head;
  const T* Vh = (const T*)p.v + kv_head;

  v8 qf[KS];
  {
    const auto rq = tile_rsrc((const T*)p.q + head, rr.q_wg0 / BR, BR, N, RB);
    const int off = ((rr.qrow - rr.q_wg0) * D + 8 * hi) * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(v8, load16(rq, off + 32 * s));
  }
  int koff[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) koff[st] = l32 * RB + (((2 * st + hi) ^ k_swz<D>(l32)) << 4);
  int voff[DB];
  {
    const int g = lane >> 4, i = lane & 15;
    const int r = 4 * (g >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 4 * db + 2 * (g & 1) + ((i & 3) >> 1);
      voff[db] = r * RB + ((c ^ v_swz<D>(r)) << 4) + 8 * (i & 1);
    }
  }

  auto copy_tile = [&](const T* xh, int j, unsigned char* dst, auto is_v) __attribute__((always_inline)) {
    const auto rs = tile_rsrc(xh, j, BC, rr.kl, RB);
#pragma unroll
    for (int c = 0; c < NDMA; ++c) {
      const int blk = c * NW + wave;
      const int slot = blk * 64 + lane;
      const int r = slot / CPR, ps = slot % CPR;
      const int lc = ps ^ (decltype(is_v)::value ? v_swz<D>(r) : k_swz<D>(r));
      lds_copy16(rs, dst + blk * 1024, r * RB + (lc << 4));
    }
  };
  auto kfrag = [&](const unsigned char* kb, int u) __attribute__((always_inline)) {
    return *(const v8*)(kb + 32 * (u / KS) * RB + koff[u % KS]);  // u = sb*KS + st
  };
  auto vfrag = [&](const unsigned char* vb, int u) __attribute__((always_inline)) {
    const unsigned char* b = vb + 16 * (u / DB) * RB + voff[u % DB];  // u = ps*DB + db
    const v4 a0 = __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)b));
    const v4 a1 =
        __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(b + 8 * RB)));
    return __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  // m: reference maximum (raw score units); base = -m * c, +inf while m = -inf
  float m = -INFINITY, base = INFINITY, l = 0.0f;

  auto tile = [&](int j, const unsigned char* kb, const unsigned char* vb, auto masked)
      __attribute__((always_inline)) {
    // S = K Q^T, operand reads LA steps ahead
    f32x16 s[SB];
#pragma unroll
    for (int x = 0; x < SB; ++x) s[x] = f32x16{};
    v8 ring[LA + 1];
#pragma unroll
    for (int t = 0; t < NS + LA; ++t) {
      if (t < NS) {
        ring[t % (LA + 1)] = kfrag(kb, t);
        operand_fence();
      }
      const int u = t - LA;
      if (u >= 0) {
        s[u / KS] = E::mma(ring[u % (LA + 1)], qf[u % KS], s[u / KS]);
        operand_fence();
      }
    }
    // first V operands, in flight during the softmax
    v8 vring[LA + 1];
#pragma unroll
    for (int t = 0; t < LA; ++t) vring[t] = vfrag(vb, t);
    operand_fence();
    if constexpr (decltype(masked)::value) {
      if constexpr (WIN)
        apply_mask_window<SB, CAUSAL>(s, j * BC, rr.kl, rr.qrow, hi, p.win_left, p.win_right);
      else
        apply_mask<SB, CAUSAL>(s, j * BC, rr.kl, rr.qrow, hi);
    }
    v8 pf[PS];
    lazy_softmax<E, SB, DB>(s, p.c, m, base, l, o, pf);
    // O += P V, operand reads LA steps ahead
#pragma unroll
    for (int t = LA; t < NPV + LA; ++t) {
      if (t < NPV) {
        vring[t % (LA + 1)] = vfrag(vb, t);
        operand_fence();
      }
      const int u = t - LA;
      o[u % DB] = E::mma(vring[u % (LA + 1)], pf[u / DB], o[u % DB]);
      operand_fence();
    }
  };
  // Iteration j uses buffer j % 2 and copies tile j + 1 into the buffer
  // iteration j - 1 used; every copy has landed at the end of an iteration.
  // Copies past the last tile have an empty byte range and move nothing.
  auto step = [&](int j, const unsigned char* kc, const unsigned char* vc, unsigned char* kn,
                  unsigned char* vn) __attribute__((always_inline)) {
    copy_tile(Kh, j + 1, kn, std::false_type{});
    copy_tile(Vh, j + 1, vn, std::true_type{});
    if constexpr (WIN) {
      if (j >= wt0 && j < rr.wnt) {
        if (j >= whead && j < rr.wfull) tile(j, kc, vc, std::false_type{});
        else tile(j, kc, vc, std::true_type{});
      }
    } else {
      if (j < rr.wfull) tile(j, kc, vc, std::false_type{});
      else if (j < rr.wnt) tile(j, kc, vc, std::true_type{});
    }
    wait_vmem();
    __syncthreads();
  };

  // Tiles are numbered from t0 (0 without a window); buffers follow j - t0.
  copy_tile(Kh, t0, k0s, std::false_type{});
  copy_tile(Vh, t0, v0s, std::true_type{});
  wait_vmem();
  __syncthreads();
  for (int j = t0; j < rr.nt; j += 2) {
    step(j, k0s, v0s, k1s, v1s);
    if (j + 1 < rr.nt) step(j + 1, k1s, v1s, k0s, v0s);
  }
  epilogue<T, D, DB>(p, rr, hi, m, l, o);
}

// Calls f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{}).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// bf16 / fp16 kernel, software-pipelined (the default for 16-bit inputs).
//
// The unit of work is a 32-key half h of a 64-key LDS tile:
//   S(h) = K(h) Q^T (MFMA),  P(h) from S(h) (vector ALU),  O += V(h)^T P(h)^T (MFMA).
// Step h issues the MFMAs of S(h+1) and of O += V(h-1)^T P(h-1)^T while the
// vector ALU turns S(h) into P(h). The two MFMA streams and the vector work
// of a step do not depend on each other, so a single wave keeps the matrix
// core and the ALU busy at the same time. K runs one tile ahead of V:
// iteration t reads K of tile t+1 and V of tile t while the copies of K t+2
// and V t+1 land (two LDS buffers per operand).
//
// The reference maximum is lazy and needs no row maximum per tile. P(h) is
// formed against the row's current reference m; since the row sum of P(h)
// is needed anyway, it also tells whether any score got too far above m: if
// a lane's partial sum exceeds E::kPBound, or is inf / NaN (first tile, where
// m = -inf), a rarely taken branch takes the true maximum of the half, moves
// m there, rescales O and l and recomputes P(h). Otherwise every P is at most
// E::kPBound, which the 16-bit P and the fp32 accumulators hold without loss,
// and O / l is the same exact softmax for any reference.
//
// Each wave owns 32 query rows and two waves share each SIMD. Within a wave
// at most one key tile needs a mask (a tile covers a wave's row range, see
// row_range), and it is the wave's last tile.
// ---------------------------------------------------------------------------

// Bit cast between operand types of one size; a zero value otherwise (for
// code paths that a kernel variant compiles but never takes).
template <class To, class From>
__device__ __forceinline__ To same_size_cast(const From& x) {
  if constexpr (sizeof(To) == sizeof(From)) return __builtin_bit_cast(To, x);
  else return To{};
}

// DV < D (head dim 256): the workgroup owns columns [vh*DV, vh*DV + DV) of V
// and O, vh = 0 .. D/DV - 1, and computes the whole S over all D dimensions;
// the workgroups of one query tile reach the same reference maxima and sums
// with no communication, and the first one writes LSE.
template <class E, int D, int NW, bool CAUSAL, bool F8, bool VL = false, int DV = D>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_pipe(Params p) {
  using T = typename E::T;  // P, V in LDS and O (bfloat16 for fp8 inputs)
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  using QT = std::conditional_t<F8, i32x8, v8>;  // one Q or K operand of the S product
  static_assert(!(F8 && VL), "packed batches take 16-bit inputs");
  static_assert(DV == D || (!F8 && !VL && D % DV == 0), "column slices: 16-bit inputs");
  constexpr int NVH = D / DV;  // workgroups per query tile (column slices of V and O)
  constexpr int BR = NW * 32;  // query rows per workgroup
  constexpr int BC = 64;       // keys per LDS tile
  constexpr int KS = F8 ? D / 64 : D / 16;  // S MFMA steps over the head dim
  constexpr int DB = DV / 32;  // 32-wide blocks of the O^T columns this workgroup owns
  constexpr int RB = D * 2;    // bytes per 16-bit row in memory (and per 16-bit K row in LDS)
  constexpr int VRB = DV * 2;  // bytes per V row (slice) in LDS
  constexpr int KRB = F8 ? D : RB;  // bytes per K row (global and LDS)
  constexpr int CPR = DV / 8;  // 16-byte slots per V row (slice) in LDS
  constexpr int KCPR = KRB / 16;    // 16-byte slots per K row
  constexpr int TB = BC * RB;  // bytes per K buffer
  constexpr int TBV = BC * VRB;  // bytes per V buffer
  constexpr int NKC = BC * KRB / 1024;  // 1 KB copies per K tile
  constexpr int NDMA = (NKC + NW - 1) / NW;  // K copies per wave per tile (some idle when ragged)
  constexpr int NVC = TBV / 1024;  // 1 KB copies per 16-bit V tile
  constexpr int NDMAV = NVC / NW;  // V copies per wave per tile
  constexpr int NPV = 2 * DB;  // PV MFMA steps per half (2 x 16 keys)
  constexpr int LA = FA_PIPE_LOOKAHEAD > 0 ? FA_PIPE_LOOKAHEAD : (D == 128 && DV == D ? 2 : 1);
  static_assert(F8 || NKC % NW == 0, "16-bit tiles must split into 1 KB copies per wave");
  static_assert(F8 || NVC % NW == 0, "16-bit V tiles must split into 1 KB copies per wave");

  // One named array per buffer: distinct objects let the compiler see that a
  // copy in flight into one buffer cannot alias operand reads from another.
  __shared__ __attribute__((aligned(1024))) unsigned char k0s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char k1s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char v0s[TBV];
  __shared__ __attribute__((aligned(1024))) unsigned char v1s[TBV];
  auto kbuf = [&](int i) __attribute__((always_inline)) -> unsigned char* { return i == 0 ? k0s : k1s; };
  auto vbuf = [&](int i) __attribute__((always_inline)) -> unsigned char* { return i == 0 ? v0s : v1s; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // The workgroup's work unit u of head bh. Causal work is folded: a
  // workgroup takes query tile n_qt-1-u and then tile u of one head, so every
  // workgroup streams n_qt+1 key-tile runs and the launch needs no
  // longest-first order to stay balanced; the workgroups are then issued head
  // by head, and those that run together on an XCD stream the same heads' K/V
  // through its L2. The middle tile of an odd n_qt is one workgroup's only
  // tile.
  const int units = CAUSAL ? (p.n_qt + 1) / 2 : p.n_qt;
  int bh, u, vh = 0;
  if constexpr (VL) {
    varlen_item(p.H, units, bh, u);
  } else {
    const int bid = blockIdx.x, total = gridDim.x;
    int logical = bid;
    if (total % kXcds == 0) logical = (bid % kXcds) * (total / kXcds) + bid / kXcds;
    if constexpr (NVH > 1) {  // the column slices of a unit are consecutive (one XCD)
      vh = logical % NVH;
      logical /= NVH;
    }
    bh = logical / units;
    u = logical - bh * units;
  }
  int n_qt = p.n_qt;
  if constexpr (VL) {
    // Packed batch: the item's sequence becomes a one-head problem whose
    // query tiles are folded the same way; units past them have no work.
    if (!enter_segment<T, T, D>(p, bh, u * BR)) return;
    bh = 0;
    n_qt = (p.N + BR - 1) / BR;
    if (CAUSAL && u >= (n_qt + 1) / 2) return;
  }
  const int N = p.N;

  // Q^T operand: lane holds its query row's head-dim elements
  // [16*st + 8*hi, +8) (16-bit) or [64*st + 32*hi, +32) (fp8).
  QT qf[KS];
  auto load_q = [&](const RowRange& r, int hi) __attribute__((always_inline)) {
    const size_t qhead = (size_t)r.bh * N * D;
    const auto rq = tile_rsrc((const unsigned char*)p.q + qhead * (KRB / D), r.q_wg0 / BR, BR, N, KRB);
    const int row = r.qrow - r.q_wg0;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (F8) {
        const int off = row * KRB + 64 * s + 32 * hi;
        qf[s] = __builtin_shufflevector(load16(rq, off), load16(rq, off + 16), 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        qf[s] = __builtin_bit_cast(v8, load16(rq, row * KRB + 32 * s + 16 * hi));
      }
    }
  };

  // One query tile of one head, start to finish; with desc, its key tiles
  // are streamed last to first.
  auto process = [&](int bh, int qt, bool desc) __attribute__((always_inline)) {
  // Lane-derived values are recomputed per work item from a lane index the
  // compiler cannot hoist, so that they are not kept live across the items
  // (16-bit d = 128; when the kernel still spilled, this halved its scratch).
  // The fp8 and column-slice instances keep an opaque copy of the kernel's
  // lane index (measured 0.5% faster there).
  constexpr bool FRESH = !F8 && DV == D;
  const int lx = FRESH ? fresh_lane() : lane;   // slots, rows, epilogue
  const int ln = FRESH ? lx : pinned_int(lane);  // operand read offsets
  const int l32 = lx & 31, hi = lx >> 5;
  // K operand addresses: 16-bit, one 16-byte slot per MFMA step; fp8, two.
  int koff[F8 ? 2 * KS : KS];
  if constexpr (F8) {
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        koff[2 * st + x] = (ln & 31) * KRB + (((4 * st + 2 * (ln >> 5) + x) ^ k8_swz<D>(ln & 31)) << 4);
  } else {
#pragma unroll
    for (int st = 0; st < KS; ++st)
      koff[st] = (ln & 31) * RB + (((2 * st + (ln >> 5)) ^ k_swz<D>(ln & 31)) << 4);
  }
  int voff[DB];
  {
    const int g = ln >> 4, i = ln & 15;
    const int r = 4 * (g >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 4 * db + 2 * (g & 1) + ((i & 3) >> 1);
      voff[db] = r * VRB + ((c ^ v_swz<DV>(r)) << 4) + 8 * (i & 1);
    }
  }
  RowRange rr = row_range_at<BR, BC, CAUSAL>(p, bh, qt, wave, l32);
  const size_t head = (size_t)rr.bh * N * D, kv_head = (size_t)rr.kv_bh * N * D;  // elements
  const unsigned char* Kh = (const unsigned char*)p.k + kv_head * (KRB / D);
  const unsigned char* Vh = (const unsigned char*)p.v + kv_head * (KRB / D) + vh * VRB;
  (void)head;
  // The key tile of step j: j, or nt-1-j last to first. Steps at or past nt
  // (copies and scores ahead of the end) keep tile j, whose keys are all
  // masked for the workgroup's rows (causal bound or key_len).
  auto ktile = [&](int j) __attribute__((always_inline)) { return desc && j < rr.nt ? rr.nt - 1 - j : j; };

  load_q(rr, hi);
  // One buffer resource per operand over the head's first kl key rows (the
  // host keeps a head under 1 GiB): a tile's copy only adds its byte offset,
  // and rows at or beyond kl (a ragged last tile, tiles past the end) read
  // as zeros.
  const auto rsK = buffer_rsrc(Kh, rr.kl * KRB);
  const auto rsV = buffer_rsrc(Vh, rr.kl * KRB);
  // K tile j (and V tile j for 16-bit inputs) straight into LDS, 16-byte
  // slots permuted per row as the operand reads expect.
  auto copy_tile = [&](int j, unsigned char* dst, auto is_v) __attribute__((always_inline)) {
    constexpr bool IV = decltype(is_v)::value;
    // rb: bytes per row in memory; an LDS row holds cpr 16-byte slots
    constexpr int cpr = IV ? CPR : KCPR, rb = IV ? RB : KRB;
    constexpr int nd = IV ? NDMAV : NDMA, nc = IV ? NVC : NKC;
#pragma unroll
    for (int c = 0; c < nd; ++c) {
      const int blk = c * NW + wave;
      if (nc % NW == 0 || blk < nc) {
        const int slot = blk * 64 + lx;
        const int r = slot / cpr, ps = slot % cpr;
        const int lc = ps ^ (IV ? v_swz<DV>(r) : F8 ? k8_swz<D>(r) : k_swz<D>(r));
        lds_copy16(IV ? rsV : rsK, dst + blk * 1024, ktile(j) * (BC * rb) + r * rb + (lc << 4));
      }
    }
  };
  // fp8 V: this lane's 16 codes of the tile in flight, widened to bf16
  // (exactly) and stored into the 16-bit V layout at the end of the iteration.
  constexpr int VSLOTS = BC * D / 16;  // 16-code pieces per fp8 V tile
  const int vslot = wave * 64 + lx;
  i32x4 vreg = {};
  auto vload = [&](int j) __attribute__((always_inline)) {
    if (vslot < VSLOTS) vreg = load16(rsV, ktile(j) * (BC * D) + vslot * 16);
  };
  auto vstore = [&](unsigned char* dst) __attribute__((always_inline)) {
    if (vslot < VSLOTS) {
      const int r = vslot / (D / 16), cc = vslot % (D / 16);
      i32x4 w0, w1;
      u32x2 t;
      t = fp8x4_to_bf16x4((unsigned)vreg[0]); w0[0] = t[0]; w0[1] = t[1];
      t = fp8x4_to_bf16x4((unsigned)vreg[1]); w0[2] = t[0]; w0[3] = t[1];
      t = fp8x4_to_bf16x4((unsigned)vreg[2]); w1[0] = t[0]; w1[1] = t[1];
      t = fp8x4_to_bf16x4((unsigned)vreg[3]); w1[2] = t[0]; w1[3] = t[1];
      *(i32x4*)(dst + r * RB + (((2 * cc) ^ v_swz<D>(r)) << 4)) = w0;
      *(i32x4*)(dst + r * RB + (((2 * cc + 1) ^ v_swz<D>(r)) << 4)) = w1;
    }
  };
  // K operand of S MFMA step st over keys [32*h, 32*h + 32) of the tile at kb
  auto kfrag = [&](const unsigned char* kb, int h, int st) __attribute__((always_inline)) -> QT {
    if constexpr (F8) {
      const unsigned char* b = kb + 32 * h * KRB;
      return __builtin_shufflevector(*(const i32x4*)(b + koff[2 * st]),
                                     *(const i32x4*)(b + koff[2 * st + 1]), 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      return *(const v8*)(kb + 32 * h * RB + koff[st]);
    }
  };
  // V^T operand of PV step u = ps*DB + db over keys 32*h + 16*ps + [0, 16)
  auto vfrag = [&](const unsigned char* vb, int h, int u) __attribute__((always_inline)) {
    const unsigned char* b = vb + (32 * h + 16 * (u / DB)) * VRB + voff[u % DB];
    const v4 a0 = __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)b));
    const v4 a1 =
        __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(b + 8 * VRB)));
    return __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // S^T = K Q^T over one 32-key half (the first tile, before the pipeline runs)
  auto scores = [&](const unsigned char* kb, int h, f32x16& s) __attribute__((always_inline)) {
    s = f32x16{};
    QT ring[LA + 1];
#pragma unroll
    for (int t = 0; t < KS + LA; ++t) {
      if (t < KS) ring[t % (LA + 1)] = kfrag(kb, h, t);
      const int u = t - LA;
      if (u >= 0) {
        if constexpr (F8)  // formats 0/0: fp8 e4m3 operands; E8M0 scales 127 = 1.0
          s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ring[u % (LA + 1)], qf[u], s, 0, 0, 0,
                                                              127, 0, 127);
        else
          s = E::mma(ring[u % (LA + 1)], qf[u], s);
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  // m: reference maximum (raw score units); base = -m * c, +inf while m = -inf
  float m = -INFINITY, base = INFINITY, l = 0.0f;
  const float c = p.c;

  // The masks of one half (its first key k0) for this lane's query row.
  auto mask_half = [&](f32x16& sh, int k0) __attribute__((always_inline)) {
    auto& s1 = *reinterpret_cast<f32x16(*)[1]>(&sh);
    apply_mask<1, CAUSAL>(s1, k0, rr.kl, rr.qrow, hi);
  };
  // The rare branch of probs: move the reference maximum of the rows of this
  // half whose exponentials left the bound, rescale O and l, recompute P.
  auto fix_probs = [&](const f32x16& s, v8 (&pf)[2], float& rs) __attribute__((always_inline)) {
    float x = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) x = fmaxf(x, s[i]);
    const float mn = fmaxf(m, max_halves(x));
    const float alpha = pinned(mn == m ? 1.0f : fast_exp2((m - mn) * c));
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    m = mn;
    base = -mn * c;
    const float bu = mn == -INFINITY ? 0.0f : base;
    rs = 0.0f;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ps][e] = E::cvt(fast_exp2(fmaf(s[8 * ps + e], c, bu)));
      rs = E::sum8(pf[ps], rs);
    }
  };
  // P of one half from its raw scores s (k0 = its first key); updates l and,
  // on the rare branch, m, base and O. The running sum adds the same rounded
  // P values that multiply V, so the weights applied to V's rows sum to one up
  // to fp32 accumulation.
  auto probs = [&](f32x16& s, v8 (&pf)[2], int k0, auto masked) __attribute__((always_inline)) {
    if constexpr (FA_PIPE_IGLP >= 0) __builtin_amdgcn_iglp_opt(FA_PIPE_IGLP);
    if constexpr (decltype(masked)::value) mask_half(s, k0);
    float rs = 0.0f;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ps][e] = E::cvt(fast_exp2(fmaf(s[8 * ps + e], c, base)));
      rs = E::sum8(pf[ps], rs);
    }
    if (__builtin_amdgcn_ballot_w64(!(rs <= E::kPBound)) != 0) fix_probs(s, pf, rs);
    l += rs;
  };

  // P of the item's first half (first key k0), while m is still -inf: the
  // reference is set from this half's true row maximum at once (O and l are
  // still zero), with no first try against m.
  auto first_probs = [&](f32x16& s, v8 (&pf)[2], int k0, auto masked) __attribute__((always_inline)) {
    if constexpr (decltype(masked)::value) mask_half(s, k0);
    float x = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) x = fmaxf(x, s[i]);
    m = max_halves(x);
    base = -m * c;
    const float bu = m == -INFINITY ? 0.0f : base;
    float rs = 0.0f;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ps][e] = E::cvt(fast_exp2(fmaf(s[8 * ps + e], c, bu)));
      rs = E::sum8(pf[ps], rs);
    }
    l = rs;
  };

  f32x16 sa, sb;
  v8 pfa[2], pfb[2];
  // The S product of half h of the K tile at kb (when hn) and O += V^T P^T of
  // half h of the V tile at vb as one stream of products: each operand read
  // is issued LA products before the product that takes it, and fences that
  // only vector ALU, scalar and global-memory instructions may cross keep the
  // scheduler from sinking the reads back to their products (which would
  // leave every product waiting out a whole LDS latency). The softmax
  // arithmetic that follows in program order still moves up among them.
  constexpr int kFence = 0x2 | 0x4 | 0x10 | 0x400;  // VALU, SALU, VMEM, transcendental
  auto mma_half = [&](const unsigned char* kb, int h, f32x16& s, const unsigned char* vb,
                      const v8 (&pf)[2], auto hn) __attribute__((always_inline)) {
    constexpr int NS = decltype(hn)::value ? KS : 0;
    constexpr int NT = NS + NPV;
    if constexpr (NS > 0) s = f32x16{};
    v8 ring[LA + 1];
#pragma unroll
    for (int t = 0; t < NT + LA; ++t) {
      if (t < NT) {
        if (t < NS) ring[t % (LA + 1)] = same_size_cast<v8>(kfrag(kb, h, t));
        else ring[t % (LA + 1)] = vfrag(vb, h, t - NS);
        __builtin_amdgcn_sched_barrier(kFence);
      }
      const int u = t - LA;
      if (u >= 0) {
        if (u < NS) s = E::mma(ring[u % (LA + 1)], same_size_cast<v8>(qf[u]), s);
        else o[(u - NS) % DB] = E::mma(ring[u % (LA + 1)], pf[(u - NS) / DB], o[(u - NS) % DB]);
        __builtin_amdgcn_sched_barrier(kFence);
      }
    }
  };
  // For fp8 inputs: the S product of half h (scaled fp8 MFMAs, K operands read
  // just ahead) and then O += V^T P^T of half h in bf16.
  auto mma_half_f8 = [&](const unsigned char* kb, int h, f32x16& s, const unsigned char* vb,
                         const v8 (&pf)[2], auto hn) __attribute__((always_inline)) {
    if constexpr (decltype(hn)::value) scores(kb, h, s);
    v8 ring[LA + 1];
#pragma unroll
    for (int t = 0; t < NPV + LA; ++t) {
      if (t < NPV) ring[t % (LA + 1)] = vfrag(vb, h, t);
      const int u = t - LA;
      if (u >= 0) o[u % DB] = E::mma(ring[u % (LA + 1)], pf[u / DB], o[u % DB]);
    }
  };
  // One iteration: tile t's V (vb) and tile t+1's K (kb). On entry sb holds
  // S of half 2t+1 and pfa P of half 2t; on exit sb holds S of half 2t+3 and
  // pfa P of half 2t+2.
  auto iteration = [&](int t, const unsigned char* kb, const unsigned char* vb, auto has_next,
                       auto mask_a, auto mask_b) __attribute__((always_inline)) {
    if constexpr (F8) {
      mma_half_f8(kb, 0, sa, vb, pfa, has_next);
      probs(sb, pfb, BC * ktile(t) + 32, mask_a);
      mma_half_f8(kb, 1, sb, vb, pfb, has_next);
    } else {
      mma_half(kb, 0, sa, vb, pfa, has_next);
      probs(sb, pfb, BC * ktile(t) + 32, mask_a);
      mma_half(kb, 1, sb, vb, pfb, has_next);
    }
    if constexpr (decltype(has_next)::value) probs(sa, pfa, BC * ktile(t + 1), mask_b);
  };
  // K tile j lives in buffer j % 2, V tile j in buffer j % 2. Iteration t
  // reads K t+1 and V t and refills the buffers of K t (with K t+2) and of
  // V t-1 (with V t+1), so every copy has a whole iteration to land; at the
  // end of an iteration every copy has landed. Copies past the end have an
  // empty byte range and move nothing.
  // fp8 V tiles take registers instead: loaded with the copies, stored to
  // vx just before the iteration's barrier.
  auto copies = [&](int t, unsigned char* kx, unsigned char* vx) __attribute__((always_inline)) {
    copy_tile(t + 2, kx, std::false_type{});
    if constexpr (F8) vload(t + 1);
    else copy_tile(t + 1, vx, std::true_type{});
  };
  auto sync_after = [&](unsigned char* vx) __attribute__((always_inline)) {
    if constexpr (F8) vstore(vx);
    wait_vmem();
    __syncthreads();
  };

  copy_tile(0, k0s, std::false_type{});
  copy_tile(1, k1s, std::false_type{});
  if constexpr (F8) {
    vload(0);
    vstore(v0s);
  } else {
    copy_tile(0, v0s, std::true_type{});
  }
  wait_vmem();
  __syncthreads();
  // The wave's first step: last to first, the tiles past its rows' last key
  // come first and are skipped.
  const int s0 = desc ? rr.nt - rr.wnt : 0;
  if (rr.wnt > 0 && s0 == 0) {
    scores(k0s, 0, sa);
    scores(k0s, 1, sb);
    if (!desc && 0 < rr.wfull) first_probs(sa, pfa, 0, std::false_type{});
    else first_probs(sa, pfa, BC * ktile(0), std::true_type{});
  }
  __syncthreads();  // K of tile 0 is read by every wave before its buffer is refilled
  // Steps [w_lo, w_hi) are the wave's: ascending [0, wnt); last to first
  // [nt - wnt, nt), so the wave skips the tiles past its rows' last key, which
  // come first.
  const int w_lo = s0, w_hi = desc ? rr.nt : rr.wnt;
  // Masked steps: one variant with every mask applied (an unneeded mask
  // changes nothing) and the next tile always scored: past the last tile the
  // next tile's keys are all masked for the wave's rows (causal bound or
  // key_len; the buffer holds finite stale or zero data), so it adds nothing.
  // Unmasked steps reach only keys below the wave's first row and key_len.
  // Ascending, steps [0, ts) are unmasked and the rest are masked (the
  // wave's diagonal and ragged tiles, then the steps in which only other
  // waves compute). Last to first, the first kDiag steps hold the diagonal
  // and ragged tiles (nt*BC <= q_wg0 + BR), then steps [kDiag, nt-1) are
  // unmasked, and the last one is masked; a wave whose first step s0 is
  // past 0 scores its first tile in step s0-1.
  // Both orders run the same two loops, masked then unmasked, in two passes
  // (one inlined copy of each; more copies of the iteration make the kernel
  // spill). Two steps per pass of a loop, from an even t, so that every buffer
  // is named at compile time: with a buffer chosen at run time the compiler
  // cannot tell the operand reads from the copies in flight and waits for
  // every copy.
  constexpr int kDiag = BR / BC;
  static_assert(BR % BC == 0 && kDiag % 2 == 0, "an even number of whole key tiles per query tile");
  const int ts = desc ? rr.nt - 1 : max(0, rr.wfull - 1);
  int t = 0;
#pragma nounroll
  for (int pass = 0; pass < 2; ++pass) {
    const int me = pass == 0 ? (desc ? min(kDiag, rr.nt) : 0) : rr.nt;
    for (; t < me; t += 2) {
      static_for<2>([&](auto P) __attribute__((always_inline)) {
        constexpr int q = decltype(P)::value;
        const int tt = t + q;
        if (tt < me) {  // workgroup-uniform: every wave reaches the barrier
          copies(tt, kbuf(q), vbuf(q ^ 1));
          if (tt >= w_lo && tt < w_hi) {
            iteration(tt, kbuf(q ^ 1), vbuf(q), std::true_type{}, std::true_type{}, std::true_type{});
          } else if (tt + 1 == w_lo && rr.wnt > 0) {
            scores(kbuf(q ^ 1), 0, sa);
            scores(kbuf(q ^ 1), 1, sb);
            first_probs(sa, pfa, BC * ktile(tt + 1), std::true_type{});
          }
          sync_after(vbuf(q ^ 1));
        }
      });
    }
    for (; t + 2 <= ts; t += 2) {
      static_for<2>([&](auto P) __attribute__((always_inline)) {
        constexpr int q = decltype(P)::value;
        copies(t + q, kbuf(q), vbuf(q ^ 1));
        iteration(t + q, kbuf(q ^ 1), vbuf(q), std::true_type{}, std::false_type{},
                  std::false_type{});
        sync_after(vbuf(q ^ 1));
      });
    }
  }
  // Every copy has landed and every wave is done with K and V: the buffers
  // now stage O (8 KB per wave for D = 128, two waves per buffer).
  wait_vmem();
  __syncthreads();
  static_assert(NW <= 8 && TB >= 2 * 32 * DV * 2 && TBV >= 2 * 32 * DV * 2, "O staging space");
  unsigned char* stage = (wave < 2 ? k0s : wave < 4 ? k1s : wave < 6 ? v0s : v1s) + (wave & 1) * (32 * DV * 2);
  epilogue_staged<T, DV, DB, D>(p, rr.bh, rr.qw0, lx, m, l, o, stage, vh * DV, vh == 0);
  // staging reads done before the next tile's copies land
  __syncthreads();
  };

  // 16-bit whole batches: the short item streams its key tiles last to
  // first. It then starts on the tiles nearest its diagonal, which the long
  // items of the same head were reading most recently, instead of the head's
  // first tiles, which L2 has dropped by then (head dim 128, N = 8192: 12%
  // fewer bytes fetched for 0.6% of the time). fp8 inputs and packed batches
  // keep the ascending order, which is faster there (0.7% and 1.0%).
  constexpr bool kShortDesc = !F8 && !VL;
  const int items = CAUSAL && u != n_qt - 1 - u ? 2 : 1;
#pragma nounroll
  for (int it = 0; it < items; ++it)
    process(bh, CAUSAL && it == 0 ? n_qt - 1 - u : u, kShortDesc && it == 1);
}

// ---------------------------------------------------------------------------
// fp8 e4m3 kernel, software-pipelined: both products on the fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4), S^T = K Q^T per 32-key half and
// O^T += V^T P^T per 64-key tile (FlashAttention (ES), "FlashAttention-3
// (2024)", names FP8 for the whole fused kernel).
//
// The same workgroup shape, causal folding, XCD-aware order and lazy
// reference maximum as the 16-bit pipelined kernel; what differs:
//   * K and V tiles are both fp8 and both reach LDS through direct-to-LDS
//     copies. The V^T operand of a P V product (one head dimension, 32
//     consecutive keys per lane) comes from four transposing byte reads
//     (ds_read_b64_tr_b8): in each 16-lane group, lane 2j+h addresses key j,
//     head dims 8h..8h+7, and lane i receives head dim i of the 8 keys.
//   * P is rounded to e4m3 as P' = P * 2^4 (the 4 folded into the exponent
//     bias; the product's E8M0 scale 2^-4 undoes it exactly), so P down to
//     2^-10 keeps e4m3's normal precision. The row sum l adds the same rounded
//     P' that multiply V, on the matrix cores: one 16x16x128 product per tile
//     of an e4m3 0/1 matrix with the tile's P^T operand, whose rows 0 and 4
//     select the lane groups of each query, so that the first accumulator
//     register of lane l < 32 is row l's sum (and 0 in lanes 32-63).
//   * The products take a whole tile's P (K = 64 keys), but each lane holds 16
//     keys of each half; one v_permlane32_swap per 4 keys trades halves with
//     lane l^32, after which lane (q, h) holds the 32 keys of half h of query
//     q in order, as the B operand wants.
//   * P of a tile's first half is formed one block before the product; if the
//     second half then moves the row's reference maximum, the move is a whole
//     number n of powers of two and the pending first half's e4m3 values are
//     scaled by 2^-n in place (exact unless they fall below e4m3's normal
//     range; l sums the re-rounded values, as V is multiplied by them).
//
// Per iteration t (K of tile t+1 in kb, V of tile t in vb), block A: the S
// products of tile t+1 with the softmax of tile t's second half; block B:
// the P V products of tile t with the softmax of tile t+1's first half.
// Three score buffers rotate: s1 (tile t, second half), x (tile t+1, first
// half, consumed in block B) and y (tile t+1, second half, next s1).
// ---------------------------------------------------------------------------

// v8_swz: fp8 V rows (D bytes): the 16 rows x 2 slots one transposing read
// touches per 32 lanes land on distinct banks.
template <int D>
__device__ __forceinline__ int v8_swz(int r) {
  if constexpr (D == 128) return ((r >> 1) & 3) << 1;
  return ((r >> 2) & 1) << 1;
}

constexpr int kP8Shift = 4;          // P' = P * 2^4 before rounding to e4m3
constexpr float kP8Bound = 420.0f;  // a lane's half sum of P' above this: rescale

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_pipe8(Params p) {
  using T = __bf16;  // O
  constexpr int BR = NW * 32;   // query rows per workgroup
  constexpr int BC = 64;        // keys per LDS tile
  constexpr int KS = D / 64;    // S MFMA steps over the head dim per half
  constexpr int DB = D / 32;    // 32-wide blocks of O^T (P V products per tile)
  constexpr int TB = BC * D;    // bytes per K or V tile
  constexpr int CPR = D / 16;   // 16-byte slots per row
  constexpr int NC = TB / 1024;  // 1 KB copies per tile
  constexpr int ND = (NC + NW - 1) / NW;  // copies per wave per tile (some idle)
  constexpr int LA = FA_PIPE_LOOKAHEAD > 0 ? FA_PIPE_LOOKAHEAD : 1;
  static_assert(D == 64 || D == 128, "head dim 64 or 128");

  __shared__ __attribute__((aligned(1024))) unsigned char k0s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char k1s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char v0s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char v1s[TB];
  // (the staging array's smaller alignment places it after the tiles, whose
  // addresses then fit the LDS instructions' 16-bit offsets)
  __shared__ __attribute__((aligned(16))) unsigned char ostage[NW * 32 * D * 2];
  // The kernel is at the edge of its 256 registers: with these values in
  // registers it spilled, and scratch reloads in the loop wait on the
  // vector-memory counter, that is on the tile copies in flight. So each
  // wave keeps its lanes' operand-read offsets
  // (koff, voff) and its Q operand in LDS and reads them back where used,
  // indexed by a lane index the compiler cannot hoist (fresh_lane), so that
  // nothing derived from them stays live across the loop. Q is read as
  // 16-byte pieces: a 32-byte LDS load is split without the information that
  // tells its address apart from the copies' destinations, and then waits
  // for every copy.
  __shared__ int ores[NW][2 * KS + DB][64];
  __shared__ i32x4 qres[NW][2 * KS][64];
  auto kbuf = [&](int i) __attribute__((always_inline)) -> unsigned char* { return i == 0 ? k0s : k1s; };
  auto vbuf = [&](int i) __attribute__((always_inline)) -> unsigned char* { return i == 0 ? v0s : v1s; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // Work unit u of head bh, causal query tiles folded in pairs, as in
  // attn_fwd_pipe.
  const int units = CAUSAL ? (p.n_qt + 1) / 2 : p.n_qt;
  int bh, u;
  {
    const int bid = blockIdx.x, total = gridDim.x;
    int logical = bid;
    if (total % kXcds == 0) logical = (bid % kXcds) * (total / kXcds) + bid / kXcds;
    bh = logical / units;
    u = logical - bh * units;
  }
  const int n_qt = p.n_qt;
  const int N = p.N;

  // Q^T operand: lane holds its query row's head dims [64*st + 32*hi, +32).
  i32x8 qf[KS];

  auto process = [&](int qt) __attribute__((always_inline)) {
  const int ln = pinned_int(lane);
  int koff[2 * KS];
#pragma unroll
  for (int st = 0; st < KS; ++st)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      koff[2 * st + x] = (ln & 31) * D + (((4 * st + 2 * (ln >> 5) + x) ^ k8_swz<D>(ln & 31)) << 4);
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) ores[wave][i][lane] = koff[i];
  // V^T operand of P V block db, read q at voff[db] + 8 * q * D: key row
  // 32*(group/2) + 8q + (i/2), head dims 32db + 16*(group%2) + 8*(i%2) + [0, 8).
  int voff[DB];
  {
    const int g = (ln >> 4) & 3, i = ln & 15;
    const int r = 32 * (g >> 1) + (i >> 1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[db] = r * D + (((2 * db + (g & 1)) ^ v8_swz<D>(r)) << 4) + 8 * (i & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) ores[wave][2 * KS + db][lane] = voff[db];
  }
  const RowRange rr = row_range_at<BR, BC, CAUSAL>(p, bh, qt, wave, l32);
  const size_t kv_head = (size_t)rr.kv_bh * N * D;  // bytes
  {
    const auto rq = tile_rsrc((const unsigned char*)p.q + (size_t)rr.bh * N * D, rr.q_wg0 / BR, BR, N, D);
    const int row = rr.qrow - rr.q_wg0;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = row * D + 64 * s + 32 * hi;
      qf[s] = __builtin_shufflevector(load16(rq, off), load16(rq, off + 16), 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qres[wave][2 * s][lane] = __builtin_shufflevector(qf[s], qf[s], 0, 1, 2, 3);
      qres[wave][2 * s + 1][lane] = __builtin_shufflevector(qf[s], qf[s], 4, 5, 6, 7);
    }
  }
  const auto rsK = buffer_rsrc((const unsigned char*)p.k + kv_head, rr.kl * D);
  const auto rsV = buffer_rsrc((const unsigned char*)p.v + kv_head, rr.kl * D);
  // Tile j of K or V straight into LDS, 16-byte slots permuted per row.
  auto copy_tile = [&](int j, unsigned char* dst, auto is_v) __attribute__((always_inline)) {
    constexpr bool IV = decltype(is_v)::value;
#pragma unroll
    for (int cc = 0; cc < ND; ++cc) {
      const int blk = cc * NW + wave;
      if (NC % NW == 0 || blk < NC) {
        const int slot = blk * 64 + lane;
        const int r = slot / CPR, ps = slot % CPR;
        const int lc = ps ^ (IV ? v8_swz<D>(r) : k8_swz<D>(r));
        lds_copy16(IV ? rsV : rsK, dst + blk * 1024, j * TB + r * D + (lc << 4));
      }
    }
  };
  // S^T = K Q^T over keys [32h, 32h + 32) of the K tile at kb
  auto scores = [&](const unsigned char* kb, int h, f32x16& s, int fl) __attribute__((always_inline)) {
    s = f32x16{};
    i32x8 ring[LA + 1];
#pragma unroll
    for (int t = 0; t < KS + LA; ++t) {
      if (t < KS) {
        const unsigned char* b = kb + 32 * h * D;
        const int k0 = ores[wave][2 * t][fl], k1 = ores[wave][2 * t + 1][fl];
        ring[t % (LA + 1)] = __builtin_shufflevector(*(const i32x4*)(b + k0), *(const i32x4*)(b + k1),
                                                     0, 1, 2, 3, 4, 5, 6, 7);
      }
      const int v = t - LA;
      if (v >= 0) {  // formats 0/0: fp8 e4m3 operands; E8M0 scales 127 = 1.0
        const i32x8 q = __builtin_shufflevector(qres[wave][2 * v][fl], qres[wave][2 * v + 1][fl], 0, 1, 2, 3,
                                                4, 5, 6, 7);
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ring[v % (LA + 1)], q, s, 0, 0, 0, 127, 0, 127);
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  // base = -m * c + kP8Shift (+inf while m = -inf): P' = exp2(c * s + base).
  // ls[0] sums the rounded P (the weights V is multiplied by, so O is their
  // normalised combination); lx sums the unrounded P' for the log-sum-exp.
  float m = -INFINITY, base = INFINITY, lx = 0.0f;
  f32x4 ls = {};
  const float c = p.c;
  // e4m3 A operand of the row-sum product (the format of the P^T operand, so
  // that both spread the K dimension over the lanes alike): lane (row r =
  // lane % 16, group g = lane / 16) holds 1.0 (code 0x38) in row 0 for groups
  // 0 and 2 and in row 4 for groups 1 and 3, else 0. The P^T operand's lane
  // group g holds query l % 32 of its lanes: groups 0 and 2 queries 0-15,
  // groups 1 and 3 queries 16-31. Output row 0 (lanes 0-15) is then the sum
  // of queries 0-15, row 4 (lanes 16-31) of queries 16-31, and lanes 32-63
  // hold 0, so summing lanes l and l^32 gives each row's sum once.
  i32x8 sel_a{};
  {
    const int r = lane & 15, g = lane >> 4;
    const int w = (r == 0 && (g & 1) == 0) || (r == 4 && (g & 1) == 1) ? 0x38383838 : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) sel_a[i] = w;
  }

  // P' of one half (16 scores of this lane's row) against `b`, rounded to
  // e4m3 into 4 words; rx gets the sum of the unrounded values.
  auto round_half = [&](const f32x16& s, float b, i32x4& pw, float& rx) __attribute__((always_inline)) {
    rx = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = fast_exp2(fmaf(s[4 * w + e], c, b));
      // (the first conversion's other half is overwritten by the second)
      int d = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], __builtin_bit_cast(int, x[2]), false);
      d = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], d, true);
      pw[w] = d;
      rx += (x[0] + x[1]) + (x[2] + x[3]);
    }
  };
  auto half_max = [&](const f32x16& s) __attribute__((always_inline)) {
    float x = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) x = fmaxf(x, s[i]);
    return max_halves(x);
  };
  // The 4 e4m3 words of a pending half scaled by 2^-n (n >= 0).
  auto rescale_half = [&](i32x4& pw, int n) __attribute__((always_inline)) {
    const float sc = __builtin_ldexpf(1.0f, -n);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(pw[w], false);
      const f32x2 up = __builtin_amdgcn_cvt_pk_f32_fp8(pw[w], true);
      int d = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0] * sc, lo[1] * sc, pw[w], false);
      pw[w] = __builtin_amdgcn_cvt_pk_fp8_f32(up[0] * sc, up[1] * sc, d, true);
    }
  };
  // P' of a half with the reference check. Without a pending half the rare
  // branch moves the reference to the row maximum; with one (pend, the P' of
  // the tile's first half, not yet multiplied) it moves it up by a whole
  // number n of powers of two and scales pend by 2^-n.
  auto probs = [&](f32x16& s, i32x4& pw, int k0, auto masked, auto pending, i32x4& pend)
      __attribute__((always_inline)) {
    if constexpr (FA_PIPE_IGLP >= 0) __builtin_amdgcn_iglp_opt(FA_PIPE_IGLP);
    if constexpr (decltype(masked)::value) {
      auto& s1 = *reinterpret_cast<f32x16(*)[1]>(&s);
      apply_mask<1, CAUSAL>(s1, k0, rr.kl, rr.qrow, hi);
    }
    float rx;
    round_half(s, base, pw, rx);
    if (__builtin_amdgcn_ballot_w64(!(rx <= kP8Bound)) != 0) {
      const float mx = half_max(s);
      float alpha;
      if (decltype(pending)::value && m != -INFINITY) {
        // up by whole powers of two: the reference stays exactly base - steps
        const float steps = fmaxf(0.0f, ceilf((mx - m) * c));
        const int n = (int)fminf(steps, 126.0f);
        alpha = pinned(__builtin_ldexpf(1.0f, -n));
        m += steps / c;
        base -= steps;
        rescale_half(pend, n);
      } else {
        const float mn = fmaxf(m, mx);
        alpha = pinned(mn == m ? 1.0f : fast_exp2((m - mn) * c));  // exp2(-inf) = 0
        m = mn;
        base = fmaf(-mn, c, (float)kP8Shift);  // +inf while the row has no key
      }
      lx *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) ls[i] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      round_half(s, m == -INFINITY ? 0.0f : base, pw, rx);
    }
    lx += rx;
  };
  // O^T += V^T P^T over the tile in vb: p0, p1 the rounded P' of its halves.
  auto pv = [&](const unsigned char* vb, const i32x4& p0, const i32x4& p1, int fl)
      __attribute__((always_inline)) {
    i32x8 b;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x2 r = __builtin_amdgcn_permlane32_swap((unsigned)p0[w], (unsigned)p1[w], false, false);
      b[2 * w] = (int)r[0];
      b[2 * w + 1] = (int)r[1];
    }
    constexpr int sb = 127 - kP8Shift;  // E8M0 2^-4 undoes P' = P * 2^4
    // row sums (formats 0/0: e4m3 A and B)
    ls = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel_a, b, ls, 0, 0, 0, 127, 0, sb);
    i32x8 ring[LA + 1];
#pragma unroll
    for (int t = 0; t < DB + LA; ++t) {
      if (t < DB) {
        const unsigned char* a = vb + ores[wave][2 * KS + t][fl];
        i32x8 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const auto rq = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2*)(a + 8 * q * D));
          v[2 * q] = rq[0];
          v[2 * q + 1] = rq[1];
        }
        ring[t % (LA + 1)] = v;
      }
      const int v = t - LA;
      if (v >= 0)
        o[v] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ring[v % (LA + 1)], b, o[v], 0, 0, 0,
                                                               127, 0, sb);
    }
  };

  f32x16 sA, sB, sC;
  i32x4 p0, p1;
  // One iteration with score buffers s1 (tile t, second half), x, y (tile
  // t+1): block A, then block B.
  auto iteration = [&](int t, const unsigned char* kb, const unsigned char* vb, f32x16& s1,
                       f32x16& x, f32x16& y, auto has_next, auto mask_a, auto mask_b)
      __attribute__((always_inline)) {
    constexpr bool HN = decltype(has_next)::value;
    const int fl = fresh_lane();  // this iteration's lane index (not held across iterations)
    if constexpr (HN) {
      scores(kb, 0, x, fl);
      scores(kb, 1, y, fl);
    }
    probs(s1, p1, BC * t + 32, mask_a, std::true_type{}, p0);
    pv(vb, p0, p1, fl);
    if constexpr (HN) probs(x, p0, BC * (t + 1), mask_b, std::false_type{}, p1);
  };
  auto copies = [&](int t, unsigned char* kx, unsigned char* vx) __attribute__((always_inline)) {
    copy_tile(t + 2, kx, std::false_type{});
    copy_tile(t + 1, vx, std::true_type{});
  };
  auto sync_after = [&]() __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
  };

  copy_tile(0, k0s, std::false_type{});
  copy_tile(1, k1s, std::false_type{});
  copy_tile(0, v0s, std::true_type{});
  wait_vmem();
  __syncthreads();
  if (rr.wnt > 0) {
    const int fl = fresh_lane();
    scores(k0s, 0, sB, fl);
    scores(k0s, 1, sA, fl);
    if (0 < rr.wfull) probs(sB, p0, 0, std::false_type{}, std::false_type{}, p1);
    else probs(sB, p0, 0, std::true_type{}, std::false_type{}, p1);
  }
  __syncthreads();  // K of tile 0 is read by every wave before its buffer is refilled
  // Iterations [0, ts): unmasked with a next tile, two per pass (the K/V
  // buffers alternate, and so do the roles of sA and sC).
  const int ts = max(0, rr.wfull - 1);
  int t = 0;
  for (; t + 2 <= ts; t += 2) {
    copies(t, k0s, v1s);
    iteration(t, k1s, v0s, sA, sB, sC, std::true_type{}, std::false_type{}, std::false_type{});
    sync_after();
    copies(t + 1, k1s, v0s);
    iteration(t + 1, k0s, v1s, sC, sB, sA, std::true_type{}, std::false_type{}, std::false_type{});
    sync_after();
  }
  // The rest as in attn_fwd_pipe: one variant with every mask applied and
  // the next tile always scored (past the wave's last tile its keys are all
  // masked), unrolled over the two buffer parities (t is even here) with the
  // score buffers rotating as in the pass above.
  for (; t < rr.nt; t += 2) {
    if (t < rr.nt) {  // workgroup-uniform
      copies(t, k0s, v1s);
      if (t < rr.wnt)
        iteration(t, k1s, v0s, sA, sB, sC, std::true_type{}, std::true_type{}, std::true_type{});
      sync_after();
    }
    if (t + 1 < rr.nt) {
      copies(t + 1, k1s, v0s);
      if (t + 1 < rr.wnt)
        iteration(t + 1, k0s, v1s, sC, sB, sA, std::true_type{}, std::true_type{}, std::true_type{});
      sync_after();
    }
  }
  // O / l through this wave's own staging slice (K/V buffers stay free);
  // LSE from the unrounded sum
  epilogue_staged<T, D, DB>(p, rr.bh, rr.qw0, lane, (kP8Shift - base) / c, ls[0], o,
                            ostage + wave * (32 * D * 2), 0, true,
                            lx * (1.0f / (1 << kP8Shift)));
  __syncthreads();  // every wave is past the K/V buffers before the next item's copies
  };

  const int items = CAUSAL && u != n_qt - 1 - u ? 2 : 1;
#pragma nounroll
  for (int it = 0; it < items; ++it) process(CAUSAL && it == 0 ? n_qt - 1 - u : u);
}

// ---------------------------------------------------------------------------
// fp8 e4m3 kernel: S^T on the fp8 matrix cores (32x32x64), P V in bf16.
// V's fp8 codes are widened to bf16 exactly when staged into LDS (every e4m3
// value is a bf16 value), and P is rounded to bf16 as in the bf16 kernel.
// ---------------------------------------------------------------------------

template <int D, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, FA_WAVES_PER_EU) void attn_fwd_fp8(Params p) {
  using E = Bf16;
  using T8 = unsigned char;
  constexpr int BR = NW * 32;
  constexpr int KS = D / 64;   // 64-wide reduction steps in S^T
  constexpr int SB = BC / 32;
  constexpr int DB = D / 32;
  constexpr int KST = D + 16;  // bytes per K row in LDS
  constexpr int VST = D + FA_V_SKEW;  // bf16 elements per V row in LDS
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 16;  // 16-byte (16-code) chunks per row
  constexpr int CH = (BC * CPR + NT - 1) / NT;  // 16-byte chunks per thread per tile
  constexpr bool kRagged = BC * CPR % NT != 0;  // the last chunk slot is idle on some threads

  __shared__ __attribute__((aligned(16))) T8 ks[2][BC * KST];
  __shared__ __attribute__((aligned(16))) __bf16 vs[2][BC * VST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const RowRange rr = row_range<BR, BC, CAUSAL>(p, wave, l32);
  const int N = p.N;
  const size_t head = (size_t)rr.bh * N * D, kv_head = (size_t)rr.kv_bh * N * D;
  const T8* Kh = (const T8*)p.k + kv_head;
  const T8* Vh = (const T8*)p.v + kv_head;

  // Q^T operand: lane holds query row qrow, head-dim 64*s + 32*hi .. +31.
  i32x8 qf[KS];
  {
    const auto rq = tile_rsrc((const T8*)p.q + head, rr.q_wg0 / BR, BR, N, D);
    const int off = (rr.qrow - rr.q_wg0) * D + 32 * hi;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const i32x4 a = load16(rq, off + 64 * s);
      const i32x4 b = load16(rq, off + 64 * s + 16);
      qf[s] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.0f;
  const float thr = fminf(kRescaleLog2 / p.c, 1e30f);  // finite even for tiny scales

  const int kv_lim = rr.kl;
  i32x4 kreg[CH], vreg[CH];
  auto gload = [&](int j) __attribute__((always_inline)) {
    const auto rk = tile_rsrc(Kh, j, BC, kv_lim, D);
    const auto rv = tile_rsrc(Vh, j, BC, kv_lim, D);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int chunk = tid + c * NT;
      if (kRagged && chunk >= BC * CPR) continue;
      const int off = (chunk / CPR) * D + (chunk % CPR) * 16;
      kreg[c] = load16(rk, off);
      vreg[c] = load16(rv, off);
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int chunk = tid + c * NT;
      const int r = chunk / CPR, col = (chunk % CPR) * 16;
      if (kRagged && chunk >= BC * CPR) continue;
      *(i32x4*)(&ks[buf][r * KST + col]) = kreg[c];
      i32x4 w0, w1;
      u32x2 t;
      t = fp8x4_to_bf16x4((unsigned)vreg[c][0]); w0[0] = t[0]; w0[1] = t[1];
      t = fp8x4_to_bf16x4((unsigned)vreg[c][1]); w0[2] = t[0]; w0[3] = t[1];
      t = fp8x4_to_bf16x4((unsigned)vreg[c][2]); w1[0] = t[0]; w1[1] = t[1];
      t = fp8x4_to_bf16x4((unsigned)vreg[c][3]); w1[2] = t[0]; w1[3] = t[1];
      *(i32x4*)(&vs[buf][r * VST + col]) = w0;
      *(i32x4*)(&vs[buf][r * VST + col + 8]) = w1;
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int j = 0; j < rr.nt; ++j) {
    const int buf = j & 1;
    gload(j + 1);
    auto tile = [&](auto masked) __attribute__((always_inline)) {
      const T8* kt = ks[buf];
      f32x16 s[SB];
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        s[sb] = f32x16{};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const T8* ka = kt + (32 * sb + l32) * KST + 64 * st + 32 * hi;
          const i32x4 a0 = *(const i32x4*)ka;
          const i32x4 a1 = *(const i32x4*)(ka + 16);
          const i32x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
          // formats 0/0 = fp8 e4m3 for both operands; E8M0 scales 127 = 1.0
          s[sb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[st], s[sb], 0, 0, 0, 127,
                                                                  0, 127);
        }
      }
      if constexpr (decltype(masked)::value) apply_mask<SB, CAUSAL>(s, j * BC, rr.kl, rr.qrow, hi);
      bf16x8 pf[SB * 2];
      online_softmax<E, SB, DB>(s, p.c, thr, m, l, o, pf);
      pv_product<E, SB, DB, VST>(vs[buf], lane, pf, o);
    };
    if (j < rr.wfull) tile(std::false_type{});
    else if (j < rr.wnt) tile(std::true_type{});
    sstore(buf ^ 1);
    __syncthreads();
  }
  epilogue<__bf16, D, DB>(p, rr, hi, m, l, o);
}

// ---------------------------------------------------------------------------
// fp32 kernel: both products on v_mfma_f32_32x32x2_f32 (full fp32 inputs, no
// reduced-precision operand path), P kept in fp32.
// ---------------------------------------------------------------------------
template <int D, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_f32(Params p) {
  constexpr int BR = NW * 32;
  constexpr int KS = D / 2;
  constexpr int SB = BC / 32;
  constexpr int DB = D / 32;
  constexpr int KST = D + 1;  // odd stride: the 32 rows read per step hit 32 banks
  constexpr int VST = D + 4;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 4;
  constexpr int CH = (BC * CPR + NT - 1) / NT;  // 16-byte chunks per thread per tile
  constexpr bool kRagged = BC * CPR % NT != 0;  // the last chunk slot is idle on some threads

  __shared__ __attribute__((aligned(16))) float ks[2][BC * KST];
  __shared__ __attribute__((aligned(16))) float vs[2][BC * VST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const RowRange rr = row_range<BR, BC, CAUSAL>(p, wave, l32);
  const int N = p.N;
  const size_t head = (size_t)rr.bh * N * D, kv_head = (size_t)rr.kv_bh * N * D;
  const float* Kh = (const float*)p.k + kv_head;
  const float* Vh = (const float*)p.v + kv_head;

  // Q^T operand: lane holds Q[qrow][2*s + hi]
  float qf[KS];
  {
    const auto rq = tile_rsrc((const float*)p.q + head, rr.q_wg0 / BR, BR, N, D * 4);
    const int off = ((rr.qrow - rr.q_wg0) * D + hi) * 4;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rq, off + 8 * s, 0, 0));
  }
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.0f;

  const int kv_lim = rr.kl;
  i32x4 kreg[CH], vreg[CH];
  auto gload = [&](int j) __attribute__((always_inline)) {
    const auto rk = tile_rsrc(Kh, j, BC, kv_lim, D * 4);
    const auto rv = tile_rsrc(Vh, j, BC, kv_lim, D * 4);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int chunk = tid + c * NT;
      if (kRagged && chunk >= BC * CPR) continue;
      const int off = ((chunk / CPR) * D + (chunk % CPR) * 4) * 4;
      kreg[c] = load16(rk, off);
      vreg[c] = load16(rv, off);
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int chunk = tid + c * NT;
      const int r = chunk / CPR, col = (chunk % CPR) * 4;
      if (kRagged && chunk >= BC * CPR) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) ks[buf][r * KST + col + e] = __int_as_float(kreg[c][e]);
      *(i32x4*)(&vs[buf][r * VST + col]) = vreg[c];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int j = 0; j < rr.nt; ++j) {
    const int buf = j & 1;
    gload(j + 1);
    if (j < rr.wnt) {
      const float* kt = ks[buf];
      const float* vt = vs[buf];
      f32x16 s[SB];
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        s[sb] = f32x16{};
#pragma unroll
        for (int st = 0; st < KS; ++st)
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[(32 * sb + l32) * KST + 2 * st + hi],
                                                       qf[st], s[sb], 0, 0, 0);
      }
      const int k0 = j * BC;
      if (k0 + BC > rr.kl || (CAUSAL && k0 + BC - 1 > rr.qw0))
        apply_mask<SB, CAUSAL>(s, k0, rr.kl, rr.qrow, hi);
      float mx = s[0][0];
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
      mx = max_halves(mx);
      const float m_new = fmaxf(m, mx);
      if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
        const float alpha = pinned((m_new > m) ? fast_exp2((m - m_new) * p.c) : 1.0f);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
      m = m_new;
      const float base = (m == -INFINITY) ? 0.0f : -m * p.c;
      float rs = 0.0f;
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[sb][i] = fast_exp2(fmaf(s[sb][i], p.c, base));
          rs += s[sb][i];
        }
      l += rs;
      // O^T += V^T P^T, one key per lane half per step, keys in accumulator order
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = acc_row(sb, i, hi);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[key * VST + 32 * db + l32], s[sb][i],
                                                         o[db], 0, 0, 0);
        }
    }
    sstore(buf ^ 1);
    __syncthreads();
  }
  epilogue<float, D, DB>(p, rr, hi, m, l, o);
}

// ---------------------------------------------------------------------------
// Decode against a key/value cache: few queries, long key sequences
//
// Split over keys: every wave owns one (K/V head, 32-row block, key chunk)
// unit, where the rows are the group's query heads times the Nq queries
// (row r: query head g * group + r / Nq, query r % Nq) and the chunk is a run
// of 32-key tiles. It streams its tiles once from HBM (K straight into the
// MFMA operand registers, V through a private LDS slice for the transposing
// reads), keeps the online softmax of its rows, and writes the normalised
// partial O and its LSE to the workspace. attn_decode_merge then combines a
// row's chunks: LSE = log sum exp(LSE_s), O = sum exp(LSE_s - LSE) O_s. The
// waves of a workgroup share nothing, so a wave without a unit just exits.
// ---------------------------------------------------------------------------
constexpr int kDecodeWaves = 4;

template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kDecodeWaves * 64, 2) void attn_decode_split(DecodeParams p) {
  using T = typename E::T;
  using v8 = typename E::v8;
  constexpr int KS = D / 16;            // S MFMA steps over the head dim
  constexpr int DB = D / 32;            // 32-wide head-dim blocks of O^T
  constexpr int RB = D * 2;             // bytes per K / V row
  constexpr int VST = D + FA_V_SKEW;    // V row stride in LDS (elements)
  constexpr int CPR = D / 8;            // 16-byte pieces per row
  constexpr int VCH = 32 * CPR / 64;    // V pieces per lane per 32-key tile
  __shared__ __attribute__((aligned(16))) T vs[kDecodeWaves][32 * VST];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kDecodeWaves + wave;
  if (unit >= p.units) return;
  const int chunk = unit % p.S;
  const int rest = unit / p.S;
  const int rb = rest % p.n_rb;
  const int kvh = rest / p.n_rb;  // b * H_kv + g
  const int b = kvh / p.H_kv, g = kvh - b * p.H_kv;
  const int l32 = lane & 31, hi = lane >> 5;
  const int r = rb * 32 + l32;
  const bool row_ok = r < p.R;
  const int hq = g * p.group + (row_ok ? r / p.Nq : 0);
  const int qi = row_ok ? r % p.Nq : 0;
  const size_t qrow = ((size_t)b * p.H + hq) * p.Nq + qi;  // row of Q, O and LSE

  int kl = p.Nk;
  if (p.key_len != nullptr) {
    const int x = p.key_len[b];
    kl = x < 0 ? 0 : (x > p.Nk ? p.Nk : x);
  }
  kl = __builtin_amdgcn_readfirstlane(kl);
  const int nt = (kl + 31) / 32;
  const int t0 = chunk * p.chunk_tiles;
  const int t1 = min(nt, t0 + p.chunk_tiles);
  const int pos = kl - p.Nq + qi;  // the query's position: causal keys j <= pos

  // Q^T operand: lane holds its row's head-dim elements [16*st + 8*hi, +8).
  v8 qf[KS];
  {
    const T* qr = (const T*)p.q + qrow * D;
#pragma unroll
    for (int st = 0; st < KS; ++st) qf[st] = row_ok ? *(const v8*)(qr + 16 * st + 8 * hi) : v8{};
  }
  // K / V of the K/V head over its first kl rows: rows beyond read as zeros.
  const size_t kv_off = (size_t)kvh * p.Nk * RB;
  const auto rsK = buffer_rsrc((const unsigned char*)p.k + kv_off, kl * RB);
  const auto rsV = buffer_rsrc((const unsigned char*)p.v + kv_off, kl * RB);
  i32x4 kr[KS], vr[VCH];
  auto load = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < KS; ++st) kr[st] = load16(rsK, (32 * t + l32) * RB + 32 * st + 16 * hi);
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int pc = lane + 64 * c;
      vr[c] = load16(rsV, (32 * t + pc / CPR) * RB + 16 * (pc % CPR));
    }
  };
  T* vt = vs[wave];

  const float c = p.c;
  const float thr = fminf(kRescaleLog2 / c, 1e30f);
  float m = -INFINITY, l = 0.0f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};

  if (t0 < t1) load(t0);
  for (int t = t0; t < t1; ++t) {
    f32x16 sc[1] = {f32x16{}};
#pragma unroll
    for (int st = 0; st < KS; ++st) sc[0] = E::mma(__builtin_bit_cast(v8, kr[st]), qf[st], sc[0]);
    // V of tile t into this wave's slice; the previous tile's reads of it
    // were issued earlier by this wave, and LDS serves a wave in order.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int cc = 0; cc < VCH; ++cc) {
      const int pc = lane + 64 * cc;
      *(i32x4*)(vt + (pc / CPR) * VST + 8 * (pc % CPR)) = vr[cc];
    }
    if (t + 1 < t1) load(t + 1);
    if (CAUSAL || 32 * (t + 1) > kl) apply_mask<1, CAUSAL>(sc, 32 * t, kl, pos, hi);
    v8 pf[2];
    online_softmax<E, 1, DB>(sc, c, thr, m, l, o, pf);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the V slice is written
    __builtin_amdgcn_wave_barrier();
    pv_product<E, 1, DB, VST>(vt, lane, pf, o);
  }

  const float lt = sum_halves(l);
  const bool live = lt > 0.0f;
  const float inv = live ? 1.0f / lt : 0.0f;
  if (row_ok) {
    float* wo = p.ws_o + (qrow * p.S + chunk) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = o[db][4 * gq + e] * inv;
        *(f32x4*)(wo + 32 * db + 8 * gq + 4 * hi) = x;
      }
    if (hi == 0) p.ws_lse[qrow * p.S + chunk] = live ? m * p.scale_eff + logf(lt) : -INFINITY;
  }
}

// One wave per query row: combine its S partial results.
template <class OutT, int D>
__global__ __launch_bounds__(64) void attn_decode_merge(DecodeParams p) {
  constexpr int E = D / 64;  // head-dim elements per lane
  const size_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const float* ls = p.ws_lse + row * p.S;
  float mx = -INFINITY;
  for (int s = lane; s < p.S; s += 64) mx = fmaxf(mx, ls[s]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) mx = fmaxf(mx, __shfl_xor(mx, w, 64));
  float acc[E] = {};
  float L = 0.0f;
  if (mx > -INFINITY) {
    const float* wo = p.ws_o + row * p.S * D;
    // unrolled so that several chunks' loads are in flight at once
#pragma unroll 4
    for (int s = 0; s < p.S; ++s) {
      const float w = expf(ls[s] - mx);  // 0 for an empty chunk
      L += w;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(w, wo[(size_t)s * D + lane + 64 * e], acc[e]);
    }
  }
  const float inv = L > 0.0f ? p.o_scale / L : 0.0f;
  OutT* out = (OutT*)p.o + row * D;
#pragma unroll
  for (int e = 0; e < E; ++e) out[lane + 64 * e] = (OutT)(acc[e] * inv);
  if (lane == 0) p.lse[row] = L > 0.0f ? mx + logf(L) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Backward: dQ, dK, dV by recomputing P from the forward's LSE
//
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),  Delta = rowsum(dO * O),
//   dQ = scale * dS K,  dK = scale * dS^T Q,  P = exp2(c*s - LSE*log2(e)).
// Two passes on one stream: attn_bwd_dq_dma gives every wave 32 query rows
// and streams the 32-key K/V tiles (the forward's orientation: lanes own
// queries, so LSE and Delta are per-lane values; it computes Delta and
// LSE*log2(e) of its rows and stores them for the next pass);
// attn_bwd_dkdv_dma gives every wave 32 keys and
// streams 32-query Q/dO tiles over the query heads that share its K/V head
// (lanes own keys, so dK and dV accumulate with no cross-wave reduction and
// no atomics). Both recompute S; products whose second operand comes out of
// an accumulator (dQ from dS^T, dV from P, dK from dS) read that tile with
// the forward's transposing LDS reads (tr_product).
// ---------------------------------------------------------------------------
#ifndef FA_BWD_KV_OCC
#define FA_BWD_KV_OCC 2  // waves per SIMD the dK/dV pass is compiled for (1: 512 registers)
#endif
#ifndef FA_BWD_KV_SUB
#define FA_BWD_KV_SUB 2  // dK/dV pass: 32-row query tiles per iteration (1: three buffers, 2: two)
#endif
#ifndef FA_BWD_LOOKAHEAD
#define FA_BWD_LOOKAHEAD 2  // backward passes: LDS operand reads issued this many MFMAs ahead
#endif
#ifndef FA_BWD_WAVES
#define FA_BWD_WAVES 4  // waves per workgroup of the backward passes
#endif
// The backward passes' work units in the order they are numbered (head by
// head, longest first), dealt so that each XCD owns consecutive units: the
// workgroups running together on an XCD then share their heads' tiles in its
// L2, as in the forward kernels.
__device__ __forceinline__ int bwd_block() {
  const int bid = blockIdx.x, total = gridDim.x;
  return total % kXcds == 0 ? (bid % kXcds) * (total / kXcds) + bid / kXcds : bid;
}

constexpr int kBwdWaves = FA_BWD_WAVES;    // waves per workgroup
constexpr int kBwdRows = kBwdWaves * 32;   // query rows (dQ) or keys (dK/dV) per workgroup

// The row's 16 accumulator values scaled and written as 4-element runs: lane
// owns column `col` of the D-layout tile, rows are the head-dim elements.
template <class T, int DB>
__device__ __forceinline__ void store_grad(T* row_ptr, int hi, float scale, const f32x16 (&a)[DB]) {
  typedef T v4t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v4t out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (T)(a[db][4 * g + e] * scale);
      *(v4t*)(row_ptr + 32 * db + 8 * g + 4 * hi) = out;
    }
}

// ---------------------------------------------------------------------------
// The streamed 32-row tiles of both passes reach LDS through buffer_load ...
// lds (no staging registers): four buffers in the dQ pass (a tile's copy is
// issued three iterations before its dQ product and two before its S and dP
// products), two buffers of two tiles in the dK/dV pass (one iteration
// ahead). Every tile is stored with the V-operand slot permutation (v_swz):
// transposing reads use it as the forward's V reads do, and row reads (the A
// operands of S and dP) look their 16-byte slot up through the same
// permutation.
// ---------------------------------------------------------------------------

template <int D>
struct SwzTile {
  static constexpr int RB = D * 2, CPR = D / 8, DB = D / 32;
  int voff[DB];  // this lane's transposing-read offsets (as the forward's V reads)
  int roff;      // this lane's row-read base: row l32
  int sw;        // v_swz of this lane's row
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int r = 4 * (g >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 4 * db + 2 * (g & 1) + ((i & 3) >> 1);
      voff[db] = r * RB + ((c ^ v_swz<D>(r)) << 4) + 8 * (i & 1);
    }
    roff = (lane & 31) * RB;
    sw = v_swz<D>(lane & 31);
  }
  // 16 bytes of row l32, logical slot c
  __device__ __forceinline__ int row(int c) const { return roff + ((c ^ sw) << 4); }
};

// acc^T[n][col] += sum_k Y[k][n] * M[k][col] over the 32 rows k of a swizzled
// tile Y, M given as the packed 16-bit operand of a D-layout accumulator.
template <class E, int D>
__device__ __forceinline__ void tr_product(const unsigned char* tile, const SwzTile<D>& sz,
                                           const typename E::v8 (&m)[2], f32x16 (&acc)[D / 32]) {
  using v4 = typename E::v4;
  using v8 = typename E::v8;
  constexpr int DB = D / 32, RB = D * 2, LA = FA_BWD_LOOKAHEAD;
  v8 ring[LA + 1];
#pragma unroll
  for (int t = 0; t < 2 * DB + LA; ++t) {
    if (t < 2 * DB) {
      const unsigned char* b = tile + 16 * (t / DB) * RB + sz.voff[t % DB];
      const v4 a0 = __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)b));
      const v4 a1 = __builtin_bit_cast(
          v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(b + 8 * RB)));
      ring[t % (LA + 1)] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const int u = t - LA;
    if (u >= 0) acc[u % DB] = E::mma(ring[u % (LA + 1)], m[u / DB], acc[u % DB]);
  }
}

// S = X Y^T and dP = Z W^T over the head dim for one 32-row tile: X, Z rows
// of swizzled LDS tiles (A operands), Y, W in registers (B operands); operand
// reads issued FA_BWD_LOOKAHEAD steps ahead.
template <class E, int D>
__device__ __forceinline__ void two_products(const unsigned char* x, const unsigned char* z,
                                             const SwzTile<D>& sz, int hi,
                                             const typename E::v8 (&y)[D / 16],
                                             const typename E::v8 (&w)[D / 16], f32x16& s,
                                             f32x16& dp) {
  using v8 = typename E::v8;
  constexpr int KS = D / 16, LA = FA_BWD_LOOKAHEAD;
  v8 ra[LA + 1], rb[LA + 1];
#pragma unroll
  for (int t = 0; t < KS + LA; ++t) {
    if (t < KS) {
      ra[t % (LA + 1)] = *(const v8*)(x + sz.row(2 * t + hi));
      rb[t % (LA + 1)] = *(const v8*)(z + sz.row(2 * t + hi));
    }
    const int u = t - LA;
    if (u >= 0) {
      s = E::mma(ra[u % (LA + 1)], y[u], s);
      dp = E::mma(rb[u % (LA + 1)], w[u], dp);
    }
  }
}

// Rows [32*t, 32*t + 32) of a head (cut at `limit` rows) into `dst`, slots
// permuted by v_swz; each wave copies its share of the 1 KB blocks.
template <int D>
__device__ __forceinline__ void copy_rows_swz(const void* head, int t, int limit, unsigned char* dst,
                                              int wave, int lane) {
  constexpr int RB = D * 2, CPR = D / 8, NCP = 32 * RB / 1024;
  static_assert(NCP % kBwdWaves == 0, "1 KB copies split evenly over the waves");
  const auto rs = tile_rsrc(head, t, 32, limit, RB);
#pragma unroll
  for (int c = 0; c < NCP / kBwdWaves; ++c) {
    const int blk = c * kBwdWaves + wave;
    const int slot = blk * 64 + lane;
    const int r = slot / CPR, ps = slot % CPR;
    lds_copy16(rs, dst + blk * 1024, r * RB + ((ps ^ v_swz<D>(r)) << 4));
  }
}

template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64, 2) void attn_bwd_dq_dma(BwdParams p) {
  using T = typename E::T;
  using v8 = typename E::v8;
  constexpr int KS = D / 16, DB = D / 32, TB = 32 * D * 2;
  constexpr int NCPW = TB / 1024 / kBwdWaves;  // copies per wave per tile and tensor
  constexpr int NB = 4;  // K / V buffers: tile j + 3 is copied while j and j + 1 are read
  // One named array per buffer: distinct objects let the compiler see that
  // the copies in flight into one buffer cannot alias the operand reads from
  // another, so those reads do not wait for the copies to land.
  __shared__ __attribute__((aligned(1024))) unsigned char k0s[TB], k1s[TB], k2s[TB], k3s[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char v0s[TB], v1s[TB], v2s[TB], v3s[TB];
  static_assert(NB == 4, "four named buffers per operand");
  auto kb = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? k0s : i == 1 ? k1s : i == 2 ? k2s : k3s;
  };
  auto vb = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? v0s : i == 1 ? v1s : i == 2 ? v2s : v3s;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int N = p.N;
  const int bid = bwd_block();
  const int bh = bid / p.n_qt;
  const int qt = p.n_qt - 1 - (bid - bh * p.n_qt);
  const int b = bh / p.H, kvh = b * p.H_kv + (bh - b * p.H) / p.group;
  int kl = N;
  if (p.key_len != nullptr) {
    const int x = p.key_len[b];
    kl = x < 0 ? 0 : (x > N ? N : x);
  }
  kl = __builtin_amdgcn_readfirstlane(kl);
  const int q_wg0 = qt * kBwdRows, qw0 = q_wg0 + 32 * wave, qrow = qw0 + l32;
  int kv_end = kl;
  if (CAUSAL) kv_end = min(kv_end, min(N, q_wg0 + kBwdRows));
  const int nt = (kv_end + 31) / 32;
  int w_end = CAUSAL ? min(kv_end, qw0 + 32) : kv_end;
  if (qw0 >= N) w_end = 0;
  const int wnt = (w_end + 31) / 32;
  int wfull = kl / 32;
  if (CAUSAL) wfull = min(wfull, (qw0 + 1) / 32);
  wfull = min(wfull, wnt);

  const size_t head = (size_t)bh * N * D, kv_head = (size_t)kvh * N * D;
  const T* Kh = (const T*)p.k + kv_head;
  const T* Vh = (const T*)p.v + kv_head;
  v8 qf[KS], df[KS];
  {
    const auto rq = tile_rsrc((const T*)p.q + head, 0, N, N, D * 2);
    const auto rd = tile_rsrc((const T*)p.dout + head, 0, N, N, D * 2);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      qf[st] = __builtin_bit_cast(v8, load16(rq, qrow * D * 2 + 32 * st + 16 * hi));
      df[st] = __builtin_bit_cast(v8, load16(rd, qrow * D * 2 + 32 * st + 16 * hi));
    }
  }
  const bool row_ok = qrow < N;
  // Delta = rowsum(dO * O) and LSE * log2 e of this lane's query row: the
  // lane and its partner l ^ 32 hold the two halves of the row's dO, so each
  // reads the same half of O, and the two partial sums meet in one lane
  // exchange. Both are stored for the dK/dV pass (which runs after this one);
  // rows at or past N read as zeros and are not stored.
  float dl = 0.0f, lse2 = INFINITY;
  {
    const auto ro = tile_rsrc((const T*)p.o + head, 0, N, N, D * 2);
    float acc = 0.0f;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const v8 of = __builtin_bit_cast(v8, load16(ro, qrow * D * 2 + 32 * st + 16 * hi));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)df[st][e], (float)of[e], acc);
    }
    dl = sum_halves(acc);
    if (row_ok) {
      const float L = p.lse[(size_t)bh * N + qrow];
      lse2 = L == -INFINITY ? INFINITY : L * 1.4426950408889634f;
      if (hi == 0) {
        p.delta[(size_t)bh * N + qrow] = dl;
        p.lse2[(size_t)bh * N + qrow] = lse2;
      }
    }
  }
  const float c = p.c;
  SwzTile<D> sz;
  sz.init(pinned_int(lane));

  auto copies = [&](int j, int buf) __attribute__((always_inline)) {
    copy_rows_swz<D>(Kh, j, kv_end, kb(buf), wave, lane);
    copy_rows_swz<D>(Vh, j, kv_end, vb(buf), wave, lane);
  };
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};
  copies(0, 0);
  copies(1, 1);
  copies(2, 2);
  wait_vmem_keep<2 * NCPW>();  // tiles 0 and 1 landed (tile 2 may be in flight)
  __syncthreads();
  // Software pipeline over the key tiles: iteration j issues the S and dP
  // products of tile j + 1 in the same basic block as the softmax of tile j
  // and its dQ product, so the matrix cores have work while the vector ALU
  // forms dS. Tile j + 1's products are computed even where this wave will
  // not use them (past its last tile, or past nt): they only read LDS, and
  // their results are dropped. Tiles this wave does not need (j >= wnt) are
  // fully masked (the causal bound or key_len), so they add exact zeros to dQ.
  // The loop is unrolled over the four buffers: buffer indices and LDS
  // addresses are compile-time, and the S / dP registers of consecutive tiles
  // alternate between two sets (sp[j % 2], dpp[j % 2]) with no copies.
  f32x16 sp[2][1] = {{f32x16{}}, {f32x16{}}}, dpp[2] = {f32x16{}, f32x16{}};
  two_products<E, D>(kb(0), vb(0), sz, hi, qf, df, sp[0][0], dpp[0]);
  auto tile = [&](int j, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value, nb1 = (buf + 1) % NB, x = buf & 1;
    f32x16 (&s)[1] = sp[x];
    const f32x16& dp = dpp[x];
    if (j >= wfull) apply_mask<1, CAUSAL>(s, 32 * j, kl, qrow, hi);
    sp[x ^ 1][0] = f32x16{};
    dpp[x ^ 1] = f32x16{};
    two_products<E, D>(kb(nb1), vb(nb1), sz, hi, qf, df, sp[x ^ 1][0], dpp[x ^ 1]);
    v8 ds[2];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * ps + e;
        const float pr = fast_exp2(fmaf(s[0][i], c, -lse2));
        ds[ps][e] = E::cvt(pr * (dp[i] - dl));
      }
    tr_product<E, D>(kb(buf), sz, ds, dq);
  };
  for (int j0 = 0; j0 < nt; j0 += NB) {
    static_for<NB>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      const int j = j0 + q;
      if (j < nt) {  // workgroup-uniform: the barrier below is reached by every wave
        copies(j + 3, (q + 3) % NB);  // past the end: empty ranges, nothing moves
        if (j < wnt) tile(j, qc);
        wait_vmem_keep<2 * NCPW>();  // tile j+2 landed; tile j+3 may be in flight
        __syncthreads();
      }
    });
  }
  wait_vmem();
  if (row_ok) store_grad<T, DB>((T*)p.dq + head + (size_t)qrow * D, hi, p.scale, dq);
}

template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64, FA_BWD_KV_OCC) void attn_bwd_dkdv_dma(BwdParams p) {
  using T = typename E::T;
  using v8 = typename E::v8;
  // An iteration takes SUB query tiles of 32 rows (one barrier, one set of
  // copies and one cursor step for all of them); NB buffers of SUB tiles.
  constexpr int SUB = FA_BWD_KV_SUB, NB = SUB == 1 ? 3 : 2, AHEAD = NB - 1;
  constexpr int KS = D / 16, DB = D / 32, TB = 32 * D * 2;
  constexpr int NCPW = TB / 1024 / kBwdWaves;  // 1 KB copies per wave per 32-row tile and tensor
  static_assert(SUB == 1 || SUB == 2, "one or two 32-row query tiles per iteration");
  // One named array per buffer (the third only when NB = 3): distinct
  // objects let the compiler see that the copies in flight into one buffer
  // cannot alias the reads from another, so those reads do not wait for them.
  constexpr int QB3 = NB > 2 ? SUB * TB : 16, LS3 = NB > 2 ? 64 : 4;
  __shared__ __attribute__((aligned(1024))) unsigned char q0s[SUB * TB], q1s[SUB * TB], q2s[QB3];
  __shared__ __attribute__((aligned(1024))) unsigned char o0s[SUB * TB], o1s[SUB * TB], o2s[QB3];
  // row statistics, rows 0 .. 32 SUB - 1 used
  __shared__ __attribute__((aligned(16))) float l0s[64], l1s[64], l2s[LS3];
  __shared__ __attribute__((aligned(16))) float d0s[64], d1s[64], d2s[LS3];
  auto qb = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? q0s : i == 1 ? q1s : q2s;
  };
  auto ob = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? o0s : i == 1 ? o1s : o2s;
  };
  auto ls = [&](int i) __attribute__((always_inline)) -> float* { return i == 0 ? l0s : i == 1 ? l1s : l2s; };
  auto dls = [&](int i) __attribute__((always_inline)) -> float* { return i == 0 ? d0s : i == 1 ? d1s : d2s; };
  // NKL of the wave's K operands live in LDS instead of registers (d = 128:
  // with all of them in registers the pass needs a few more than the 256 it
  // has, and the compiler's scratch reloads of the spilled ones in the loop
  // wait on the vector-memory counter, that is on the tile copies in flight).
  constexpr int NKL = D == 128 ? 2 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char kres[kBwdWaves][NKL > 0 ? NKL * 1024 : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int N = p.N;
  const int bid = bwd_block();
  const int kvh = bid / p.n_kt;
  const int kt = bid - kvh * p.n_kt;
  const int b = kvh / p.H_kv, g = kvh - b * p.H_kv;
  int kl = N;
  if (p.key_len != nullptr) {
    const int x = p.key_len[b];
    kl = x < 0 ? 0 : (x > N ? N : x);
  }
  kl = __builtin_amdgcn_readfirstlane(kl);
  const int k_wg0 = kt * kBwdRows, kw0 = k_wg0 + 32 * wave, key = kw0 + l32;
  const int nqt = (N + 31) / 32;
  const int t_begin = CAUSAL ? k_wg0 / 32 : 0;  // a multiple of 4: iterations start at even tiles
  const int per_head = k_wg0 < kl ? (nqt - t_begin + SUB - 1) / SUB : 0;  // iterations per head
  const int n_iter = per_head * p.group;
  const bool wave_live = kw0 < kl;

  const size_t kv_head = (size_t)kvh * N * D;
  v8 kf[KS], vf[KS];
  {
    const auto rk = tile_rsrc((const T*)p.k + kv_head, 0, N, N, D * 2);
    const auto rv = tile_rsrc((const T*)p.v + kv_head, 0, N, N, D * 2);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      kf[st] = __builtin_bit_cast(v8, load16(rk, key * D * 2 + 32 * st + 16 * hi));
      vf[st] = __builtin_bit_cast(v8, load16(rv, key * D * 2 + 32 * st + 16 * hi));
    }
  }
#pragma unroll
  for (int st = 0; st < NKL; ++st) *(v8*)(kres[wave] + st * 1024 + lane * 16) = kf[st];
  const float c = p.c;
  SwzTile<D> sz;
  sz.init(pinned_int(lane));

  // Cursor of iteration u: first query tile t and query head hq (index within
  // the group) of a scan that runs over t from t_begin + SUB (per_head - 1)
  // down to t_begin in steps of SUB, for each head of the group in turn;
  // advanced once per iteration (no division in the loop). Past n_iter the
  // head index is clamped and the row limit is 0. Descending order: every
  // workgroup of a head starts at the head's last query tiles whatever its
  // key block, so the workgroups running together on an XCD read the same
  // Q / dO tile at about the same time and fetch it through L2 once (in
  // ascending order each would start at its own diagonal and read a
  // different tile).
  struct Cur {
    int u, t, hq;
  };
  const int ph = max(per_head, 1);
  const int t_last = t_begin + SUB * (ph - 1);
  auto advance = [&](Cur c) __attribute__((always_inline)) -> Cur {
    ++c.u;
    c.t -= SUB;
    if (c.t < t_begin) c.t = t_last, ++c.hq;
    return c;
  };
  auto qhead_of = [&](const Cur& c) __attribute__((always_inline)) -> size_t {
    return ((size_t)b * p.H + g * p.group + min(c.hq, p.group - 1)) * N;
  };
  auto copies = [&](const Cur& c, int buf) __attribute__((always_inline)) {
    const size_t qhead = qhead_of(c);
    const int lim = c.u < n_iter ? N : 0;
#pragma unroll
    for (int x = 0; x < SUB; ++x) {
      copy_rows_swz<D>((const T*)p.q + qhead * D, c.t + x, lim, qb(buf) + x * TB, wave, lane);
      copy_rows_swz<D>((const T*)p.dout + qhead * D, c.t + x, lim, ob(buf) + x * TB, wave, lane);
    }
  };
  // Row statistics of an iteration's rows (lse2 = LSE * log2 e, and Delta)
  // straight into LDS beside its Q and dO rows, issued by the last wave ahead
  // of its tile copies: lane i takes row 32 t + i; lanes past the
  // iteration's rows, rows at or past N and every row past the last
  // iteration fall outside the copy's range and land as zeros. Such rows have
  // zero Q and dO rows too, so there P = 1 and dS = 0 exactly, and they add
  // nothing to dK or dV.
  auto stats_copy = [&](const Cur& c, int buf) __attribute__((always_inline)) {
    if (wave == kBwdWaves - 1) {
      const int rows = c.u < n_iter ? max(0, min(32 * SUB, N - 32 * c.t)) : 0;
      const size_t row0 = rows > 0 ? qhead_of(c) + 32 * c.t : 0;
      lds_copy4(buffer_rsrc(p.lse2 + row0, rows * 4), (unsigned char*)ls(buf), 4 * lane);
      lds_copy4(buffer_rsrc(p.delta + row0, rows * 4), (unsigned char*)dls(buf), 4 * lane);
    }
  };
  Cur c0{0, t_last, 0};  // iteration u
  Cur c1 = advance(c0);  // u + 1
  Cur c2 = advance(c1);  // u + 2

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = f32x16{}, dv[db] = f32x16{};
  if (n_iter > 0) {
    stats_copy(c0, 0);
    if constexpr (AHEAD == 2) stats_copy(c1, 1);
    copies(c0, 0);
    if constexpr (AHEAD == 2) copies(c1, 1);
    // statistics and the tiles of iteration 0 landed (those of 1 may be in flight)
    wait_vmem_keep<(AHEAD - 1) * 2 * NCPW * SUB>();
  }
  __syncthreads();
  // Iteration u uses buffer u % NB, a compile-time index (the loop is
  // unrolled over the buffers). Masks: only the wave's diagonal query tile
  // (some key above some query row) and a ragged last key block (keys at or
  // past kl) need one; there the masked scores are set to -inf in place before
  // the exponentials, elsewhere the scores go straight through.
  auto iter = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const Cur& ca = AHEAD == 2 ? c2 : c1;
    stats_copy(ca, (buf + AHEAD) % NB);
    copies(ca, (buf + AHEAD) % NB);
#pragma unroll
    for (int x = 0; x < SUB; ++x) {
      const int t = c0.t + x;
      const unsigned char* qt = qb(buf) + x * TB;
      const unsigned char* ot = ob(buf) + x * TB;
      if (wave_live && (!CAUSAL || 32 * t + 31 >= kw0)) {
        f32x16 s = {}, dp = {};
        v8 kk[KS];
        {
          // an offset the compiler cannot see through: the operands are read
          // back from LDS here, not kept live in registers from the store
          int ko = lane * 16;
          __asm__ volatile("" : "+v"(ko));
#pragma unroll
          for (int st = 0; st < KS; ++st)
            kk[st] = st < NKL ? *(const v8*)(kres[wave] + st * 1024 + ko) : kf[st];
        }
        two_products<E, D>(qt, ot, sz, hi, kk, vf, s, dp);
        if ((CAUSAL && 32 * t < kw0 + 31) || kw0 + 32 > kl) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qry = 32 * t + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool ok = key < kl && (!CAUSAL || key <= qry);
            s[i] = ok ? s[i] : -INFINITY;
          }
        }
        v8 pf[2], dsf[2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 l4 = *(const f32x4*)(ls(buf) + 32 * x + 8 * q4 + 4 * hi);
          const f32x4 d4 = *(const f32x4*)(dls(buf) + 32 * x + 8 * q4 + 4 * hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * q4 + e;
            const float pr = fast_exp2(fmaf(s[i], c, -l4[e]));
            pf[i >> 3][i & 7] = E::cvt(pr);
            dsf[i >> 3][i & 7] = E::cvt(pr * (dp[i] - d4[e]));
          }
        }
        tr_product<E, D>(ot, sz, pf, dv);
        tr_product<E, D>(qt, sz, dsf, dk);
      }
    }
    // the next iteration's tiles and statistics landed (the copies issued
    // here may stay in flight when they run two iterations ahead)
    wait_vmem_keep<(AHEAD - 1) * 2 * NCPW * SUB>();
    __syncthreads();
    c0 = c1;
    c1 = c2;
    c2 = advance(c2);
  };
  for (int u0 = 0; u0 < n_iter; u0 += NB) {
    static_for<NB>([&](auto qc) __attribute__((always_inline)) {
      if (u0 + decltype(qc)::value < n_iter) iter(qc);  // workgroup-uniform
    });
  }
  wait_vmem();
  if (key < N) {
    store_grad<T, DB>((T*)p.dk + kv_head + (size_t)key * D, hi, p.scale, dk);
    store_grad<T, DB>((T*)p.dv + kv_head + (size_t)key * D, hi, 1.0f, dv);
  }
}

// ---------------------------------------------------------------------------
// Launch table
// ---------------------------------------------------------------------------
constexpr int kWaves = FA_WAVES;  // x 32 query rows per workgroup

template <class K>
hipError_t launch(K kernel, const Params& p, int threads, hipStream_t stream, int units = 0) {
  // units: workgroups per (batch, head); one per query tile unless given
  const long long grid = (long long)p.B * p.H * (units > 0 ? units : p.n_qt);
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  Params local = p;
  void* args[] = {&local};
  return hipLaunchKernel((const void*)kernel, dim3((unsigned)grid), dim3(threads), args, 0,
                         stream);
}

// 16-bit kernel choice. The pipelined kernel (FA_WIDE_WAVES * 32 query rows
// per workgroup) wins without a causal mask and, with one, once the sequence
// gives every workgroup a long run of key tiles; short causal sequences keep
// the direct-to-LDS kernel, whose smaller workgroups spread the little work
// of the short query tiles over more CUs (measured on MI355X).
bool use_pipe(int N, bool causal) { return !causal || N >= FA_PIPE_MIN_N; }

// Workgroups per (batch, head) of the pipelined kernel: one per query tile,
// or per folded pair of causal query tiles.
int pipe_units(const Params& p, bool causal) { return causal ? (p.n_qt + 1) / 2 : p.n_qt; }

template <class E, int D, bool C>
hipError_t launch_16bit(const Params& p, hipStream_t s) {
  if (p.win_left >= 0 || p.win_right >= 0)
    return launch(attn_fwd_16bit_dma<E, D, FA_KEY_TILE, FA_DMA_WAVES, C, true>, p,
                  FA_DMA_WAVES * 64, s);
  if (use_pipe(p.N, C))
    return launch(attn_fwd_pipe<E, D, FA_WIDE_WAVES, C, false>, p, FA_WIDE_WAVES * 64, s,
                  pipe_units(p, C));
  return launch(attn_fwd_16bit_dma<E, D, FA_KEY_TILE, FA_DMA_WAVES, C>, p, FA_DMA_WAVES * 64, s);
}

// Packed batches take the kernel a single sequence of the longest length
// would take (p.N is that length).
template <class E, int D, bool C>
hipError_t launch_16bit_varlen(const Params& p, hipStream_t s) {
  if (use_pipe(p.N, C))
    return launch(attn_fwd_pipe<E, D, FA_WIDE_WAVES, C, false, true>, p, FA_WIDE_WAVES * 64, s,
                  pipe_units(p, C));
  return launch(attn_fwd_16bit_dma<E, D, FA_KEY_TILE, FA_DMA_WAVES, C, false, true>, p,
                FA_DMA_WAVES * 64, s);
}

template <int D, bool C>
hipError_t launch_d(Kind kind, const Params& p, hipStream_t s) {
  constexpr int T = kWaves * 64;
  switch (kind) {
    case Kind::BF16: return launch_16bit<Bf16, D, C>(p, s);
    case Kind::F16: return launch_16bit<F16, D, C>(p, s);
    case Kind::FP8:
      if (use_pipe(p.N, C))
        return launch(attn_fwd_pipe<Bf16, D, FA_WIDE_WAVES, C, true>, p, FA_WIDE_WAVES * 64, s,
                      pipe_units(p, C));
      return launch(attn_fwd_fp8<D, kWaves, FA_KEY_TILE, C>, p, T, s);
    case Kind::FP8_P8:  // every shape: one kernel, one rounding of P
      return launch(attn_fwd_pipe8<D, FA_WIDE_WAVES, C>, p, FA_WIDE_WAVES * 64, s, pipe_units(p, C));
    case Kind::F32: return launch(attn_fwd_f32<D, kWaves, 32, C>, p, T, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int rows_per_block(Kind kind, int d, int N, bool causal, bool window) {
  if (d == 256) {
    if ((kind != Kind::BF16 && kind != Kind::F16) || window) return 0;
    return use_pipe(N, causal) ? FA_WIDE_WAVES * 32 : 4 * 32;
  }
  if (d != 64 && d != 128) return 0;
  if (window) return kind == Kind::BF16 || kind == Kind::F16 ? FA_DMA_WAVES * 32 : 0;
  if (kind == Kind::BF16 || kind == Kind::F16)
    return use_pipe(N, causal) ? FA_WIDE_WAVES * 32 : FA_DMA_WAVES * 32;
  if (kind == Kind::FP8 && use_pipe(N, causal)) return FA_WIDE_WAVES * 32;
  if (kind == Kind::FP8_P8) return FA_WIDE_WAVES * 32;
  return kWaves * 32;
}

hipError_t launch_forward(Kind kind, int d, bool causal, const Params& p, hipStream_t stream) {
  if (d == 256) {
    // the pipelined kernel on 128-column slices of V and O (two workgroups
    // per query tile, or per folded pair of causal tiles)
    if ((kind == Kind::BF16 || kind == Kind::F16) && use_pipe(p.N, causal)) {
      const int units = 2 * pipe_units(p, causal);
      constexpr int T = FA_WIDE_WAVES * 64;
      if (kind == Kind::BF16)
        return causal ? launch(attn_fwd_pipe<Bf16, 256, FA_WIDE_WAVES, true, false, false, 128>, p, T, stream, units)
                      : launch(attn_fwd_pipe<Bf16, 256, FA_WIDE_WAVES, false, false, false, 128>, p, T, stream, units);
      return causal ? launch(attn_fwd_pipe<F16, 256, FA_WIDE_WAVES, true, false, false, 128>, p, T, stream, units)
                    : launch(attn_fwd_pipe<F16, 256, FA_WIDE_WAVES, false, false, false, 128>, p, T, stream, units);
    }
    // two workgroups (column halves of O) per query tile
    const long long grid = 2LL * p.B * p.H * p.n_qt;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    Params local = p;
    void* args[] = {&local};
    const void* k = nullptr;
    if (kind == Kind::BF16) k = causal ? (const void*)attn_fwd_d256<Bf16, 4, true> : (const void*)attn_fwd_d256<Bf16, 4, false>;
    else if (kind == Kind::F16) k = causal ? (const void*)attn_fwd_d256<F16, 4, true> : (const void*)attn_fwd_d256<F16, 4, false>;
    else return hipErrorInvalidValue;
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3(4 * 64), args, 0, stream);
  }
  if (d == 64) return causal ? launch_d<64, true>(kind, p, stream) : launch_d<64, false>(kind, p, stream);
  if (d == 128) return causal ? launch_d<128, true>(kind, p, stream) : launch_d<128, false>(kind, p, stream);
  return hipErrorInvalidValue;
}

int varlen_rows_per_block(int max_seqlen, bool causal) {
  return use_pipe(max_seqlen, causal) ? FA_WIDE_WAVES * 32 : FA_DMA_WAVES * 32;
}

hipError_t launch_forward_varlen(Kind kind, int d, bool causal, const Params& p,
                                 hipStream_t stream) {
  if (p.cu_seqlens == nullptr) return hipErrorInvalidValue;
  if (kind == Kind::BF16) {
    if (d == 64) return causal ? launch_16bit_varlen<Bf16, 64, true>(p, stream) : launch_16bit_varlen<Bf16, 64, false>(p, stream);
    if (d == 128) return causal ? launch_16bit_varlen<Bf16, 128, true>(p, stream) : launch_16bit_varlen<Bf16, 128, false>(p, stream);
  } else if (kind == Kind::F16) {
    if (d == 64) return causal ? launch_16bit_varlen<F16, 64, true>(p, stream) : launch_16bit_varlen<F16, 64, false>(p, stream);
    if (d == 128) return causal ? launch_16bit_varlen<F16, 128, true>(p, stream) : launch_16bit_varlen<F16, 128, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

int decode_splits(int units_base, int Nk, int* chunk_tiles) {
  // About 4 waves per CU in all (one per SIMD), chunks of at least four
  // 32-key tiles. Measured on the 16-sequence, 16K-key grouped decode: 1024
  // waves 5.3 TB/s; 768 waves 4.8 (CUs left idle); 2048 waves 4.9, 4096 4.4
  // (more concurrent key streams and partial results).
  const int nt = (Nk + 31) / 32;
  const long long target = 1024;
  long long S = (target + units_base - 1) / units_base;
  S = std::max(1LL, std::min(S, (long long)(nt + 3) / 4));
  const int ct = (int)((nt + S - 1) / S);
  *chunk_tiles = ct;
  return (nt + ct - 1) / ct;
}

namespace {
template <class E, int D, bool C>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  DecodeParams local = p;
  void* args[] = {&local};
  const long long grid = ((long long)p.units + kDecodeWaves - 1) / kDecodeWaves;
  const long long rows = (long long)p.B * p.H * p.Nq;
  if (grid <= 0 || grid > 0x7fffffffLL || rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipError_t e = hipLaunchKernel((const void*)attn_decode_split<E, D, C>, dim3((unsigned)grid),
                                 dim3(kDecodeWaves * 64), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)attn_decode_merge<typename E::T, D>, dim3((unsigned)rows),
                         dim3(64), args, 0, stream);
}
template <class E>
hipError_t launch_decode_e(int d, bool causal, const DecodeParams& p, hipStream_t s) {
  if (d == 64) return causal ? launch_decode_t<E, 64, true>(p, s) : launch_decode_t<E, 64, false>(p, s);
  if (d == 128) return causal ? launch_decode_t<E, 128, true>(p, s) : launch_decode_t<E, 128, false>(p, s);
  return hipErrorInvalidValue;
}
}  // namespace

namespace {
template <class E, int D, bool C>
hipError_t launch_backward_t(const BwdParams& p, hipStream_t stream) {
  BwdParams local = p;
  void* args[] = {&local};
  const long long g_dq = (long long)p.B * p.H * p.n_qt;
  const long long g_kv = (long long)p.B * p.H_kv * p.n_kt;
  if (g_dq > 0x7fffffffLL || g_kv > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // the dQ pass also writes every row's Delta and LSE * log2 e to the
  // workspace, which the dK/dV pass (queued after it) reads
  hipError_t e = hipLaunchKernel((const void*)attn_bwd_dq_dma<E, D, C>, dim3((unsigned)g_dq),
                                 dim3(kBwdWaves * 64), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)attn_bwd_dkdv_dma<E, D, C>, dim3((unsigned)g_kv),
                         dim3(kBwdWaves * 64), args, 0, stream);
}
template <class E>
hipError_t launch_backward_e(int d, bool causal, const BwdParams& p, hipStream_t s) {
  if (d == 64) return causal ? launch_backward_t<E, 64, true>(p, s) : launch_backward_t<E, 64, false>(p, s);
  if (d == 128) return causal ? launch_backward_t<E, 128, true>(p, s) : launch_backward_t<E, 128, false>(p, s);
  return hipErrorInvalidValue;
}
}  // namespace

int bwd_rows_per_block() { return kBwdRows; }

hipError_t launch_backward(Kind kind, int d, bool causal, const BwdParams& p, hipStream_t stream) {
  if (kind == Kind::BF16) return launch_backward_e<Bf16>(d, causal, p, stream);
  if (kind == Kind::F16) return launch_backward_e<F16>(d, causal, p, stream);
  return hipErrorInvalidValue;
}

// Device scratch of fa_fwd_decode_noalloc: a fixed array in the code object,
// one copy on every device the library runs on, held until the process ends.
// Host code never names it as an address: the device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and kept
// per device; kernels receive that address like a caller's workspace.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = ptr;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

hipError_t launch_decode(Kind kind, int d, bool causal, const DecodeParams& p, hipStream_t stream) {
  if (kind == Kind::BF16) return launch_decode_e<Bf16>(d, causal, p, stream);
  if (kind == Kind::F16) return launch_decode_e<F16>(d, causal, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
