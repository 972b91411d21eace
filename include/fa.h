/*
 * fa.h -- C ABI of libfa, the exact IO-aware attention forward for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (FlashAttention (ES), "El problema de la atención estándar"):
 *
 *     O   = softmax(scale * Q K^T + mask) V
 *     LSE = per-row log-sum-exp of the masked, scaled logits (natural log)
 *
 * computed the way the pages' "Innovaciones clave" describe: Q, K and V are
 * split into tiles held in on-chip memory, each query row keeps a running
 * maximum and a running sum of exponentials that are corrected as new key
 * tiles arrive (online softmax), QK^T, the mask, the softmax and the product
 * with V are fused into one kernel, and only O and LSE are written. No N x N
 * matrix exists anywhere, on the device or the host.
 *
 * Masks (the pages list masking as part of the fused kernel without saying
 * which): the entry (i, j) of the logits is replaced by -inf unless
 *     j < key_len[b]               (key padding; key_len NULL means N)
 *     and (causal == 0 or j <= i)  (causal)
 * A row with no allowed key yields O = 0 and LSE = -inf.
 *
 * Conventions shared by every entry point:
 *   - Q, K, V, O are device pointers to dense row-major [B, H, N, d] tensors
 *     (d fastest, then N, then H, then B), 16-byte aligned.
 *   - LSE is a device pointer to float [B, H, N], 4-byte aligned.
 *   - key_len is NULL or a device pointer to int32 [B]; values are clamped to
 *     [0, N] on the device, so any int32 value is accepted.
 *   - The caller owns every buffer. The library allocates no memory and
 *     keeps no state but a per-thread error string, except the one fixed
 *     device array behind fa_fwd_decode_noalloc (see there); every other
 *     call is re-entrant and thread-safe.
 *   - Calls are asynchronous: they enqueue work on `stream` (a hipStream_t;
 *     NULL = the null stream) and return. Results are ready once the stream
 *     is synchronised. A fault inside the kernel surfaces at the caller's
 *     next synchronisation, not as a return value.
 *   - Errors are returned as fa_status codes, never by aborting. Argument
 *     checks run on the host before any HIP call; on an argument error no
 *     device work is enqueued and no buffer is touched.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 8  /* 2: fa_fwd_gqa; 3: fa_fwd_decode; 4: fa_bwd; 5: fa_fwd_window;
                             6: fa_fwd_varlen; 7: fa_fwd_decode_noalloc; 8: fa_fwd_fp8_p8 */

typedef enum {
  FA_DTYPE_FP32 = 0,     /* float32 in, float32 out                          */
  FA_DTYPE_FP16 = 1,     /* IEEE half in, half out                           */
  FA_DTYPE_BF16 = 2,     /* bfloat16 in, bfloat16 out                        */
  FA_DTYPE_FP8_E4M3 = 3  /* OCP fp8 e4m3 ("fn", max 448) in, bfloat16 out    */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* a NULL or misaligned pointer, a size < 1, an
                              out-of-range dtype, a scale or descale that is
                              not finite and > 0, sizes whose products
                              overflow, or an H_kv that does not divide H   */
  FA_ERR_UNSUPPORTED = -2, /* a head dimension d other than 64 or 128 (or
                              256 with 16-bit inputs to the forward), a
                              dtype an entry point does not take, or one
                              head's N x d tensor of 1 GiB or more          */
  FA_ERR_HIP = -3          /* the HIP runtime refused the launch            */
} fa_status;

/*
 * fa_fwd -- attention forward for one batch of B x H heads.
 *
 *   Q, K, V  [in]  device, [B,H,N,d] of `dtype` (fp8 e4m3 when dtype == 3)
 *   O        [out] device, [B,H,N,d]; of `dtype`, or bfloat16 for fp8 input
 *   LSE      [out] device, float [B,H,N], natural-log log-sum-exp per row
 *   B, H, N  batch, heads, sequence length (queries and keys), each >= 1
 *   d        head dimension; 64 or 128, or 256 for bfloat16 / float16 inputs
 *            (and N*d*sizeof(element) < 2^30: one head's Q, K or V below
 *            1 GiB)
 *   scale    multiplies QK^T before the mask; finite and > 0 (the pages use
 *            1/sqrt(d))
 *   causal   0 or 1 (any non-zero value means 1)
 *   key_len  NULL or device int32 [B] (see above)
 *   dtype    a fa_dtype value; fp8 input here means descales of 1.0
 *   stream   hipStream_t the work is enqueued on
 *
 * Returns FA_OK once the kernel is enqueued, or a negative fa_status.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t* key_len, int dtype, void* stream);

/*
 * fa_fwd_fp8 -- fa_fwd for fp8 e4m3 inputs quantised per tensor (the FP8
 * support of FlashAttention (ES), "FlashAttention-3 (2024)").
 *
 * The stored codes Q8, K8, V8 represent Q = q_descale * Q8, K = k_descale *
 * K8 and V = v_descale * V8. The logits are scale * q_descale * k_descale *
 * (Q8 K8^T); O = v_descale * softmax(...) V8, written as bfloat16. S = Q K^T
 * runs on the fp8 matrix cores; P stays in bfloat16 for the P V product.
 * Both products accumulate in fp32. The descales must be finite and > 0.
 * fa_fwd(..., FA_DTYPE_FP8_E4M3, ...) equals this call with descales 1.0.
 * Arguments otherwise as fa_fwd.
 */
int fa_fwd_fp8(const void* Q8, const void* K8, const void* V8, void* O_bf16, float* LSE,
               int B, int H, int N, int d, float scale, int causal,
               const int32_t* key_len, float q_descale, float k_descale,
               float v_descale, void* stream);

/*
 * fa_fwd_fp8_p8 -- fa_fwd_fp8 with both products on the fp8 matrix cores:
 * P is rounded to e4m3 for the P V product, as in the FP8 form of
 * FlashAttention (ES), "FlashAttention-3 (2024)" (FP8 operands, fp32
 * accumulation).
 *
 * Arguments, layouts, ownership and status codes as fa_fwd_fp8 (d 64 or
 * 128). The row sum l adds the same rounded P that multiply V, so O is still
 * a convex combination of V's rows; its weights carry e4m3's rounding (3
 * mantissa bits, at most 2^-4 relative per weight), so a row's error is at
 * most about 2 * 2^-4 * sum_j w_j |v_j - O| per column: small where the
 * weights spread over many keys (the long fp8 workload stays within 5e-2 of
 * the exact result), up to ~0.1 where two or three keys with different V
 * rows share a row's weight. LSE is computed from the unrounded P.
 */
int fa_fwd_fp8_p8(const void* Q8, const void* K8, const void* V8, void* O_bf16, float* LSE,
                  int B, int H, int N, int d, float scale, int causal,
                  const int32_t* key_len, float q_descale, float k_descale,
                  float v_descale, void* stream);

/*
 * fa_fwd_gqa -- fa_fwd with K/V heads shared by groups of query heads
 * (multi-query attention, which the FlashAttention-2 paragraph of
 * FlashAttention (ES), "Evolución y desarrollos posteriores", lists among
 * that version's additions, and its grouped generalisation).
 *
 *   Q, O     as fa_fwd: [B,H,N,d]
 *   K, V     [in] device, [B,H_kv,N,d] of `dtype`
 *   H_kv     K/V heads, >= 1 and dividing H. Query head h of a batch entry
 *            attends with K/V head h / (H / H_kv): consecutive query heads
 *            form a group. H_kv == 1 is multi-query attention, H_kv == H is
 *            fa_fwd.
 *   q_descale, k_descale, v_descale
 *            as fa_fwd_fp8, for every dtype (1.0 for plain inputs): the
 *            logits are scale * q_descale * k_descale * (Q K^T) and O is
 *            v_descale * softmax(...) V.
 * Other arguments, layouts, masks, ownership and errors as fa_fwd; an H_kv
 * that is < 1 or does not divide H returns FA_ERR_INVALID_ARG.
 */
int fa_fwd_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE,
               int B, int H, int H_kv, int N, int d, float scale, int causal,
               const int32_t* key_len, int dtype, float q_descale, float k_descale,
               float v_descale, void* stream);

/*
 * fa_fwd_window -- fa_fwd_gqa with a sliding-window (banded) mask on top of
 * the causal and padding masks (richer masks appear in the pages only as the
 * FlashMask title in the bibliography of FlashAttention (ES)): key j is
 * allowed for query i only if also
 *     window_left < 0  or j >= i - window_left
 *     window_right < 0 or j <= i + window_right
 * (a negative bound is no bound). Key tiles wholly outside every row's band
 * are skipped. bfloat16 / float16 inputs with d 64 or 128 (others:
 * FA_ERR_UNSUPPORTED); other arguments as fa_fwd_gqa.
 */
int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  int B, int H, int H_kv, int N, int d, float scale, int causal,
                  int window_left, int window_right, const int32_t* key_len, int dtype,
                  float q_descale, float k_descale, float v_descale, void* stream);

/*
 * fa_fwd_varlen -- a packed batch of B sequences of unequal length (packed
 * variable-length batches are among the richer masks named through the
 * FlashMask title in the bibliography of FlashAttention (ES)). The sequences
 * are concatenated along the row axis of every head, and each one is attended
 * on its own, exactly as fa_fwd_gqa would attend it as a batch entry of its own
 * length with every key valid.
 *
 *   Q          [in]  device, [H,total,d] of `dtype`: row r of head h is
 *                    Q + (h*total + r)*d
 *   K, V       [in]  device, [H_kv,total,d] of `dtype`
 *   O          [out] device, [H,total,d] of `dtype`
 *   LSE        [out] device, float [H,total], natural log
 *   cu_seqlens [in]  device, int32 [B+1]: sequence b holds rows
 *                    [cu_seqlens[b], cu_seqlens[b+1]); meant to be
 *                    non-decreasing from 0 to total
 *   B          sequences, >= 1
 *   H, H_kv    query and K/V heads, grouped as in fa_fwd_gqa
 *   total      packed rows per head, >= 1
 *   max_seqlen the longest sequence, >= 1: the grid covers this many rows
 *              per sequence
 *   d, scale, causal, dtype, stream as fa_fwd_gqa (causal: row i of a
 *              sequence sees that sequence's keys 0..i)
 *
 * Device-side bounds: each cu_seqlens value is clamped to [0, total], an end
 * below its start is taken as the start (an empty sequence), and a sequence
 * longer than max_seqlen is cut to its first max_seqlen rows. Rows of O and LSE
 * outside every (cut) sequence are not written. Overlapping sequences (a
 * decreasing cu_seqlens) give unspecified values in the overlap but stay
 * within the buffers. bfloat16 / float16 inputs with d 64 or 128 (others:
 * FA_ERR_UNSUPPORTED); a NULL cu_seqlens, B, H, total, max_seqlen < 1 or an
 * H_kv not dividing H return FA_ERR_INVALID_ARG. The library allocates
 * nothing.
 */
int fa_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  const int32_t* cu_seqlens, int B, int H, int H_kv, int total,
                  int max_seqlen, int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_decode -- the newest Nq queries of each batch entry against its
 * key/value cache (attention over the KV cache of streaming generation, which
 * FlashAttention (ES), "Soluciones especializadas", names as a use of the
 * method; FlashDecoding++ in its bibliography).
 *
 *   Q        [in]  device, [B,H,Nq,d] of `dtype`
 *   K, V     [in]  device, [B,H_kv,Nk,d] of `dtype` (the caches)
 *   O        [out] device, [B,H,Nq,d] of `dtype`
 *   LSE      [out] device, float [B,H,Nq], natural log
 *   H_kv     K/V heads, >= 1 and dividing H, grouped as in fa_fwd_gqa
 *   Nq, Nk   queries per head and cache length, each >= 1
 *   key_len  NULL or device int32 [B]: batch entry b holds kl_b =
 *            clamp(key_len[b], 0, Nk) valid keys (Nk when NULL)
 *   causal   query i sits at position kl_b - Nq + i: key j is allowed iff
 *            j < kl_b and, when causal, j <= kl_b - Nq + i. A query with no
 *            allowed key gets O = 0 and LSE = -inf.
 *   dtype    FA_DTYPE_BF16 or FA_DTYPE_FP16 (others: FA_ERR_UNSUPPORTED)
 *   workspace, workspace_bytes
 *            device scratch owned by the caller, 16-byte aligned, at least
 *            fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d) bytes; its
 *            contents on entry do not matter and on return are undefined.
 *            Calls that overlap in time need separate workspaces.
 *   d        64 or 128
 *   scale, stream as fa_fwd.
 *
 * The keys of each K/V head are split into chunks processed in parallel,
 * each writing a normalised partial O and its LSE to the workspace; a second
 * kernel on the same stream merges a row's chunks. Errors as fa_fwd, plus
 * FA_ERR_INVALID_ARG for a NULL, misaligned or too small workspace.
 */
int fa_fwd_decode(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                  const int32_t* key_len, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Workspace bytes fa_fwd_decode needs for these sizes (it depends on nothing
 * else); 0 if the sizes are invalid (a value < 1, H_kv not dividing H, or
 * products out of range).
 */
size_t fa_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d);

/*
 * fa_fwd_decode_noalloc -- fa_fwd_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, arguments and results, with
 * the per-chunk partial results held in the library's own device scratch
 * instead of a caller workspace. The call itself allocates nothing.
 *
 * The scratch is one fixed array of FA_DECODE_NOALLOC_MAX_BYTES in the
 * library's code object: each device the library runs on holds its own copy
 * from the first kernel launch until the process ends. Sizes whose
 * fa_decode_workspace_bytes() exceed FA_DECODE_NOALLOC_MAX_BYTES return
 * FA_ERR_UNSUPPORTED (use fa_fwd_decode with a workspace). Every call on a
 * device shares that device's scratch and leaves its partial results there:
 * calls that may overlap in time on one device (different streams or host
 * threads) race, and must be ordered by the caller. Nothing in the scratch
 * needs to start at any value. Errors as fa_fwd_decode (no workspace
 * checks), plus FA_ERR_HIP if the scratch's device address cannot be looked
 * up.
 */
#define FA_DECODE_NOALLOC_MAX_BYTES (8u << 20)
int fa_fwd_decode_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                          int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                          const int32_t* key_len, int dtype, void* stream);

/*
 * fa_bwd -- gradients of fa_fwd / fa_fwd_gqa with respect to Q, K and V.
 *
 * The pages report training speedups (FlashAttention (ES), "Resultados
 * empíricos") without writing the backward out; this is the calculus of the
 * forward's definition with its masks. With P the attention probabilities:
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *     dQ = scale * dS K,  dK = scale * dS^T Q,
 * where P is recomputed from Q, K and the forward's LSE (no N x N matrix is
 * stored). Grouped K/V heads receive the sum over the query heads sharing
 * them.
 *
 *   Q, O, dO [in]  device, [B,H,N,d] of `dtype`; O and LSE as the forward
 *                  returned them for these Q, K, V, scale, causal, key_len
 *   K, V     [in]  device, [B,H_kv,N,d] of `dtype`
 *   LSE      [in]  device, float [B,H,N]
 *   dQ       [out] device, [B,H,N,d] of `dtype`
 *   dK, dV   [out] device, [B,H_kv,N,d] of `dtype`
 *   dtype    FA_DTYPE_BF16 or FA_DTYPE_FP16 (others: FA_ERR_UNSUPPORTED)
 *   workspace, workspace_bytes
 *            device scratch owned by the caller, 16-byte aligned, at least
 *            fa_bwd_workspace_bytes(B, H, N) bytes (two floats per query row);
 *            overlapping calls need separate workspaces.
 *   d        64 or 128
 *   other arguments as fa_fwd_gqa (H_kv == H for ungrouped heads).
 * Errors as fa_fwd, plus FA_ERR_INVALID_ARG for a NULL, misaligned or too
 * small workspace. Two kernels run in order on `stream` (the first also
 * writes the rows' Delta and LSE * log2 e to the workspace for the second).
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int H_kv, int N, int d,
           float scale, int causal, const int32_t* key_len, int dtype, void* workspace,
           size_t workspace_bytes, void* stream);

/* Workspace bytes fa_bwd needs (0 if a size is < 1 or the product overflows). */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/* A static, human-readable name for a fa_status value (never NULL). */
const char* fa_status_str(int status);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

/*
 * A static description of the last error returned on the calling thread
 * (which argument was rejected, or the HIP error string); "" after FA_OK.
 */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
