/*
 * attn.h -- C ABI of the fused exact-attention forward pass on MI355X (gfx950).
 *
 * Computes, for every packed sequence b, head h and query row i,
 *
 *     O[i]   = sum_j softmax_j(scale * q_i . k_j  [j <= i if causal]) v_j
 *     LSE[i] = ln sum_j exp(scale * q_i . k_j)          (over the same keys)
 *
 * i.e. exact softmax attention, evaluated tile by tile with an online softmax
 * (running row max and row sum, earlier partial results corrected when the
 * max grows) so the N x N score matrix never reaches HBM.  Sources: the
 * ainexis.cn deep dive on FlashAttention-4 (background: tiling plus online
 * softmax; "horizontal extension", concept two: running max / running sum),
 * jsqmd.com news on FlashAttention-4 (section two: tiles computed on chip).
 *
 * Two algorithmic options from the same pages are exposed through
 * attn_fwd_opts:
 *   - conditional rescaling (wittx news "FlashAttention-4", section on
 *     skipping 90% of rescales): the output and row-sum rescale is applied
 *     only when a tile's row max exceeds the running max by more than a
 *     threshold in log2 units (8.0 = a factor of 256); the final division by
 *     the row sum makes the result exact whichever max was kept;
 *   - software exp2 (wittx, section on faking a hardware instruction in
 *     software; jsqmd section four, item 1): a fixed fraction of the
 *     exponentials uses range reduction 2^y = 2^floor(y) * p(y - floor(y))
 *     with a cubic p evaluated by Horner's rule on FMA, the rest use the
 *     hardware exp2.
 * The tile order follows the causal/varlen load-balancing scheduler idea of
 * the newton.com.tw wiki "FlashAttention-4", core-technology section:
 * query blocks with the most key tiles are dispatched first.  On MI355X the
 * default order also keeps all query blocks of one (sequence, head) pair on
 * one XCD, dispatched one after another, so that they share that XCD's L2
 * for the pair's K and V.
 *
 * ------------------------------------------------------------------ layouts
 *   q, k : bf16 [T, H, d_qk]   token-major, heads interleaved, contiguous
 *   v, o : bf16 [T, H, d_v]
 *   lse  : fp32 [H, T]
 *   cu_seqlens : NULL for fixed length (T = B*N, sequence b = tokens
 *                [b*N, (b+1)*N)); otherwise a DEVICE int32 array [B+1] with
 *                cu[0] = 0, non-decreasing, cu[B] = T, and N >= the longest
 *                sequence (N sizes the launch grid).  Its contents are a
 *                precondition and are not validated (that would need a sync).
 * All pointers are device pointers.  q, k, v, o must be 16-byte aligned;
 * lse and cu_seqlens 4-byte aligned.
 *
 * Supported head dims (d_qk, d_v): (64, 64), (128, 128), (192, 128).
 * (N + 256) * H * max(d_qk, d_v) * 2 must be below 4 GiB (the K and V rows of
 * one sequence are addressed through 32-bit buffer ranges, and tile requests
 * reach up to 255 rows past their end); else ATTN_ERR_SHAPE.
 * Causal masking is square (query i sees keys j <= i of its own sequence).
 * scale: any finite value (negative values are handled exactly); when
 * |scale| * log2(e) < 1e-30 it is raised to 1e-30, which changes no output
 * (all logits already round to zero) and keeps masked keys at exp2(-inf) = 0.
 *
 * ---------------------------------------------------------------- ownership
 * The caller owns every buffer.  The library never allocates, frees,
 * retains or synchronises: each call enqueues kernels on `stream` and
 * returns.  There is no hidden global state besides the kernel code.
 *
 * ------------------------------------------------------------------- errors
 * Every entry point returns ATTN_OK (0) or a negative attn_status.  All
 * argument checks happen before any HIP call, so a rejected call has no
 * effect.  ATTN_ERR_LAUNCH reports a failed kernel launch (hipGetLastError).
 */
#ifndef EXACT_ATTENTION_57_AMD_ATTN_H
#define EXACT_ATTENTION_57_AMD_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,         /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,        /* B, H, N out of range or grid too large */
  ATTN_ERR_UNSUPPORTED = -3,  /* (d_qk, d_v) not one of the supported pairs */
  ATTN_ERR_ALIGN = -4,        /* pointer misaligned */
  ATTN_ERR_VALUE = -5,        /* non-finite scale or invalid option value */
  ATTN_ERR_LAUNCH = -6,       /* the HIP launch failed */
  ATTN_ERR_SCRATCH = -7       /* larger than attn_bwd_noalloc's scratch array holds */
} attn_status;

/* Schedules for the (sequence, head, query-block) work items. */
#define ATTN_SCHEDULE_LONGEST_FIRST 0  /* causal: query blocks with most key tiles first */
#define ATTN_SCHEDULE_NATURAL 1        /* query blocks in increasing order */

typedef struct attn_fwd_opts {
  /* Conditional-rescale threshold in log2 units.  >= 0: rescale a row only
   * when the tile's row max exceeds the kept max by more than this (0 gives
   * results bitwise equal to always rescaling).  < 0: always rescale, the
   * classic online softmax.  Default 8.0 (a factor of 256).  At most 64
   * (else ATTN_ERR_VALUE): a row that skips its rescale weights keys by up
   * to 2^threshold, and its fp32 row sum and output accumulators must stay
   * far below the fp32 range; non-finite values are rejected too. */
  float rescale_threshold_log2;
  /* Sixteenths of the exponentials computed with the software exp2:
   * one of 0, 2, 4, 8 (0, 1/8, 1/4, 1/2).  Default 0. */
  int poly_exp_sixteenths;
  /* ATTN_SCHEDULE_LONGEST_FIRST (default: per (sequence, head) pair,
   * longest query blocks first, pairs spread over the XCDs) or
   * ATTN_SCHEDULE_NATURAL (grid order).  Results are identical bit for bit;
   * only the speed differs. */
  int schedule;
  /* Optional DEVICE uint64[4] the kernel ADDS to (caller zeroes it):
   * [0] row-tile pairs where a rescale was considered (after a row's first
   * tile), [1] rescales applied, [2] (wave, tile) pairs computed, [3] work
   * items (query blocks) that ran.  NULL (default) disables counting.
   * Counts [0], [1] stay 0 for block-sparse runs. */
  uint64_t* stats;
  /* Optional DEVICE uint8 block mask for block-sparse attention
   * (FlexAttention-style variants on the same kernels: wittx news
   * "FlashAttention-4", section on writing GPU kernels in Python; newton.com.tw
   * wiki, development history): element [b][h][qb][kb], shape
   * [B, H, nb, nb] with nb = ceil(N / 128), nonzero keeps the 128 x 128 block
   * of query rows qb*128.. and keys kb*128.. of sequence b, head h.  Query i
   * then attends to the keys j of kept blocks (and j <= i if causal); a query
   * with no such key gets o = 0 and lse = -inf.  Blocks past a sequence's
   * end are ignored.  Workgroups visit only the key tiles some of their rows
   * keep.  Requires N <= 32768 and poly_exp_sixteenths = 0 (else
   * ATTN_ERR_SHAPE / ATTN_ERR_UNSUPPORTED).  NULL (default): dense. */
  const uint8_t* block_mask;
} attn_fwd_opts;

/* Fill *opts with the defaults above. */
void attn_fwd_opts_default(attn_fwd_opts* opts);

/* Forward pass with default options.  N == 0 is a no-op returning ATTN_OK.
 * Arguments: see the layouts above; `causal` is 0 or non-zero. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
             float scale, int causal, hipStream_t stream);

/* Forward pass with explicit options (opts == NULL means the defaults). */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
                float scale, int causal, hipStream_t stream, const attn_fwd_opts* opts);

/* Static description of an attn_status value (never NULL). */
const char* attn_strerror(int status);

/* Test hook: y[i] = the kernels' own exp2 of x[i], n elements of device fp32.
 * use_poly = 0: hardware exp2 (v_exp_f32); 1: the software range-reduced
 * cubic.  Same ownership and error rules as attn_fwd (n == 0 is a no-op). */
int attn_debug_exp2(const float* x, float* y, int n, int use_poly, hipStream_t stream);

/* Work decomposition the forward kernels use for a head-dim pair, needed to
 * interpret the statistics counters: *rows_per_item query rows per work
 * item, *keys_per_tile keys per K/V tile, *rows_per_wave query rows per
 * wave64.  Any output pointer may be NULL.  Returns ATTN_OK, or
 * ATTN_ERR_UNSUPPORTED for an unsupported (d_qk, d_v).  No HIP call. */
int attn_fwd_geometry(int d_qk, int d_v, int* rows_per_item, int* keys_per_tile, int* rows_per_wave);

/* Backward pass: gradients of the forward's O with respect to q, k and v.
 *
 * The backward pass of the same pages (wittx news "FlashAttention-4",
 * section on backward-pass optimisation; newton.com.tw wiki, core-technology
 * section): given dO = dLoss/dO and the forward's o and lse, with P the
 * softmax probabilities recomputed from lse,
 *     D_i = dO_i . O_i,   dS_ij = P_ij (dO_i . v_j - D_i),
 *     dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 *     dv_j = sum_i P_ij dO_i          (j over the keys query i sees).
 * dq is reduced over the keys inside one workgroup per query block and dk,
 * dv inside one per key block: no atomics, the result is the same bit for bit
 * on every run (the pages' deterministic mode, here the only mode).
 *
 * Layouts as for attn_fwd: q, k, dq, dk bf16 [T, H, d_qk]; v, o, dout, dv
 * bf16 [T, H, d_v]; lse fp32 [H, T] as attn_fwd wrote it (natural log).
 * delta: caller-owned fp32 workspace [H, T] (T = B*N for fixed length, or
 * cu_seqlens[B]; H*B*N floats always suffice), overwritten with D; its
 * contents on entry are ignored.  dq, dk, dv are overwritten.  cu_seqlens,
 * B, H, N, scale and causal must be the values of the forward call.
 * Supported (d_qk, d_v): (64, 64), (128, 128), (192, 128) (the forward's
 * pairs; others return ATTN_ERR_UNSUPPORTED), with the forward's 4 GiB limit on
 * one sequence's rows of one head ((N + 256) * H * max(d_qk, d_v) * 2 bytes).  Alignment: 16 bytes for the bf16 tensors, 4 for
 * lse, delta and cu_seqlens.  Ownership, streams and errors as attn_fwd
 * (validation before any HIP call, asynchronous on `stream`). */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
             float scale, int causal, hipStream_t stream);

/* Allocation-free backward pass, for callers that cannot allocate device
 * memory (work under stream capture, serving loops or harnesses that forbid
 * allocation): attn_bwd with the same arguments except `delta`.  The D
 * workspace lives in a static device array of the library (64 MiB, held by
 * every GPU the library runs on until the process ends), so the call
 * allocates nothing; it needs H * B * N <= ATTN_NOALLOC_MAX_ROWS, else
 * ATTN_ERR_SCRATCH (checked, like every other argument, before any HIP
 * call).  All calls on one GPU share its array: calls that overlap in time on
 * the same GPU (other streams or threads) race on it and must not be issued.
 * The first call on a device looks the array's address up (hipGetSymbolAddress,
 * no allocation); ATTN_ERR_LAUNCH if that fails.  Results are attn_bwd's
 * bit for bit (the same kernels). */
#define ATTN_NOALLOC_MAX_ROWS (16 * 1024 * 1024)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
                     float scale, int causal, hipStream_t stream);

/* FP8 forward pass: attention of E4M3 inputs with per-tensor dequantisation
 * factors.  The pages name FP8 as the low-precision arithmetic of the Hopper
 * generation (ainexis.cn deep dive, background, third stage) and as a
 * precision for later versions (wittx news "FlashAttention-4", closing
 * section); the operation is attn_fwd's on the dequantised values
 *     q = q_descale * q8,  k = k_descale * k8,  v = v_descale * v8,
 * with the same online softmax and conditional rescaling (threshold 8 in
 * log2 units).  Both matrix products run on the gfx950 FP8 matrix cores; the
 * probabilities P (<= 256) are rounded to E4M3 (nearest even) for the second
 * product and l is the sum of those rounded values, so O is a weighted mean of
 * v rows with weights off by at most 2^-4 relative (2^-10 absolute below the
 * E4M3 normal range) each, and LSE carries the same weight error.
 *
 * q8, k8: OCP E4M3 bytes [T, H, d_qk], v8: [T, H, d_v] (token-major, heads
 * interleaved); o: bf16 [T, H, d_v]; lse: fp32 [H, T] (natural log of the
 * scaled logits scale * q . k).  cu_seqlens, B, H, N, causal: as attn_fwd.
 * Supported (d_qk, d_v): attn_fwd's (64, 64), (128, 128), (192, 128) (else
 * ATTN_ERR_UNSUPPORTED); (N + 256) * H * d_qk must stay below 2^31 (bytes of
 * one sequence's rows of one head, addressed through 32-bit buffer ranges;
 * else ATTN_ERR_SHAPE).  scale: any finite
 * value; q_descale, k_descale, v_descale: finite and > 0 (else
 * ATTN_ERR_VALUE).  Alignment: 16 bytes for q8, k8, v8, o; 4 for lse and
 * cu_seqlens.  Ownership, streams and errors as attn_fwd. */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o, float* lse,
                 const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
                 float scale, float q_descale, float k_descale, float v_descale,
                 int causal, hipStream_t stream);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_57_AMD_ATTN_H */
