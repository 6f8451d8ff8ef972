// C-ABI entry points: argument validation, kernel selection, launch.
// Declarations and the contract (layouts, ownership, errors) are in
// include/attn.h.  Every check runs before the first HIP call.
#include "attn.h"

#include <math.h>
#include <stdint.h>

#include "attn_api_internal.h"
#include "attn_bwd_kernel.h"
#include "attn_fwd_kernel.h"

namespace {

constexpr int kVersion = 400;  // 0.4.0
constexpr int kMaxGridYZ = 65535;
// Largest conditional-rescale threshold (log2 units).  A row that skips its
// rescale weights keys by up to 2^tau, so its row sum and output accumulators
// grow to about N * 2^tau * max|v| in fp32; 64 keeps that far below the fp32
// range (2^128) for any sequence the 32-bit token indices allow.
constexpr float kMaxRescaleThreshold = 64.0f;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dims(int d_qk, int d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
}

}  // namespace

namespace attn_internal {

int bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              const void* dq, const void* dk, const void* dv, const float* delta, bool with_delta,
              const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v, float scale) {
  if (B < 1 || H < 1 || N < 0) return ATTN_ERR_SHAPE;
  if (!supported_dims(d_qk, d_v)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  if (N == 0) return kNothingToDo;  // no tokens: nothing to do
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || (with_delta && !delta)) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return ATTN_ERR_ALIGN;
  if (!aligned(lse, 4) || (with_delta && !aligned(delta, 4)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
    return ATTN_ERR_ALIGN;
  const int rows = attn_grad::block_rows();
  const int64_t nb = ((int64_t)N + rows - 1) / rows;
  if ((int64_t)H * B * nb > INT32_MAX) return ATTN_ERR_SHAPE;   // one workgroup per (sequence, head, block)
  if ((int64_t)B * N > INT32_MAX) return ATTN_ERR_SHAPE;        // token indices are 32-bit in the kernels
  if ((int64_t)B * N * H > INT32_MAX) return ATTN_ERR_SHAPE;    // rows of the D pass
  // one sequence's Q, K, V or dO rows of one head are addressed through a
  // 32-bit buffer range, with tile requests up to 255 rows past its end
  if (((int64_t)N + 256) * H * (d_qk > d_v ? d_qk : d_v) * 2 > (int64_t)UINT32_MAX) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

int bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, float* delta, const int32_t* cu_seqlens, int B, int H, int N,
               int d_qk, int d_v, float scale, int causal, hipStream_t stream) {
  const int rows = attn_grad::block_rows();
  attn_grad::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.delta = delta;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.H = H;
  p.N = N;
  p.n_blocks = (int)(((int64_t)N + rows - 1) / rows);
  p.scale = scale;
  p.c = scale * 1.44269504088896340736f;
  const hipError_t err = attn_grad::launch_bwd(p, d_qk, d_v, causal != 0, stream);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace attn_internal

extern "C" {

void attn_fwd_opts_default(attn_fwd_opts* opts) {
  if (!opts) return;
  opts->rescale_threshold_log2 = 8.0f;
  opts->poly_exp_sixteenths = 0;
  opts->schedule = ATTN_SCHEDULE_LONGEST_FIRST;
  opts->stats = nullptr;
  opts->block_mask = nullptr;
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H or N out of range (B, H >= 1, N >= 0, grid limits)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dims: (d_qk, d_v) must be (64,64), (128,128) or (192,128)";
    case ATTN_ERR_ALIGN: return "misaligned pointer: q, k, v, o need 16 bytes; lse, cu_seqlens 4 bytes";
    case ATTN_ERR_VALUE: return "invalid value: non-finite scale or option out of range";
    case ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
    case ATTN_ERR_SCRATCH: return "too large for the allocation-free entry point: H*B*N above ATTN_NOALLOC_MAX_ROWS";
    default: return "unknown attn status";
  }
}

int attn_version(void) { return kVersion; }

int attn_fwd_geometry(int d_qk, int d_v, int* rows_per_item, int* keys_per_tile, int* rows_per_wave) {
  if (!supported_dims(d_qk, d_v)) return ATTN_ERR_UNSUPPORTED;
  if (rows_per_item) *rows_per_item = attn::query_block_rows();
  if (keys_per_tile) *keys_per_tile = attn::keys_per_tile(d_qk);
  if (rows_per_wave) *rows_per_wave = attn::rows_per_wave();
  return ATTN_OK;
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
                float scale, int causal, hipStream_t stream, const attn_fwd_opts* opts) {
  attn_fwd_opts def;
  attn_fwd_opts_default(&def);
  const attn_fwd_opts& op = opts ? *opts : def;

  if (B < 1 || H < 1 || N < 0) return ATTN_ERR_SHAPE;
  if (!supported_dims(d_qk, d_v)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  if (!isfinite(op.rescale_threshold_log2) || op.rescale_threshold_log2 > kMaxRescaleThreshold) return ATTN_ERR_VALUE;
  const int np = op.poly_exp_sixteenths;
  if (np != 0 && np != 2 && np != 4 && np != 8) return ATTN_ERR_VALUE;
  if (op.schedule != ATTN_SCHEDULE_LONGEST_FIRST && op.schedule != ATTN_SCHEDULE_NATURAL) return ATTN_ERR_VALUE;
  if (op.block_mask) {
    if (np != 0) return ATTN_ERR_UNSUPPORTED;                   // hardware exp2 only
    if (N > 32768) return ATTN_ERR_SHAPE;                       // 256 key blocks of 128
  }
  if (N == 0) return ATTN_OK;  // no tokens: nothing to do
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ATTN_ERR_ALIGN;
  if (!aligned(lse, 4) || (cu_seqlens && !aligned(cu_seqlens, 4))) return ATTN_ERR_ALIGN;
  if (!aligned(op.stats, 8)) return ATTN_ERR_ALIGN;

  const int rows = attn::query_block_rows();
  const int64_t nqb = ((int64_t)N + rows - 1) / rows;
  if (B > kMaxGridYZ || nqb > kMaxGridYZ) return ATTN_ERR_SHAPE;
  // the longest-first schedule launches one workgroup per (head, sequence, query block)
  if ((int64_t)H * B * nqb > INT32_MAX) return ATTN_ERR_SHAPE;
  // token indices are 32-bit inside the kernel
  if (!cu_seqlens && (int64_t)B * N > INT32_MAX) return ATTN_ERR_SHAPE;
  // one sequence's K or V rows of one head are addressed through a 32-bit
  // buffer range, and tile requests reach up to 255 rows past its end:
  // (N + 256) * H * d * 2 bytes must stay below 4 GiB
  if (((int64_t)N + 256) * H * (d_qk > d_v ? d_qk : d_v) * 2 > (int64_t)UINT32_MAX) return ATTN_ERR_SHAPE;

  attn::FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.H = H;
  p.N = N;
  p.n_qblocks = (int)nqb;
  float c = fabsf(scale) * 1.44269504088896340736f;
  if (c < 1e-30f) c = 1e-30f;
  p.c = c;
  p.neg_scale = scale < 0.0f ? 1 : 0;
  p.tau = op.rescale_threshold_log2;
  p.schedule = op.schedule;
  p.stats = reinterpret_cast<unsigned long long*>(op.stats);
  p.block_mask = op.block_mask;
  p.mask_blocks = (int)((N + 127) / 128);

  p.next_stride = 0;
  if (op.schedule == ATTN_SCHEDULE_LONGEST_FIRST) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      p.next_stride = cus;
  }

  const hipError_t err = attn::launch_fwd(p, d_qk, d_v, causal != 0, np, stream);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
             float scale, int causal, hipStream_t stream) {
  return attn_fwd_ex(q, k, v, o, lse, cu_seqlens, B, H, N, d_qk, d_v, scale, causal, stream, nullptr);
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o, float* lse,
                 const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
                 float scale, float q_descale, float k_descale, float v_descale,
                 int causal, hipStream_t stream) {
  if (B < 1 || H < 1 || N < 0) return ATTN_ERR_SHAPE;
  if (!supported_dims(d_qk, d_v)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  for (float f : {q_descale, k_descale, v_descale})
    if (!isfinite(f) || !(f > 0.0f)) return ATTN_ERR_VALUE;
  if (N == 0) return ATTN_OK;
  if (!q8 || !k8 || !v8 || !o || !lse) return ATTN_ERR_NULL;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16)) return ATTN_ERR_ALIGN;
  if (!aligned(lse, 4) || (cu_seqlens && !aligned(cu_seqlens, 4))) return ATTN_ERR_ALIGN;
  const int rows = attn::query_block_rows();
  const int64_t nqb = ((int64_t)N + rows - 1) / rows;
  if ((int64_t)H * B * nqb > INT32_MAX) return ATTN_ERR_SHAPE;
  if (!cu_seqlens && (int64_t)B * N > INT32_MAX) return ATTN_ERR_SHAPE;
  // a (sequence, head) K or V range is addressed by a 32-bit buffer resource,
  // with tile requests up to 255 rows past its end
  if (((int64_t)N + 256) * H * d_qk > INT32_MAX) return ATTN_ERR_SHAPE;

  attn::Fp8Params p;
  p.q = static_cast<const uint8_t*>(q8);
  p.k = static_cast<const uint8_t*>(k8);
  p.v = static_cast<const uint8_t*>(v8);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.H = H;
  p.N = N;
  p.n_qblocks = (int)nqb;
  const double cd = fabs((double)scale) * (double)q_descale * (double)k_descale * 1.4426950408889634;
  float c = (float)(cd < 3.0e38 ? cd : 3.0e38);
  if (c < 1e-30f) c = 1e-30f;
  p.c = c;
  p.neg_scale = scale < 0.0f ? 1 : 0;
  p.o_scale = v_descale;
  p.tau = 8.0f;
  p.next_stride = 0;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    p.next_stride = cus;
  const hipError_t err = attn::launch_fwd_fp8(p, d_qk, d_v, causal != 0, stream);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v,
             float scale, int causal, hipStream_t stream) {
  const int st = attn_internal::bwd_check(q, k, v, o, dout, lse, dq, dk, dv, delta, true, cu_seqlens, B, H, N,
                                          d_qk, d_v, scale);
  if (st != ATTN_OK) return st == attn_internal::kNothingToDo ? ATTN_OK : st;
  return attn_internal::bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, delta, cu_seqlens, B, H, N, d_qk, d_v,
                                   scale, causal, stream);
}

int attn_debug_exp2(const float* x, float* y, int n, int use_poly, hipStream_t stream) {
  if (n < 0) return ATTN_ERR_SHAPE;
  if (use_poly != 0 && use_poly != 1) return ATTN_ERR_VALUE;
  if (n == 0) return ATTN_OK;
  if (!x || !y) return ATTN_ERR_NULL;
  if (!aligned(x, 4) || !aligned(y, 4)) return ATTN_ERR_ALIGN;
  const hipError_t err = attn::launch_exp2_debug(x, y, n, use_poly, stream);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
