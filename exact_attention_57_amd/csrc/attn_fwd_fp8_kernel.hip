// FP8 (E4M3) fused attention forward kernel for gfx950 (CDNA4, MI355X).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_kernel.h"
#include "attn_fwd_common.h"

namespace attn {

// FP8 (OCP E4M3) forward.
//
// The same work decode, ping-pong phases, LDS DMA pipeline and online softmax
// as the bf16 kernel (attn_fwd_kernel.hip), with both products on the gfx950
// FP8 matrix instruction v_mfma_f32_32x32x64_f8f6f4 (64-deep, twice the bf16
// rate), for (d_qk, d_v) = (64, 64), (128, 128) and (192, 128):
//
//   S^T = K Q^T      A: 32 bytes of one key row per lane (two ds_read_b128)
//                    per 64-deep step; B: Q^T resident (8 VGPRs per step)
//   O^T += V^T P^T   A: V^T gathered by ds_read_b64_tr_b8 (four per operand);
//                    B: the S^T accumulators after the softmax, rounded to E4M3
//
// plus one more output block whose A operand is all ones: each of its rows is
// the running row sum l of the E4M3-rounded P, so the softmax phase has no
// row-sum additions and O / l is a weighted mean of V rows with the weights
// the product actually used.  P <= 2^tau <= 256 stays inside E4M3's range
// (448).  Lane layouts (checked on the hardware): for the 32x32x64 FP8
// product lane l holds A[l % 32][32 (l / 32) + i] and B[32 (l / 32) + i][l % 32]
// in byte i; the transposing read hands lane i of each 16-lane group byte i%8
// of the 8-byte chunks addressed by lanes 2r + i/8, r = 0..7, as its bytes r.
// Method sources: as for the bf16 kernel; the FP8 precision itself is named by
// the ainexis.cn deep dive (background, third stage: FP8 on Hopper) and the
// wittx news (closing section: new precisions such as FP8 for later versions).
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

constexpr int kFp8BlockN = 128;     // keys per tile
#ifndef ATTN_FP8_PREFETCH
#define ATTN_FP8_PREFETCH 3
#endif
#ifndef ATTN_FP8_SETPRIO
#define ATTN_FP8_SETPRIO ATTN_SETPRIO
#endif
constexpr int kFp8Prefetch = ATTN_FP8_PREFETCH;   // matrix-phase operands read ahead (MFMA slots of 64 cycles)
constexpr uint32_t kE4m3One = 0x38383838u;   // four E4M3 1.0 bytes

// Four floats -> four E4M3 bytes (round to nearest even).  The conversion
// writes two bytes and keeps the other two of its destination; `dead` (any
// register whose value is no longer needed) serves as that destination, so no
// zeroing move precedes the first half.
__device__ __forceinline__ int pack_e4m3x4(float a, float b, float c, float d, int dead) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, dead, false);   // bytes 0, 1
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);              // bytes 2, 3
}
__device__ __forceinline__ f32x16_t mfma_fp8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  // format codes 0/0: both operands E4M3; scale operands 0: no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS layouts of the RB-byte rows (RB = d E4M3 values, RB/16 chunks of 16 bytes):
//  * K: the 16 consecutive rows of a quarter-wave ds_read_b128 land in 16
//    distinct 4-bank groups with chunk c of row r at
//       c ^ ((r/2) mod 8)     RB = 128 (two rows per 256-byte bank window)
//       c ^ ((r/4) mod 4)     RB = 64 (four rows per window) and RB = 192 (a
//                             row starts 12 chunks on: rows r mod 4 take four
//                             different bank quarters, the XOR the other bits)
//  * V: the 32 lanes of a half-wave ds_read_b64_tr_b8 (8 rows {0-3, 8-11} +
//    const, two chunks, two 8-byte halves) hit 32 distinct bank pairs with
//       c ^ 2 (b1(r) + 2 b3(r))  RB = 128 (b_i: bit i of r)
//       c ^ 2 b3(r)              RB = 64
// Every pattern repeats after 16 rows.
template <int RB>
__device__ __forceinline__ int k8_swz(int r) { return RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
template <int RB>
__device__ __forceinline__ int v8_swz(int r) {
  return RB == 128 ? 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) : 2 * ((r >> 3) & 1);
}

#ifndef ATTN_FP8_INTERLEAVE
#define ATTN_FP8_INTERLEAVE 0
#endif
// Logical slot at position pos of the matrix phase (score slots 0..NQK-1,
// output slots NQK..).  Plain order: all score slots, then the output slots.
// Interleaved: the kFp8Prefetch score slots whose operands are read ahead,
// then output and score slots alternating, then the remaining output slots,
// which spreads the transposing V reads over the phase.
template <int NQK>
__host__ __device__ constexpr int fp8_slot_at(int pos) {
  if (!ATTN_FP8_INTERLEAVE || pos < kFp8Prefetch) return pos;
  const int p = pos - kFp8Prefetch, left = NQK - kFp8Prefetch;
  if (p < 2 * left) return (p % 2 == 0) ? NQK + p / 2 : kFp8Prefetch + p / 2;
  return NQK + left + (p - 2 * left);
}

// Issue-order pin for the FP8 matrix phase: the MFMA at position s follows the
// LDS reads of position s + kFp8Prefetch (two for a score slot, four
// transposing reads for an output slot, none for the all-ones block).
template <int S, int NS, int NQK, int OB, int DB>
__device__ __forceinline__ void pin_fp8_schedule() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  if constexpr (S < NS) {
    constexpr int T = S + kFp8Prefetch;
    if constexpr (T < NS) {
      constexpr int L = fp8_slot_at<NQK>(T);
      constexpr int n = (L < NQK) ? 2 : (((L - NQK) % OB) < DB ? 4 : 0);
      if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(kDsRead, n, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    pin_fp8_schedule<S + 1, NS, NQK, OB, DB>();
  }
}

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_kernel(Fp8Params p) {
  static_assert((DQK == 64 && DV == 64) || (DQK == 128 && DV == 128) || (DQK == 192 && DV == 128),
                "FP8 kernel: (d_qk, d_v) = (64, 64), (128, 128) or (192, 128)");
  constexpr int BN = kFp8BlockN;
  constexpr int KB = BN / 32;              // 32-key blocks of S^T per tile
  constexpr int KP = BN / 64;              // 64-key steps of the output product
  constexpr int QK_STEPS = DQK / 64;       // 64-deep steps of the score product
  constexpr int DB = DV / 32;              // 32-row blocks of O^T
  constexpr int OB = DB + 1;               // + the all-ones block (row sums)
  constexpr int RBK = DQK, RBV = DV;        // bytes per K and per V row
  constexpr int TILE_K = BN * RBK, TILE_V = BN * RBV;
  constexpr int K_ISSUES = TILE_K / 1024 / kLoaders;
  constexpr int V_ISSUES = TILE_V / 1024 / kLoaders;
  constexpr int ISSUES = K_ISSUES + V_ISSUES;
  static_assert(TILE_K % (1024 * kLoaders) == 0 && TILE_V % (1024 * kLoaders) == 0, "tile split");
  constexpr int PERIOD_K = dma_period(RBK / 16, 16);   // the swizzles repeat every 16 rows
  constexpr int PERIOD_V = dma_period(RBV / 16, 16);
  constexpr int OFFS_K = K_ISSUES < PERIOD_K ? K_ISSUES : PERIOD_K;
  constexpr int OFFS_V = V_ISSUES < PERIOD_V ? V_ISSUES : PERIOD_V;
  constexpr int LDS_BYTES = kKBufs * TILE_K + kVBufs * TILE_V;
  constexpr int OS = DV + 8;                         // staged O row stride (bf16 elements)
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(kWaves * kRowsPerWave * OS * 2 <= LDS_BYTES, "O staging fits in the tile buffers");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  lds_u8_t* const lds = (lds_u8_t*)smem;
  auto kbuf = [&] __device__ (int i) __attribute__((always_inline)) { return lds + i * TILE_K; };
  auto vbuf = [&] __device__ (int i) __attribute__((always_inline)) { return lds + kKBufs * TILE_K + i * TILE_V; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int g = lane / 32;
  const int lq = lane % 32;

  // ---- work decode: the bf16 kernel's XCD-aware longest-first order
  const int W = p.H * p.B * p.n_qblocks;
  auto decode = [&] __device__ (int i, int& h, int& b, int& qblk) __attribute__((always_inline)) {
    const int x = i % kXcds, slot = i / kXcds;
    const int gi = x * (W / kXcds) + min(x, W % kXcds) + slot;
    const int pair = gi / p.n_qblocks;
    qblk = p.n_qblocks - 1 - (gi - pair * p.n_qblocks);
    h = pair / p.B;
    b = pair - h * p.B;
  };
  auto seq_range = [&] __device__ (int b, int& seq0, int& L) __attribute__((always_inline)) {
    if (p.cu_seqlens) {
      seq0 = p.cu_seqlens[b];
      L = p.cu_seqlens[b + 1] - seq0;
    } else {
      seq0 = b * p.N;
      L = p.N;
    }
  };
  int h, b, qblk;
  decode(blockIdx.x, h, b, qblk);
  int seq0, L;
  seq_range(b, seq0, L);
  const int T = p.cu_seqlens ? p.cu_seqlens[p.B] : p.B * p.N;
  const int q0 = qblk * kBlockM;
  if (q0 >= L) return;
  const int kend = CAUSAL ? min(L, q0 + kBlockM) : L;
  const int ntiles = (kend + BN - 1) / BN;
  const int H = p.H;
  const int64_t qk_row = (int64_t)H * DQK;            // bytes between consecutive tokens of q, k
  const int64_t v_row = (int64_t)H * DV;              // ... of v
  const int qw0 = q0 + kRowsPerWave * wave;
  const int qrow = qw0 + lq;

  // ---- Q^T operand: lane (g, lq) holds Q[qrow][64 ks + 32 g + i], i = 0..31
  i32x8_t qreg[QK_STEPS];
  {
    const uint32_t flip = p.neg_scale ? 0x80808080u : 0u;
    const int qr = min(qrow, L - 1);
    const uint8_t* qp = p.q + (int64_t)(seq0 + qr) * qk_row + (int64_t)h * DQK + 32 * g;
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) {
      const u32x4_t lo = *(const u32x4_t*)(qp + 64 * ks) ^ flip;
      const u32x4_t hi = *(const u32x4_t*)(qp + 64 * ks + 16) ^ flip;
      qreg[ks] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }

  // ---- K/V tile DMAs (keys past the sequence end read as zeros)
  const uint32_t k_rowbytes = (uint32_t)qk_row, v_rowbytes = (uint32_t)v_row;
  const uint8_t* const k_head = p.k + (int64_t)seq0 * qk_row + (int64_t)h * DQK;
  const uint8_t* const v_head = p.v + (int64_t)seq0 * v_row + (int64_t)h * DV;
  const uint32_t k_bytes = (uint32_t)((L - 1) * qk_row + DQK);
  const uint32_t v_bytes = (uint32_t)((L - 1) * v_row + DV);
  const u32x4_t k_rsrc = make_rsrc(k_head, k_bytes);
  const u32x4_t v_rsrc = make_rsrc(v_head, v_bytes);
  const int lw = wave % kLoaders;
  uint32_t koff[OFFS_K], voff[OFFS_V];
#pragma unroll
  for (int i = 0; i < OFFS_K; ++i) {
    const int slot = (lw * K_ISSUES + i) * 64 + lane;
    const int row = slot / (RBK / 16), pos = slot % (RBK / 16);
    koff[i] = (uint32_t)row * k_rowbytes + (uint32_t)(pos ^ k8_swz<RBK>(row)) * 16u;
  }
#pragma unroll
  for (int i = 0; i < OFFS_V; ++i) {
    const int slot = (lw * V_ISSUES + i) * 64 + lane;
    const int row = slot / (RBV / 16), pos = slot % (RBV / 16);
    voff[i] = (uint32_t)row * v_rowbytes + (uint32_t)(pos ^ v8_swz<RBV>(row)) * 16u;
  }
  const uint32_t k_period_bytes = (uint32_t)(PERIOD_K * 64 / (RBK / 16)) * k_rowbytes;
  const uint32_t v_period_bytes = (uint32_t)(PERIOD_V * 64 / (RBV / 16)) * v_rowbytes;

  u32x4_t pq_rsrc = {0u, 0u, 0u, 0u}, pk_rsrc = {0u, 0u, 0u, 0u};
  bool prefetch_next = false;
  if (p.next_stride > 0 && (int)blockIdx.x + p.next_stride < W) {
    int h2, b2, qblk2, seq2, L2;
    decode(blockIdx.x + p.next_stride, h2, b2, qblk2);
    seq_range(b2, seq2, L2);
    const int q2 = qblk2 * kBlockM;
    if (q2 < L2) {
      prefetch_next = true;
      const uint32_t qrows = (uint32_t)min(kBlockM, L2 - q2), krows = (uint32_t)min(kBlockM, L2);
      pq_rsrc = make_rsrc(p.q + (int64_t)(seq2 + q2) * qk_row + (int64_t)h2 * DQK, qrows * k_rowbytes);
      pk_rsrc = make_rsrc(p.k + (int64_t)seq2 * qk_row + (int64_t)h2 * DQK, krows * k_rowbytes);
    }
  }
  auto prefetch_l2 = [&] __device__ (lds_u8_t* garbage) __attribute__((always_inline)) {
    const int pw = wave - kWaves / 2;                  // 0..3 in group 1: one K or Q row per lane
    const uint32_t off = (uint32_t)(pw * 64 + lane) * k_rowbytes;
    dma_dword(pq_rsrc, off, (lds_u16_t*)garbage);
    dma_dword(pk_rsrc, off, (lds_u16_t*)garbage);
  };
  auto k_tile = [&] __device__ (int t) __attribute__((always_inline)) -> uint32_t {
    return t < ntiles ? (uint32_t)(t * BN) * k_rowbytes : k_bytes;
  };
  auto v_tile = [&] __device__ (int t) __attribute__((always_inline)) -> uint32_t {
    return t < ntiles ? (uint32_t)(t * BN) * v_rowbytes : v_bytes;
  };
  auto dma = [&] __device__ (int d, uint32_t tk, uint32_t tv, lds_u8_t* kdst, lds_u8_t* vdst)
      __attribute__((always_inline)) {
    if (d < V_ISSUES) {
      dma_chunk(v_rsrc, voff[d % PERIOD_V], tv + (uint32_t)(d / PERIOD_V) * v_period_bytes,
                (lds_u16_t*)(vdst + (lw * V_ISSUES + d) * 1024));
    } else {
      const int e = d - V_ISSUES;
      dma_chunk(k_rsrc, koff[e % PERIOD_K], tk + (uint32_t)(e / PERIOD_K) * k_period_bytes,
                (lds_u16_t*)(kdst + (lw * K_ISSUES + e) * 1024));
    }
  };

  // ---- LDS read addressing.  Score slot (ks, kb): K row 32 kb + lq, chunks
  // 4 ks + 2 g and 4 ks + 2 g + 1.  Output slot (kp, db): read j = 0..3 of
  // the V^T operand; lane s of 16-lane group G addresses key row
  // 64 kp + 16 j + 8 (r/4) + 4 g + r%4 (r = s/2), byte column
  // 32 db + 16 (G%2) + 8 (s%2), which hands destination lane (g, m) the keys
  // whose P sits in the same bytes of its B operand.
  int kread[QK_STEPS][2];
#pragma unroll
  for (int ks = 0; ks < QK_STEPS; ++ks)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) kread[ks][hh] = lq * RBK + (((4 * ks + 2 * g + hh) ^ k8_swz<RBK>(lq)) * 16);
  int vread[DB];
  {
    const int G = lane / 16, s = lane % 16, r = s / 2;
    const int row0 = 8 * (r / 4) + 4 * g + (r % 4);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vread[db] = row0 * RBV + (((2 * db + (G % 2)) ^ v8_swz<RBV>(row0)) * 16) + 8 * (s % 2);
  }

  // ---- per-wave state
  f32x16_t sacc[KB];
  float mx_raw = -__builtin_inff();
  i32x8_t pb[KP];
#pragma unroll
  for (int kp = 0; kp < KP; ++kp) pb[kp] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  f32x16_t oacc[OB];
#pragma unroll
  for (int ob = 0; ob < OB; ++ob)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[ob][r] = 0.0f;
  float m_run = -__builtin_inff();
  const float c = p.c;
  const float tau_dec =
      __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __builtin_fmaxf(p.tau, 0.0f))));

  auto row_max = [&] __device__ () __attribute__((always_inline)) -> float {
    float mx0 = sacc[0][0], mx1 = sacc[0][1];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2) {
        mx0 = __builtin_fmaxf(mx0, sacc[kb][r]);
        mx1 = __builtin_fmaxf(mx1, sacc[kb][r + 1]);
      }
    return max_with_partner(__builtin_fmaxf(mx0, mx1));
  };

  constexpr int NQK = QK_STEPS * KB;
  constexpr int NS = NQK + KP * OB;
  constexpr int kDmaStride = NS / ISSUES;
  // the operands read ahead at the end of the previous phase are score slots
  // (K tile, awaited before that point); V tiles are awaited later
  static_assert(kDmaStride >= 1 && kFp8Prefetch <= NQK, "matrix-phase slots");
  const i32x8_t ones = {(int)kE4m3One, (int)kE4m3One, (int)kE4m3One, (int)kE4m3One,
                        (int)kE4m3One, (int)kE4m3One, (int)kE4m3One, (int)kE4m3One};
  auto read_op = [&] __device__ (int s, const lds_u8_t* vt, const lds_u8_t* kt) __attribute__((always_inline))
      -> i32x8_t {
    if (s < NQK) {
      const int ks = s / KB, kb = s % KB;
      const u32x4_t lo = *(const lds_u32x4_t*)(kt + kread[ks][0] + kb * 32 * RBK);
      const u32x4_t hi = *(const lds_u32x4_t*)(kt + kread[ks][1] + kb * 32 * RBK);
      return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const int q = s - NQK, kp = q / OB, db = q % OB;
    if (db == DB) return ones;
    const lds_u8_t* vr = vt + vread[db] + 64 * kp * RBV;
    const i32x2_t r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vr));
    const i32x2_t r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vr + 16 * RBV));
    const i32x2_t r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vr + 32 * RBV));
    const i32x2_t r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vr + 48 * RBV));
    return i32x8_t{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
  };
  i32x8_t op_pre[kFp8Prefetch];
  auto prefetch = [&] __device__ (const lds_u8_t* vt, const lds_u8_t* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kFp8Prefetch; ++s) op_pre[s] = read_op(fp8_slot_at<NQK>(s), vt, kt);
  };
  auto matrix = [&] __device__ (auto dma_tag, const lds_u8_t* vt, const lds_u8_t* kt, uint32_t tk, uint32_t tv,
                                lds_u8_t* kdst, lds_u8_t* vdst) __attribute__((always_inline)) {
    constexpr bool DMA = decltype(dma_tag)::value;
    i32x8_t op[NS];
#pragma unroll
    for (int s = 0; s < kFp8Prefetch; ++s) op[s] = op_pre[s];
    const f32x16_t zero = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + kFp8Prefetch < NS) op[s + kFp8Prefetch] = read_op(fp8_slot_at<NQK>(s + kFp8Prefetch), vt, kt);
      const int L = fp8_slot_at<NQK>(s);
      if (L < NQK) {
        const int ks = L / KB, kb = L % KB;
        sacc[kb] = mfma_fp8(op[s], qreg[ks], ks == 0 ? zero : sacc[kb]);
      } else {
        const int q = L - NQK, kp = q / OB, db = q % OB;
        oacc[db] = mfma_fp8(op[s], pb[kp], oacc[db]);
      }
      if (DMA && s % kDmaStride == kDmaStride / 2 && s / kDmaStride < ISSUES) dma(s / kDmaStride, tk, tv, kdst, vdst);
    }
    mx_raw = row_max();
    asm volatile("" : "+v"(mx_raw));
    pin_fp8_schedule<0, NS, NQK, OB, DB>();
  };

  auto needs_mask = [&] __device__ (int t) __attribute__((always_inline)) {
    const int k0 = t * BN;
    return (k0 + BN > L) || (CAUSAL && k0 + BN - 1 > qw0);
  };
  // Softmax of tile t: masks, conditional rescale of O (and of the row-sum
  // block), P = exp2(c s - m) rounded to E4M3 into the B operands.
  auto softmax = [&] __device__ (int t) __attribute__((always_inline)) {
    const int k0 = t * BN;
    float mx = mx_raw;
    if (needs_mask(t)) {
      const int lim = CAUSAL ? min(L - 1, qrow) : (L - 1);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r / 4) + 4 * g + (r % 4);
          if (key > lim) sacc[kb][r] = -__builtin_inff();
        }
      mx = row_max();
    }
    const float m_tile = (mx == -__builtin_inff()) ? mx : mx * c;
    const bool need = m_tile > m_run + tau_dec;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? __builtin_fmaxf(m_run, m_tile) : m_run;
      const float alpha = need ? exp2_hw(m_run - m_new) : 1.0f;
#pragma unroll
      for (int ob = 0; ob < OB; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = oacc[ob][r];
          scale_in_place(x, alpha);
          oacc[ob][r] = x;
        }
      m_run = m_new;
    }
    const float neg_m = -m_run;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = __builtin_fmaf(sacc[kb][r], c, neg_m);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = exp2_hw(sacc[kb][r]);
    // B operand of 64-key step kp: dword w holds S^T block 2 kp + w/4,
    // registers 4 (w%4) .. 4 (w%4) + 3
#pragma unroll
    for (int kp = 0; kp < KP; ++kp)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = 2 * kp + w / 4, r = 4 * (w % 4);
        pb[kp][w] = pack_e4m3x4(sacc[kb][r], sacc[kb][r + 1], sacc[kb][r + 2], sacc[kb][r + 3], pb[kp][w]);
      }
  };

  auto run = [&] __device__ (auto grp_tag) __attribute__((always_inline)) {
    constexpr int G = decltype(grp_tag)::value;
    int b0 = 0;
    if (G == 0) prefetch(vbuf(1), kbuf(0));
    for (int j = 0; j <= ntiles; ++j) {
      const int bm1 = (b0 == 0) ? 2 : b0 - 1;
      const int bp1 = (b0 == 2) ? 0 : b0 + 1;
      const int vc = j & 1, vp = vc ^ 1;
      if (G == 0) {
        if (ATTN_FP8_SETPRIO) __builtin_amdgcn_s_setprio(ATTN_FP8_SETPRIO);
        matrix(True{}, vbuf(vp), kbuf(b0), k_tile(j + 2), v_tile(j), kbuf(bm1), vbuf(vc));
        if (ATTN_FP8_SETPRIO) __builtin_amdgcn_s_setprio(0);
        dma_wait_barrier<ISSUES>();              // K[j+1] has landed
        if (j < ntiles) softmax(j);
        prefetch(vbuf(vc), kbuf(bp1));
        dma_wait_barrier<K_ISSUES>();            // V[j] has landed
      } else {
        if (prefetch_next && j == ntiles - 1) prefetch_l2(kbuf(bm1));
        if (j >= 1 && j - 1 < ntiles) softmax(j - 1);
        prefetch(vbuf(vp), kbuf(b0));
        barrier();
        if (ATTN_FP8_SETPRIO) __builtin_amdgcn_s_setprio(ATTN_FP8_SETPRIO);
        matrix(False{}, vbuf(vp), kbuf(b0), 0u, 0u, kbuf(bm1), vbuf(vc));
        if (ATTN_FP8_SETPRIO) __builtin_amdgcn_s_setprio(0);
        barrier();
      }
      b0 = bp1;
    }
  };
  for (int i = tid; i < TILE_V / 16; i += kThreads) ((lds_u32x4_t*)vbuf(1))[i] = u32x4_t{0u, 0u, 0u, 0u};
  if (wave < kWaves / 2) {
#pragma unroll
    for (int d = V_ISSUES; d < ISSUES; ++d) dma(d, k_tile(0), 0u, kbuf(0), vbuf(0));
#pragma unroll
    for (int d = V_ISSUES; d < ISSUES; ++d) dma(d, k_tile(1), 0u, kbuf(1), vbuf(0));
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
  if (wave < kWaves / 2) run(Grp0{});
  else run(Grp1{});
  dma_wait_all();

  // ---- epilogue: O = v_descale * O^T / l (bf16), LSE = (m + log2 l) ln 2;
  // every row of the all-ones block holds l
  barrier();
  const float l_tot = oacc[DB][0];
  const float inv = p.o_scale / l_tot;
  lds_u16_t* const ost = (lds_u16_t*)lds + wave * kRowsPerWave * OS;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2_t w;
      w.x = pack_bf16x2(oacc[db][4 * jj + 0] * inv, oacc[db][4 * jj + 1] * inv);
      w.y = pack_bf16x2(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
      *(__attribute__((address_space(3))) u32x2_t*)(ost + lq * OS + db * 32 + 8 * jj + 4 * g) = w;
    }
  {
    constexpr int CPR = DV / 8;
    constexpr int RPI = 64 / CPR;
    const int cc = lane % CPR;
#pragma unroll
    for (int i = 0; i < kRowsPerWave / RPI; ++i) {
      const int r = i * RPI + lane / CPR;
      const u32x4_t w = *(const lds_u32x4_t*)(ost + r * OS + cc * 8);
      if (qw0 + r < L) *(u32x4_t*)(p.o + (int64_t)(seq0 + qw0 + r) * H * DV + (int64_t)h * DV + cc * 8) = w;
    }
  }
  if (qrow < L && g == 0)
    p.lse[(int64_t)h * T + seq0 + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.693147180559945309f;
}

template <int DQK, int DV>
static hipError_t launch_fp8_dims(const Fp8Params& p, bool causal, hipStream_t s) {
  const dim3 grid(p.H * p.B * p.n_qblocks), block(kThreads);
  if (causal) hipLaunchKernelGGL((attn_fwd_fp8_kernel<DQK, DV, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((attn_fwd_fp8_kernel<DQK, DV, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Params& p, int d_qk, int d_v, bool causal, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return launch_fp8_dims<64, 64>(p, causal, s);
  if (d_qk == 128 && d_v == 128) return launch_fp8_dims<128, 128>(p, causal, s);
  if (d_qk == 192 && d_v == 128) return launch_fp8_dims<192, 128>(p, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
