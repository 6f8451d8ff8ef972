// Fused exact-attention forward kernels for gfx950 (CDNA4, MI355X).
//
// One workgroup = 8 wave64s (two per SIMD) = one query block of 256 rows of
// one (sequence, head); each wave owns 32 query rows for the whole key loop.
// Key tiles of 64 keys are staged row-major in LDS (K and V, two stages: the
// next tile's global loads are in flight while the current tile is used); each
// wave then computes
//
//   S^T = K Q^T      bf16 MFMA 32x32x16, fp32 accumulators (Q^T resident in VGPRs)
//   online softmax   row max / conditional rescale / exp2 / row sum, in fp32
//   O^T += V^T P^T   bf16 MFMA 32x32x16, fp32 accumulators; the V^T operand
//                    comes straight from the row-major V tile through the
//                    gfx950 transposing LDS read (ds_read_b64_tr_b16)
//
// Computing the transposed score block puts one query row in each lane (lane
// l and lane l^32 hold the two halves of the row's keys), so the row max and
// row sum are lane-local plus one cross-half exchange, the rescale factor is
// a per-lane scalar, and the fp32 S^T accumulator -- rounded to bf16 -- is
// already the B operand of the second product: P never leaves the registers.
//
// Method sources (web pages on FlashAttention-4):
//  * tiling + online softmax with running max/sum: ainexis.cn deep dive,
//    background section and "horizontal extension" concept two; jsqmd news,
//    section two.
//  * conditional rescaling with threshold 8 in log2 units (factor 256), exact
//    after the final normalisation: wittx news "FlashAttention-4", section on
//    skipping 90% of rescales.
//  * exp2 by range reduction plus a Horner cubic on FMA for part of the
//    elements, hardware exp for the rest: wittx, section on faking a hardware
//    instruction in software; jsqmd section four, item 1.
//  * longest-first causal/varlen tile scheduling: newton.com.tw wiki
//    "FlashAttention-4", core-technology section.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_kernel.h"

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Cubic p(r) = 1 + C1 r + C2 r^2 + C3 r^3 minimising max |p(r)/2^r - 1| on
// [0, 1] (relative minimax, max error 8.56e-5), rounded to fp32.  Derived by
// gen_exp2_coeffs.py in this directory (a linear program on a dense grid).
constexpr float kExp2C1 = 0x1.63e66ap-1f;   // 0.695117295
constexpr float kExp2C2 = 0x1.d236c6p-3f;   // 0.227643535
constexpr float kExp2C3 = 0x1.3babb0p-4f;   // 0.0770680308

constexpr int kWave = 64;
constexpr int kWaves = 8;              // 2 waves per SIMD
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kRowsPerWave * kWaves;   // query rows per workgroup
constexpr int kBlockN = 64;            // keys per tile
constexpr int kKeyBlocks = kBlockN / 32;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

__device__ __forceinline__ float exp2_hw(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// 2^y = 2^n * p(r), n = floor(y), r = y - n in [0, 1).  y is clamped at -127
// first so that -inf (a masked key) gives a value below 2^-126 instead of NaN;
// such a term is under 2^-126 of the row's largest term.
__device__ __forceinline__ float exp2_poly(float y) {
  y = __builtin_fmaxf(y, -127.0f);
  const float n = __builtin_floorf(y);
  const float r = y - n;
  const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(kExp2C3, r, kExp2C2), r, kExp2C1), r, 1.0f);
  return __builtin_amdgcn_ldexpf(p, (int)n);
}

// Exchange a value with the partner lane l ^ 32 and combine.  The pair
// {a, b} returned by the swap is {x[l], x[l^32]} in some order on every lane,
// so max and sum are exact and identical on both lanes.
__device__ __forceinline__ float max_with_partner(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo;   // round to nearest even
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// LDS tile layouts (bf16 elements, row-major, padded rows):
//  K tile [kBlockN][DQK + 8]: the 16-byte pad shifts consecutive rows by 4
//    banks, so the 16 rows one ds_read_b128 phase touches (same column chunk)
//    land in 16 distinct 4-bank groups.
//  V tile [kBlockN][DV + 32]: the 64-byte pad shifts consecutive rows by 16
//    banks, so the 4 rows x 64 bytes a half-wave of ds_read_b64_tr_b16 reads
//    cover all 64 banks once.
template <int DQK, int DV>
struct TileLayout {
  static constexpr int K_PITCH = DQK + 8;
  static constexpr int V_PITCH = DV + 32;
  static constexpr int K_ELEMS = kBlockN * K_PITCH;
  static constexpr int V_ELEMS = kBlockN * V_PITCH;
  static constexpr int STAGE_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int K_CHUNKS = kBlockN * DQK / 8;   // 16-byte chunks per K tile
  static constexpr int V_CHUNKS = kBlockN * DV / 8;
  static constexpr int K_LOADS = (K_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int V_LOADS = (V_CHUNKS + kThreads - 1) / kThreads;
};

template <int DQK, int DV, bool CAUSAL, int NPOLY>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(FwdParams p) {
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims");
  using Lay = TileLayout<DQK, DV>;
  constexpr int QK_STEPS = DQK / 16;             // MFMA k-steps for S^T
  constexpr int D_BLOCKS = DV / 32;              // 32-row blocks of O^T

  // two stages, each holding one K tile and one V tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Lay::STAGE_ELEMS];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int g = lane / 32;       // lane half
  const int lq = lane % 32;      // query column within the wave

  // ---- work decode: blockIdx = (head, sequence, query-block slot)
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int qblk = (p.schedule == 0) ? (p.n_qblocks - 1 - (int)blockIdx.z) : (int)blockIdx.z;
  int seq0, L, T;
  if (p.cu_seqlens) {
    seq0 = p.cu_seqlens[b];
    L = p.cu_seqlens[b + 1] - seq0;
    T = p.cu_seqlens[p.B];
  } else {
    seq0 = b * p.N;
    L = p.N;
    T = p.B * p.N;
  }
  const int q0 = qblk * kBlockM;
  if (q0 >= L) return;  // uniform over the workgroup
  const int kend = CAUSAL ? min(L, q0 + kBlockM) : L;
  const int ntiles = (kend + kBlockN - 1) / kBlockN;

  const int H = p.H;
  const int64_t qk_row = (int64_t)H * DQK;   // elements between consecutive tokens
  const int64_t v_row = (int64_t)H * DV;
  const uint16_t* __restrict__ kbase = p.k + (int64_t)seq0 * qk_row + (int64_t)h * DQK;
  const uint16_t* __restrict__ vbase = p.v + (int64_t)seq0 * v_row + (int64_t)h * DV;

  const int qw0 = q0 + kRowsPerWave * wave;   // first query row of this wave
  const int qrow = qw0 + lq;                  // this lane's query row (position in the sequence)
  const bool row_valid = qrow < L;

  // ---- Q^T operand, resident for the whole key loop.  Lane (g, lq) holds
  // Q[qrow][16*ks + 8*g + i], i = 0..7, for every k-step ks.
  bf16x8_t qreg[QK_STEPS];
  {
    const int qr = min(qrow, L - 1);
    const uint16_t* qp = p.q + (int64_t)(seq0 + qr) * qk_row + (int64_t)h * DQK + 8 * g;
    const uint32_t flip = p.neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) {
      u32x4_t raw = *(const u32x4_t*)(qp + 16 * ks);
      raw ^= flip;
      qreg[ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  // ---- staging registers for the next K/V tile (global -> VGPR -> LDS)
  u32x4_t kst[Lay::K_LOADS];
  u32x4_t vst[Lay::V_LOADS];

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < Lay::K_LOADS; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / (DQK / 8);
      const int col8 = c % (DQK / 8);
      const int key = k0 + row;
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (c < Lay::K_CHUNKS && key < L) val = *(const u32x4_t*)(kbase + (int64_t)key * qk_row + col8 * 8);
      kst[i] = val;
    }
#pragma unroll
    for (int i = 0; i < Lay::V_LOADS; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / (DV / 8);
      const int col8 = c % (DV / 8);
      const int key = k0 + row;
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (c < Lay::V_CHUNKS && key < L) val = *(const u32x4_t*)(vbase + (int64_t)key * v_row + col8 * 8);
      vst[i] = val;
    }
  };

  auto store_tile = [&](int stage) {
    lds_u16_t* ks_ = (lds_u16_t*)smem + stage * Lay::STAGE_ELEMS;
    lds_u16_t* vs_ = ks_ + Lay::K_ELEMS;
#pragma unroll
    for (int i = 0; i < Lay::K_LOADS; ++i) {
      const int c = i * kThreads + tid;
      if (c < Lay::K_CHUNKS) {
        const int row = c / (DQK / 8);
        const int col8 = c % (DQK / 8);
        *(lds_u32x4_t*)(ks_ + row * Lay::K_PITCH + col8 * 8) = kst[i];
      }
    }
#pragma unroll
    for (int i = 0; i < Lay::V_LOADS; ++i) {
      const int c = i * kThreads + tid;
      if (c < Lay::V_CHUNKS) {
        const int row = c / (DV / 8);
        const int col8 = c % (DV / 8);
        *(lds_u32x4_t*)(vs_ + row * Lay::V_PITCH + col8 * 8) = vst[i];
      }
    }
  };

  // ---- running state: O^T accumulators, row max (log2 units), lane-partial row sum
  f32x16_t oacc[D_BLOCKS];
#pragma unroll
  for (int db = 0; db < D_BLOCKS; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -__builtin_inff();
  float l_part = 0.0f;
  const float c = p.c;
  const float tau = p.tau;
  uint32_t n_considered = 0, n_taken = 0, n_tiles = 0;
  bool first = true;

  // K rows are read in the order sigma(m) = m with bits 2 and 3 swapped: then
  // accumulator registers 0..7 (and 8..15) of a 32-key block hold 8
  // consecutive keys -- exactly the B-operand slots of the second product.
  const int sig = (lq & ~0xC) | ((lq & 4) << 1) | ((lq & 8) >> 1);
  // ds_read_b64_tr_b16 source addressing for the V^T operand: in each group of
  // 16 lanes, lane s reads 4 consecutive d-values of key row s/4; the
  // transpose hands lane i the values of 4 consecutive keys at d-column i.
  const int grp = lane / 16;
  const int sl = lane % 16;
  const int v_key_off = 8 * (grp / 2) + sl / 4;
  const int v_col_off = 16 * (grp % 2) + 4 * (sl % 4);

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kBlockN;
    const int stage = t & 1;
    if (t + 1 < ntiles) load_tile(k0 + kBlockN);

    if (!CAUSAL || k0 <= qw0 + kRowsPerWave - 1) {   // else: every key is above this wave's rows
      ++n_tiles;
      const lds_u16_t* ks_ = (const lds_u16_t*)smem + stage * Lay::STAGE_ELEMS;
      const lds_u16_t* vs_ = ks_ + Lay::K_ELEMS;

      // ---- S^T = K Q^T
      f32x16_t sacc[kKeyBlocks];
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < QK_STEPS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb) {
          const bf16x8_t a = *(const lds_bf16x8_t*)(ks_ + (kb * 32 + sig) * Lay::K_PITCH + 16 * ks + 8 * g);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[kb], 0, 0, 0);
        }
      }

      // ---- mask (only tiles that reach past the sequence end or this wave's diagonal)
      const bool need_mask = (k0 + kBlockN > L) || (CAUSAL && k0 + kBlockN - 1 > qw0);
      if (need_mask) {
        const int lim = CAUSAL ? min(L - 1, qrow) : (L - 1);   // last visible key
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 16 * (r / 8) + 8 * g + (r % 8);
            if (key > lim) sacc[kb][r] = -__builtin_inff();
          }
      }

      // ---- row max of this tile (raw logits; c > 0 so max commutes with scaling)
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sacc[kb][r]);
      mx = max_with_partner(mx);
      const float m_tile = (mx == -__builtin_inff()) ? mx : mx * c;

      // ---- conditional rescale
      if (first) {
        m_run = m_tile;   // O and l are still zero: nothing to rescale
        first = false;
      } else {
        bool need;
        float m_new;
        if (tau < 0.0f) {                 // classic online softmax: always rescale
          m_new = __builtin_fmaxf(m_run, m_tile);
          need = true;
        } else {
          need = m_tile > m_run + tau;
          m_new = need ? m_tile : m_run;
        }
        if (row_valid && g == 0) {
          n_considered += 1;
          n_taken += need ? 1u : 0u;
        }
        if (tau < 0.0f || __builtin_amdgcn_ballot_w64(need) != 0) {
          const float alpha = need ? exp2_hw(m_run - m_new) : 1.0f;
#pragma unroll
          for (int db = 0; db < D_BLOCKS; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          l_part *= alpha;
          m_run = m_new;
        }
      }

      // ---- P = exp2(c*s - m), row sum, bf16 B operand
      u32x4_t pb[kKeyBlocks][2];
      const float neg_m = -m_run;
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float y = __builtin_fmaf(sacc[kb][r], c, neg_m);
          pv[r] = ((r % 8) < NPOLY / 2) ? exp2_poly(y) : exp2_hw(y);
          l_part += pv[r];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int j = 0; j < 4; ++j) pb[kb][hh][j] = pack_bf16x2(pv[8 * hh + 2 * j], pv[8 * hh + 2 * j + 1]);
      }

      // ---- O^T += V^T P^T  (V^T operand by transposing LDS reads)
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, pb[kb][hh]);
          const lds_u16_t* vrow = vs_ + (kb * 32 + 16 * hh + v_key_off) * Lay::V_PITCH + v_col_off;
#pragma unroll
          for (int db = 0; db < D_BLOCKS; ++db) {
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vrow + db * 32));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vrow + 4 * Lay::V_PITCH + db * 32));
            const i16x4_t both[2] = {lo, hi};
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, both);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, oacc[db], 0, 0, 0);
          }
        }
    }

    if (t + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l (bf16), LSE = (m + log2 l) ln 2
  const float l_tot = sum_with_partner(l_part);
  if (row_valid) {
    const float inv = 1.0f / l_tot;
    uint16_t* op = p.o + (int64_t)(seq0 + qrow) * H * DV + (int64_t)h * DV;
#pragma unroll
    for (int db = 0; db < D_BLOCKS; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2_t w;
        w.x = pack_bf16x2(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
        *(u32x2_t*)(op + db * 32 + 8 * j + 4 * g) = w;
      }
    if (g == 0) {
      p.lse[(int64_t)h * T + seq0 + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.693147180559945309f;
    }
  }

  if (p.stats) {
    // wave totals -> one atomic per counter per wave
    for (int off = 32; off > 0; off >>= 1) {
      n_considered += __shfl_xor(n_considered, off);
      n_taken += __shfl_xor(n_taken, off);
    }
    if (lane == 0) {
      atomicAdd((unsigned long long*)&p.stats[0], (unsigned long long)n_considered);
      atomicAdd((unsigned long long*)&p.stats[1], (unsigned long long)n_taken);
      atomicAdd((unsigned long long*)&p.stats[2], (unsigned long long)n_tiles);
      if (wave == 0) atomicAdd((unsigned long long*)&p.stats[3], 1ull);
    }
  }
}

__global__ void exp2_debug_kernel(const float* __restrict__ x, float* __restrict__ y, int n, int use_poly) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = use_poly ? exp2_poly(x[i]) : exp2_hw(x[i]);
}

template <int DQK, int DV, bool CAUSAL>
static hipError_t launch_poly(const FwdParams& p, int npoly, hipStream_t s) {
  const dim3 grid(p.H, p.B, p.n_qblocks);
  const dim3 block(kThreads);
  switch (npoly) {
    case 0: hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, CAUSAL, 0>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, CAUSAL, 2>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, CAUSAL, 4>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, CAUSAL, 8>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t launch_dims(const FwdParams& p, bool causal, int npoly, hipStream_t s) {
  return causal ? launch_poly<DQK, DV, true>(p, npoly, s) : launch_poly<DQK, DV, false>(p, npoly, s);
}

int query_block_rows() { return kBlockM; }
int keys_per_tile() { return kBlockN; }
int rows_per_wave() { return kRowsPerWave; }

hipError_t launch_fwd(const FwdParams& p, int d_qk, int d_v, bool causal, int npoly, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return launch_dims<64, 64>(p, causal, npoly, s);
  if (d_qk == 128 && d_v == 128) return launch_dims<128, 128>(p, causal, npoly, s);
  if (d_qk == 192 && d_v == 128) return launch_dims<192, 128>(p, causal, npoly, s);
  return hipErrorInvalidValue;
}

hipError_t launch_exp2_debug(const float* x, float* y, int n, int use_poly, hipStream_t s) {
  const int threads = 256;
  hipLaunchKernelGGL(exp2_debug_kernel, dim3((n + threads - 1) / threads), dim3(threads), 0, s, x, y, n, use_poly);
  return hipGetLastError();
}

}  // namespace attn
