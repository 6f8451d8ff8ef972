// Exact-attention backward kernels for gfx950 (CDNA4, MI355X).
//
// What they compute: the gradients of O = softmax(scale Q K^T [+ causal mask]) V
// with respect to Q, K and V, given dO and the forward pass's O and LSE --
// the backward pass of the FlashAttention-4 pages (wittx, section on
// backward-pass optimisation; newton wiki, core-technology section): per
// (sequence, head), with P recomputed from the stored LSE,
//
//   D_i   = dO_i . O_i                      (row term of the softmax Jacobian)
//   P_ij  = exp(scale q_i.k_j - LSE_i)      (= 2^(c s_ij - LSE_i log2 e), c = scale log2 e)
//   dV    = P^T dO        dP = dO V^T       dS = P * (dP - D)
//   dQ    = scale dS K    dK = scale dS^T Q
//
// The pages' design reduces dQ over the key sequence with global atomic adds
// (halved there by pairing two thread blocks) and offers a deterministic
// mode that serialises those reductions.  Here no step reduces across
// workgroups: one kernel owns a block of 128 keys and accumulates its dK and
// dV over every query tile that sees those keys; a second owns a block of
// 128 queries and accumulates its dQ over the key tiles.  Each recomputes the
// score and dP tiles it needs (7 matrix products instead of 5), and the
// results are bitwise reproducible run to run.
//
// Layout of the work on the chip: each wave owns 32 rows of its workgroup's
// block; the streamed operands (Q and dO for dK/dV, K and V for dQ) are
// staged in LDS once per workgroup and read by all its waves.  Every kernel
// keeps each wave within 256 registers so that each SIMD runs two waves, in
// two groups that alternate matrix and VALU phases as the forward kernel
// does: the dQ kernel as one 8-wave workgroup of 256 queries whose waves each
// do all three products; the dK/dV kernel, up to d = 128, as one 8-wave
// workgroup of 128 keys whose two groups split the query blocks, with K in
// registers and V read from LDS, and at (192, 128) as one 8-wave workgroup
// whose two halves split the products between them (at d <= 128 too with
// ATTN_BWD_DKDV_PP=0).  The matrix products are v_mfma_f32_32x32x16_bf16
// with fp32 accumulators:
//   dQ kernel   S^T = K Q^T, dP^T = V dO^T     (K, V rows from LDS; Q, dO in registers)
//               dQ^T += K^T dS^T               (K^T by the transposing LDS read)
//   dK/dV       S = Q K^T, dP = dO V^T         (Q, dO rows from LDS; up to d = 128 K rows
//                                               in registers and V rows from LDS, both in
//                                               registers at (192, 128))
//               dV^T += dO^T P, dK^T += Q^T dS (dO^T, Q^T by the transposing read);
//               at (192, 128) S, P, dV^T in one wave group and dP, dS, dK^T in the other
// With the streamed tile's rows read in an order with bits 2 and 3 of the
// row index swapped, accumulator registers 0..7 and 8..15 of a 32 x 32
// block hold 8 consecutive rows -- the B-operand slots of the next product --
// so P and dS go from the accumulators to bf16 B operands in registers.  A
// tile read both row-wise and transposed is stored once, in a row layout whose
// swizzle keeps both kinds of read free of bank conflicts (RowSwz below), and
// the streamed tiles are copied HBM/L2 -> LDS by buffer_load ... lds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bwd_kernel.h"
#include "attn_fwd_common.h"   // LDS DMA requests, buffer resources, barriers (namespace attn)

#ifndef ATTN_BWD_PREFETCH
#define ATTN_BWD_PREFETCH 1  // dK/dV: a block's transposed operands read a phase early (d_qk = 192: dV group only)
#endif

namespace attn_grad {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef __attribute__((address_space(3))) float lds_f32_t;

constexpr int kWave = 64;
constexpr int kWaves = 4;                     // one per SIMD
constexpr int kThreads = kWave * kWaves;
constexpr int kThreads2 = 2 * kThreads;              // the 8-wave (two-group) kernels
constexpr int kRows = 32;                     // block rows per wave
constexpr int kBlock = kRows * kWaves;        // block rows per workgroup
constexpr int kTile = 64;                     // streamed rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

int block_rows() { return kBlock; }

// LDS layout of a tile of rows r with D bf16 columns (R = D/8 chunks of 16
// bytes): chunk c of row r sits at position c ^ f(r).  The row layout is
//    read 16 bytes per lane with 16 consecutive rows per
//    quarter-wave, and by ds_read_b64_tr_b16 (4 rows x 4 consecutive chunks
//    per half-wave, rows r0..r0+3 with r0 a multiple of 4): for R = 16 every
//    row starts at bank 0, and f(r) = 4 (r mod 4) + (r/4) mod 4 (the two
//    2-bit halves of r mod 16 swapped) is a permutation of the 16 rows of a
//    quarter-wave, while its upper two bits, r mod 4, tell the 4 rows of a
//    transposing read apart; for R = 8 or 24 a row starts on alternate halves
//    of the 64 banks, so the 4-bank group of chunk c of row r is
//    (c ^ f(r) ^ 8 (r mod 2)) mod 16, and f(r) = 4 b1(r) + (r/4) mod 4 (bits of
//    r/2 rotated) does the same.  Tiles read both ways are stored once.
// f is invariant under a shift of r by a multiple of 16 and keeps c ^ f(r) < R:
// for R = 16 it is a 4-bit value, for R = 8 and 24 f < 8 keeps a chunk inside
// its aligned group of 8.
template <int D>
struct RowSwz {
  static_assert(D == 64 || D == 128 || D == 192, "head dims 64, 128 and 192");
  __device__ static int f(int r) {
    return (D == 128) ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
};

// Two fp32 values -> two bf16 (round to nearest even) in one dword, low first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ int total_tokens(const BwdParams& p) {
  return p.cu_seqlens ? p.cu_seqlens[p.B] : p.B * p.N;
}
__device__ __forceinline__ void seq_range(const BwdParams& p, int b, int& seq0, int& L) {
  if (p.cu_seqlens) {
    seq0 = p.cu_seqlens[b];
    L = p.cu_seqlens[b + 1] - seq0;
  } else {
    seq0 = b * p.N;
    L = p.N;
  }
}

// Work decode of a 1-D grid of W = B*H*n_blocks workgroups.  The hardware
// deals workgroup i to XCD i mod 8; XCD x takes a contiguous run of a list
// ordered by (head, sequence) pair and block within the pair, so the blocks
// of one pair run on one XCD and share its L2 for the pair's streamed tiles.
// reverse: blocks of a pair in decreasing order (longest first for the
// causal dQ kernel, whose block b visits b+1 key tiles).
constexpr int kXcds = 8;
__device__ __forceinline__ void decode_block_n(const BwdParams& p, int n_blocks, bool reverse, int& h, int& b,
                                               int& blk) {
  const int W = p.B * p.H * n_blocks;
  const int i = blockIdx.x;
  const int x = i % kXcds, slot = i / kXcds;
  const int g = x * (W / kXcds) + min(x, W % kXcds) + slot;
  const int pair = g / n_blocks;
  blk = g - pair * n_blocks;
  if (reverse) blk = n_blocks - 1 - blk;
  h = pair / p.B;
  b = pair - h * p.B;
}
__device__ __forceinline__ void decode_block(const BwdParams& p, bool reverse, int& h, int& b, int& blk) {
  decode_block_n(p, p.n_blocks, reverse, h, b, blk);
}

template <bool V>
struct GroupTag { static constexpr bool value = V; };

// Workgroup barrier; in the race-check build (ATTN_RACE_CHECK, see
// attn_fwd_common.h) every memory access of the wave is drained first and the
// barrier is passed twice.
__device__ __forceinline__ void block_sync() {
  __syncthreads();
#if ATTN_RACE_CHECK && defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
}

// Row sigma(m): m with bits 2 and 3 swapped.
__device__ __forceinline__ int sigma(int m) { return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1); }

// ---- D = rowsum(dO * O) over d_v, one row (t, h) per DV/8 lanes.
template <int DV>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(BwdParams p) {
  constexpr int LPR = DV / 8;                 // lanes per row, 16 bytes each
  constexpr int RPB = kThreads / LPR;         // rows per workgroup
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;   // row = t H + h
  const int c = threadIdx.x % LPR;
  const int T = total_tokens(p);
  const int64_t nrows = (int64_t)T * p.H;
  float acc = 0.0f;
  if (row < nrows) {
    const u32x4_t a = *(const u32x4_t*)(p.o + row * DV + c * 8);
    const u32x4_t d = *(const u32x4_t*)(p.dout + row * DV + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(a[i]) * bf16_lo(d[i]) + bf16_hi(a[i]) * bf16_hi(d[i]);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < nrows && c == 0) {
    const int t = (int)(row / p.H), h = (int)(row % p.H);
    p.delta[(int64_t)h * T + t] = acc;
  }
}

// Per-lane LDS element offsets in a row-layout tile.  Row reads (A operand,
// 32 rows in sigma order, k-step s: 8 columns from 16 s + 8 g); transposed
// reads (A operand: columns db*32 + (lane % 32) at 8 consecutive rows from
// 8 g, as two 4-row reads; the row layout's swizzle differs between the two
// groups of 4 rows, so each has its own offset).
template <int D>
struct Reads {
  int row[D / 16];
  int tr[D / 32];
  int tr_hi[D / 32];
  __device__ Reads(int lane) {
    const int g = lane / 32, sig = sigma(lane % 32);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) row[s] = sig * D + (((2 * s + g) ^ RowSwz<D>::f(sig)) * 8);
    // in each group of 16 lanes, lane s reads 4 consecutive columns of row
    // s/4 (+ 8 for the upper lane groups); the transpose hands lane i the
    // values of 4 consecutive rows at column i
    const int lg = lane / 16, sl = lane % 16, vrow = 8 * (lg / 2) + sl / 4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + 16 * (lg % 2) + 4 * (sl % 4);
      tr[db] = vrow * D + (((d / 8) ^ RowSwz<D>::f(vrow)) * 8) + (d % 8);
      tr_hi[db] = (vrow + 4) * D + (((d / 8) ^ RowSwz<D>::f(vrow + 4)) * 8) + (d % 8);
    }
  }
};
template <int D>
__device__ __forceinline__ bf16x8_t read_row(const lds_u16_t* tile, const Reads<D>& rd, int s, int blk) {
  return *(const lds_bf16x8_t*)(tile + rd.row[s] + blk * 32 * D);
}
// rows r0 .. r0+15 (r0 a multiple of 16), column block db
template <int D>
__device__ __forceinline__ bf16x8_t read_tr(const lds_u16_t* tile, const Reads<D>& rd, int db, int r0) {
  const lds_u16_t* a = tile + rd.tr[db] + r0 * D;
  const lds_u16_t* a_hi = tile + rd.tr_hi[db] + r0 * D;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a_hi));
  const i16x4_t both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8_t, both);
}

// 8 bf16 at row `row` of a [.., H, D] tensor, columns 16 s + 8 g (zeros if !ok)
template <int D>
__device__ __forceinline__ void load_b_operand(bf16x8_t (&reg)[D / 16], const uint16_t* t, int64_t row, int H, int h,
                                               int g, bool ok) {
  const uint16_t* ptr = t + row * (int64_t)H * D + (int64_t)h * D + 8 * g;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const u32x4_t raw = ok ? *(const u32x4_t*)(ptr + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
    reg[s] = __builtin_bit_cast(bf16x8_t, raw);
  }
}

// Stage a wave's 32 x D transposed accumulator blocks (column = lane % 32 =
// output row, register r of block db = column db*32 + 8(r/4) + 4g + r%4)
// times `mul` as bf16 rows in LDS (row stride D + 8), then store whole rows
// to out[(row0 + r), h, :] for r < nvalid.
template <int D>
__device__ __forceinline__ void store_rows(const f32x16_t (&acc)[D / 32], float mul, lds_u16_t* stage, uint16_t* out,
                                           int64_t row0, int nvalid, int H, int h, int lane) {
  constexpr int OS = D + 8;
  const int g = lane / 32, lq = lane % 32;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2_t w;
      w.x = pack_bf16x2(acc[db][4 * jj + 0] * mul, acc[db][4 * jj + 1] * mul);
      w.y = pack_bf16x2(acc[db][4 * jj + 2] * mul, acc[db][4 * jj + 3] * mul);
      *(lds_u32x2_t*)(stage + lq * OS + db * 32 + 8 * jj + 4 * g) = w;
    }
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static_assert((kRows * CPR) % kWave == 0, "whole stores");
#pragma unroll
  for (int i = 0; i < kRows * CPR / kWave; ++i) {
    const int idx = i * kWave + lane, r = idx / CPR, c = idx % CPR;
    const u32x4_t w = *(const lds_u32x4_t*)(stage + r * OS + c * 8);
    if (r < nvalid) *(u32x4_t*)(out + (row0 + r) * (int64_t)H * D + (int64_t)h * D + c * 8) = w;
  }
}

// dQ workgroups: 8 waves of 32 query rows each
constexpr int kDqWaves = 8;
constexpr int kDqThreads = kDqWaves * kWave;
constexpr int kDqBlock = kDqWaves * kRows;           // query rows per workgroup

// ---- dQ in two ping-pong wave groups: the forward kernel's schedule applied
// to the dQ pass.  One workgroup of 8 waves per block of 256 query rows; each
// wave owns 32 rows (Q and dO as B operands, LSE and D in registers) and runs,
// per key tile j (64 keys, 32 at d_qk = 192), a matrix phase -- one
// stream of MFMAs: dQ^T += K_{j-1}^T dS_{j-1}^T, S^T_j = K_j Q^T,
// dP^T_j = V_j dO^T -- and a VALU phase: P_j = 2^(c S_j - LSE log2 e) and
// dS_j = P_j (dP_j - D) as bf16 B operands of the next matrix phase.  Waves
// 0-3 (group 0) and 4-7 (group 1) put one wave of each group on every SIMD
// and run half an iteration apart, separated by workgroup barriers, so that
// one group's MFMAs overlap the other group's VALU work:
//   group 0: | matrix(j)  | VALU(j)   | matrix(j+1) | ...
//   group 1: | VALU(j-1)  | matrix(j) | VALU(j)     | ...
// K tile t lives in K buffer t mod 3 and V tile t in V buffer t mod 2; group
// 0 spreads the DMAs of tile j+1 over its matrix phase j and waits for them
// before the barrier that ends iteration j.  The buffers they fill were last
// read in iteration j-1 (K_{j-2} by the dQ product of matrix(j-1), V_{j-1} by
// its dP product).  Matrix(0)'s dQ product multiplies zero dS with the
// zero-filled K buffer 2, and matrix(ntiles)'s score and dP products read a
// tile past the sequence end (zeros) and are dropped, so every iteration runs
// the same code.  The dQ slots come first in the stream: their operands
// (K_{j-1}, resident since iteration j-2) are read at the end of the wave's
// previous phase, before the tile DMAs of the current one have landed.
// matrix-phase LDS operands read this many slots ahead (fewer at d_qk = 192,
// whose six dQ blocks leave fewer registers)
template <int DQK>
constexpr int pp_prefetch() { return DQK > 128 ? 2 : 4; }

// Per-lane LDS offsets of the row and transposing reads of a row-layout tile,
// as Reads<D>, kept only once per period: for d = 64 and 192 the
// swizzle values are below 8, so they act within each aligned group of 8
// chunks and the offsets of k-step s + 4 (column block db + 2) are those of s
// (db) plus 64 elements; d = 128 has no such period.
template <int D>
struct ReadsP {
  static constexpr bool P8 = (D != 128);
  static constexpr int NR = P8 && D / 16 > 4 ? 4 : D / 16;
  static constexpr int NT = P8 && D / 32 > 2 ? 2 : D / 32;
  int row[NR];
  int tr[NT];
  int tr_hi[NT];
  __device__ ReadsP(int lane) {
    const int g = lane / 32, sig = sigma(lane % 32);
#pragma unroll
    for (int s = 0; s < NR; ++s) row[s] = sig * D + (((2 * s + g) ^ RowSwz<D>::f(sig)) * 8);
    const int lg = lane / 16, sl = lane % 16, vrow = 8 * (lg / 2) + sl / 4;
#pragma unroll
    for (int db = 0; db < NT; ++db) {
      const int d = db * 32 + 16 * (lg % 2) + 4 * (sl % 4);
      tr[db] = vrow * D + (((d / 8) ^ RowSwz<D>::f(vrow)) * 8) + (d % 8);
      tr_hi[db] = (vrow + 4) * D + (((d / 8) ^ RowSwz<D>::f(vrow + 4)) * 8) + (d % 8);
    }
  }
  __device__ int row_at(int s) const { return row[s % NR] + (s / NR) * 64; }
  __device__ int tr_at(int db) const { return tr[db % NT] + (db / NT) * 64; }
  __device__ int tr_hi_at(int db) const { return tr_hi[db % NT] + (db / NT) * 64; }
};
template <int D>
__device__ __forceinline__ bf16x8_t read_row_p(const lds_u16_t* tile, const ReadsP<D>& rd, int s, int blk) {
  return *(const lds_bf16x8_t*)(tile + rd.row_at(s) + blk * 32 * D);
}
template <int D>
__device__ __forceinline__ bf16x8_t read_tr_p(const lds_u16_t* tile, const ReadsP<D>& rd, int db, int r0) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tile + rd.tr_at(db) + r0 * D));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tile + rd.tr_hi_at(db) + r0 * D));
  const i16x4_t both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8_t, both);
}

// Per slot of the matrix phase: LDS reads issued ahead (two transposing reads
// for a dQ slot, one 16-byte read otherwise), then the MFMA.
template <int S, int NS, int NDQ, int PF>
__device__ __forceinline__ void pin_dq_schedule() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  if constexpr (S < NS) {
    if constexpr (S + PF < NS) __builtin_amdgcn_sched_group_barrier(kDsRead, (S + PF < NDQ) ? 2 : 1, 0);
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    pin_dq_schedule<S + 1, NS, NDQ, PF>();
  }
}

// Keys per tile of the ping-pong dQ kernel: 64, or 32 at d_qk = 192, where
// the six dQ blocks leave registers for one 32-key block of S and dP.
template <int DQK>
constexpr int pp_tile_keys() { return DQK > 128 ? 32 : 64; }

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_pp_kernel(BwdParams p) {
  constexpr int BK = pp_tile_keys<DQK>();
  constexpr int QK_STEPS = DQK / 16, V_STEPS = DV / 16, QBLK = DQK / 32, KB = BK / 32;
  constexpr int K_ELEMS = BK * DQK, V_ELEMS = BK * DV;
  constexpr int kKBufs = 3, kVBufs = 2;
  constexpr int TILE_LDS = kKBufs * K_ELEMS + kVBufs * V_ELEMS;
  constexpr int OUT_ELEMS = kDqWaves * kRows * (DQK + 8);
  constexpr int LDS_ELEMS = TILE_LDS > OUT_ELEMS ? TILE_LDS : OUT_ELEMS;
  static_assert(LDS_ELEMS * 2 <= 160 * 1024, "LDS budget");
  constexpr int kLoaders = kDqWaves / 2;              // group 0 issues the tile DMAs
  constexpr int K_REQ = K_ELEMS / 512, V_REQ = V_ELEMS / 512;   // 1 KB requests per tile
  static_assert(K_ELEMS % 512 == 0 && V_ELEMS % 512 == 0, "whole requests");
  static_assert(K_REQ % kLoaders == 0 && V_REQ % kLoaders == 0, "request split");
  constexpr int K_ISS = K_REQ / kLoaders, V_ISS = V_REQ / kLoaders, ISS = K_ISS + V_ISS;
  // When D divides 512, a 1 KB request covers 512 / D whole rows and a row's
  // swizzle depends on its index mod 16, so a loader's K_ISS = D / 32 requests
  // per copy need D / 32 lane offsets shared by K and V (d_qk = d_v), with
  // the requests' row offsets in the uniform soffset; otherwise (d_qk = 192)
  // each request keeps its own lane offsets.
  constexpr bool PERIODIC = (512 % DQK == 0) && DQK == DV;
  constexpr int ROWS_REQ = PERIODIC ? 512 / DQK : 0;
  constexpr int NOFF = PERIODIC ? K_ISS : ISS;
  static_assert(!PERIODIC || (K_ISS == DQK / 32 && V_ISS == K_ISS), "one lane offset per request of a copy");
  // matrix-phase slots: dQ (kb, hh, db), then score (ks, kb), then dP (vs, kb)
  constexpr int NDQ = KB * 2 * QBLK, NQK = QK_STEPS * KB, NDP = V_STEPS * KB;
  constexpr int NS = NDQ + NQK + NDP;
  constexpr int PF = pp_prefetch<DQK>();
  static_assert(PF <= NDQ, "prefetched slots are dQ slots");
  constexpr int kDmaStride = NS / ISS;
  static_assert(kDmaStride >= 1, "DMAs per matrix phase");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[LDS_ELEMS];
  lds_u16_t* const lds = (lds_u16_t*)smem;
  auto kbuf = [&] __device__ (int i) __attribute__((always_inline)) { return lds + i * K_ELEMS; };
  auto vbuf = [&] __device__ (int i) __attribute__((always_inline)) { return lds + kKBufs * K_ELEMS + i * V_ELEMS; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / kLoaders, lw = wave % kLoaders;
  const int lane = tid % kWave, g = lane / 32, lq = lane % 32;
  const int nblk = (p.N + kDqBlock - 1) / kDqBlock;
  int h, b, blk;
  decode_block_n(p, nblk, CAUSAL, h, b, blk);
  int seq0, L;
  seq_range(p, b, seq0, L);
  const int q0 = blk * kDqBlock;
  if (q0 >= L) return;                                 // uniform over the workgroup
  const int qw0 = q0 + wave * kRows;
  const int qrow = qw0 + lq;
  const bool row_valid = qrow < L;

  bf16x8_t qreg[QK_STEPS], doreg[V_STEPS];
  load_b_operand<DQK>(qreg, p.q, seq0 + qrow, p.H, h, g, row_valid);
  load_b_operand<DV>(doreg, p.dout, seq0 + qrow, p.H, h, g, row_valid);
  const int T = total_tokens(p);
  const float lse2 = row_valid ? p.lse[(int64_t)h * T + seq0 + qrow] * kLog2e : 0.0f;
  const float dq_row = row_valid ? p.delta[(int64_t)h * T + seq0 + qrow] : 0.0f;
  const int key_lim = row_valid ? (CAUSAL ? min(L - 1, qrow) : L - 1) : -1;
  const float c = p.c;

  const ReadsP<DQK> rk(lane);                          // K rows and K^T from the row layout
  const ReadsP<DV> rv(lane);                           // V rows (the compiler shares rk's when d_v = d_qk)
  const int kend = CAUSAL ? min(L, q0 + kDqBlock) : L;
  const int ntiles = (kend + BK - 1) / BK;
  const int64_t k_row = (int64_t)p.H * DQK, v_row = (int64_t)p.H * DV;     // elements per token
  const uint32_t k_rowbytes = (uint32_t)(k_row * 2), v_rowbytes = (uint32_t)(v_row * 2);
  const uint32_t k_bytes = (uint32_t)((L - 1) * k_row * 2 + DQK * 2);
  const uint32_t v_bytes = (uint32_t)((L - 1) * v_row * 2 + DV * 2);
  const attn::u32x4_t k_rsrc = attn::make_rsrc(p.k + (int64_t)seq0 * k_row + (int64_t)h * DQK, k_bytes);
  const attn::u32x4_t v_rsrc = attn::make_rsrc(p.v + (int64_t)seq0 * v_row + (int64_t)h * DV, v_bytes);
  // byte offsets of tile t in K and V; a tile past the last one starts at
  // the resources' end, so its DMAs return zeros without touching memory
  auto k_tile = [&] __device__ (int t) __attribute__((always_inline)) -> uint32_t {
    return t < ntiles ? (uint32_t)(t * BK) * k_rowbytes : k_bytes;
  };
  auto v_tile = [&] __device__ (int t) __attribute__((always_inline)) -> uint32_t {
    return t < ntiles ? (uint32_t)(t * BK) * v_rowbytes : v_bytes;
  };
  // Lane offsets: request rr of a copy fills its 1 KB block rr; lane l writes
  // the 16 bytes at LDS position 8 l of the block, i.e. chunk `pos` of tile
  // row `row`, which holds the tile's chunk pos ^ f(row) of that row.  In the
  // periodic case the offset of request i keeps only the row within the
  // request (the request's first row, rr * ROWS_REQ with rr = lw * K_ISS + i,
  // goes into soffset); f depends on the row mod 16 and K_ISS * ROWS_REQ = 16,
  // so it depends on i, not on lw.
  uint32_t lane_off[NOFF];
#pragma unroll
  for (int i = 0; i < NOFF; ++i) {
    if constexpr (PERIODIC) {
      const int r = (8 * lane) / DQK, pos = (8 * lane % DQK) / 8;
      lane_off[i] = (uint32_t)r * k_rowbytes + (uint32_t)(pos ^ RowSwz<DQK>::f(i * ROWS_REQ + r)) * 16u;
    } else {
      const bool isv = i < V_ISS;
      const int rr = isv ? lw * V_ISS + i : lw * K_ISS + (i - V_ISS);
      const int D = isv ? DV : DQK;
      const int e = rr * 512 + 8 * lane, row = e / D, pos = (e % D) / 8;
      const int f = isv ? RowSwz<DV>::f(row) : RowSwz<DQK>::f(row);
      lane_off[i] = (uint32_t)row * (isv ? v_rowbytes : k_rowbytes) + (uint32_t)(pos ^ f) * 16u;
    }
  }
  // DMA d (0 <= d < ISS) of this loader's share of tile t: V requests first
  // (d < V_ISS), then K
  auto dma = [&] __device__ (int d, int t, lds_u16_t* kdst, lds_u16_t* vdst) __attribute__((always_inline)) {
    const bool isv = d < V_ISS;
    const int i = isv ? d : d - V_ISS;
    const int rr = lw * (isv ? V_ISS : K_ISS) + i;
    if constexpr (PERIODIC) {
      attn::dma_chunk(isv ? v_rsrc : k_rsrc, lane_off[i],
                      (isv ? v_tile(t) : k_tile(t)) + (uint32_t)(rr * ROWS_REQ) * (isv ? v_rowbytes : k_rowbytes),
                      (isv ? vdst : kdst) + rr * 512);
    } else {
      attn::dma_chunk(isv ? v_rsrc : k_rsrc, lane_off[d], isv ? v_tile(t) : k_tile(t), (isv ? vdst : kdst) + rr * 512);
    }
  };

  // per-wave state: S^T and dP^T of the tile between its two phases, dS^T as
  // bf16 B operands (zero before the first VALU phase), dQ^T accumulators
  f32x16_t sacc[KB], pacc[KB], dqacc[QBLK];
  u32x4_t dsb[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) dsb[kb][hh] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int db = 0; db < QBLK; ++db) dqacc[db] = f32x16_t{};
  const f32x16_t zero = {};

  // A operand of slot s: dQ slots read K_{j-1}^T (two transposing reads),
  // score slots a K_j row chunk, dP slots a V_j row chunk
  auto read_op = [&] __device__ (int s, const lds_u16_t* kprev, const lds_u16_t* kcur, const lds_u16_t* vcur)
      __attribute__((always_inline)) -> bf16x8_t {
    if (s < NDQ) {
      const int kb = s / (2 * QBLK), hh = (s / QBLK) % 2, db = s % QBLK;
      return read_tr_p<DQK>(kprev, rk, db, kb * 32 + 16 * hh);
    }
    if (s < NDQ + NQK) {
      const int q = s - NDQ, ks = q / KB, kb = q % KB;
      return read_row_p<DQK>(kcur, rk, ks, kb);
    }
    const int q = s - NDQ - NQK, vs = q / KB, kb = q % KB;
    if constexpr (DV == DQK) return read_row_p<DV>(vcur, rk, vs, kb);
    else return read_row_p<DV>(vcur, rv, vs, kb);
  };
  bf16x8_t op_pre[PF];
  auto prefetch = [&] __device__ (const lds_u16_t* kprev) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < PF; ++s) op_pre[s] = read_op(s, kprev, kprev, kprev);
  };
  // one matrix phase; a loader also issues the DMAs of tile tn into kdst /
  // vdst, one every kDmaStride slots
  auto matrix = [&] __device__ (auto dma_tag, const lds_u16_t* kprev, const lds_u16_t* kcur, const lds_u16_t* vcur,
                                int tn, lds_u16_t* kdst, lds_u16_t* vdst) __attribute__((always_inline)) {
    constexpr bool DMA = decltype(dma_tag)::value;
    bf16x8_t op[NS];
#pragma unroll
    for (int s = 0; s < PF; ++s) op[s] = op_pre[s];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + PF < NS) op[s + PF] = read_op(s + PF, kprev, kcur, vcur);
      if (s < NDQ) {
        const int kb = s / (2 * QBLK), hh = (s / QBLK) % 2, db = s % QBLK;
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s], __builtin_bit_cast(bf16x8_t, dsb[kb][hh]),
                                                            dqacc[db], 0, 0, 0);
      } else if (s < NDQ + NQK) {
        const int q = s - NDQ, ks = q / KB, kb = q % KB;
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s], qreg[ks], ks == 0 ? zero : sacc[kb], 0, 0, 0);
      } else {
        const int q = s - NDQ - NQK, vs = q / KB, kb = q % KB;
        pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s], doreg[vs], vs == 0 ? zero : pacc[kb], 0, 0, 0);
      }
      if (DMA && s % kDmaStride == kDmaStride / 2 && s / kDmaStride < ISS) dma(s / kDmaStride, tn, kdst, vdst);
    }
    pin_dq_schedule<0, NS, NDQ, PF>();
  };
  // VALU phase of tile t (S^T, dP^T in sacc, pacc): dS = P (dP - D) with the
  // keys this lane's query does not see masked, as bf16 B operands
  auto valu = [&] __device__ (int t) __attribute__((always_inline)) {
    const int k0 = t * BK;
    const bool masked = (k0 + BK > L) || (qw0 + kRows > L) || (CAUSAL && k0 + BK - 1 > qw0);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float ds[16];
      // keys visible to this lane's query: up to key_lim (offsets within the block)
      const int lim = masked ? key_lim - (k0 + kb * 32 + 8 * g) : 64;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = (16 * (r / 8) + (r % 8) <= lim) ? __builtin_fmaf(sacc[kb][r], c, -lse2) : -__builtin_inff();
        ds[r] = __builtin_amdgcn_exp2f(x) * (pacc[kb][r] - dq_row);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dsb[kb][hh][jj] = pack_bf16x2(ds[8 * hh + 2 * jj], ds[8 * hh + 2 * jj + 1]);
    }
  };

  // Prologue: K buffer 2 (K_{-1}) zero-filled; the loaders fetch tile 0.
  for (int i = tid; i < K_ELEMS / 8; i += kDqThreads) ((lds_u32x4_t*)kbuf(2))[i] = u32x4_t{0u, 0u, 0u, 0u};
  if (grp == 0) {
#pragma unroll
    for (int d = 0; d < ISS; ++d) dma(d, 0, kbuf(0), vbuf(0));
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
  using True = GroupTag<true>;
  using False = GroupTag<false>;
  auto run = [&] __device__ (auto grp_tag) __attribute__((always_inline)) {
    constexpr bool G0 = decltype(grp_tag)::value;
    int b0 = 0;                                        // j mod 3
    if (G0) prefetch(kbuf(2));                         // operands of matrix(0)
    for (int j = 0; j <= ntiles; ++j) {
      const int bm1 = (b0 == 0) ? 2 : b0 - 1;          // (j - 1) mod 3
      const int bp1 = (b0 == 2) ? 0 : b0 + 1;          // (j + 1) mod 3
      const int vc = j & 1;
      if (G0) {
        if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(ATTN_SETPRIO);
        matrix(True{}, kbuf(bm1), kbuf(b0), vbuf(vc), j + 1, kbuf(bp1), vbuf(vc ^ 1));
        if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
        attn::barrier();
        if (j < ntiles) valu(j);
        prefetch(kbuf(b0));                            // operands of matrix(j+1)
        attn::dma_wait_barrier<0>();                   // tile j+1 has landed
      } else {
        if (j >= 1) valu(j - 1);
        prefetch(kbuf(bm1));                           // operands of matrix(j)
        attn::barrier();
        if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(ATTN_SETPRIO);
        matrix(False{}, kbuf(bm1), kbuf(b0), vbuf(vc), 0, kbuf(bp1), vbuf(vc ^ 1));
        if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
        attn::barrier();
      }
      b0 = bp1;
    }
  };
  if (grp == 0) run(True{});
  else run(False{});
  attn::dma_wait_all();
  block_sync();                                        // the staging area overlaps the tile buffers
  store_rows<DQK>(dqacc, p.scale, lds + wave * kRows * (DQK + 8), p.dq, (int64_t)seq0 + qw0, L - qw0, p.H, h, lane);
}

// ---- dK, dV in two ping-pong wave groups (d_qk = d_v <= 128): the dQ
// kernel's schedule with the roles of queries and keys swapped.  One
// workgroup of 8 waves per block of 128 keys; waves 0-3 (group 0) and 4-7
// (group 1) own the same four 32-key slices and split the 32-query blocks,
// group 0 taking the even blocks and group 1 the odd ones, each with its own
// dK^T and dV^T accumulators (summed through LDS at the end).  K and V of the
// workgroup's keys land in LDS (64 KB at d = 128); each wave copies its 32 K
// rows into registers once (the B operands of S = Q K^T, 32 VGPRs at d = 128)
// and reads V from LDS as the B operand of dP = dO V^T, so a wave's registers
// hold its accumulators, its K rows and one block's S, dP, P and dS.  Per
// block b of its group a wave runs a matrix phase -- dV^T += dO_{b-2}^T
// P_{b-2}, dK^T += Q_{b-2}^T dS_{b-2}, S_b, dP_b, one pinned stream of
// MFMAs -- and a VALU phase (P_b
// from the LSE, dS_b = P_b (dP_b - D) as bf16 B operands); the two groups run
// half an iteration apart between workgroup barriers, so one group's MFMAs
// run beside the other's VALU work:
//   group 0: | matrix(2j)   | VALU(2j)     | matrix(2j+2) ...
//   group 1: | VALU(2j-1)   | matrix(2j+1) | VALU(2j+1)   ...
// Query blocks (Q, dO, and their LSE and D rows) rotate through five LDS
// slots, block b in slot b mod 5.  During its matrix phase of iteration j a
// group fetches its block two ahead (group 0: 2j+2, group 1: 2j+3), into the
// slot whose block was last read earlier in the same iteration or before;
// group 0 waits for it before the barrier that ends iteration j, group 1
// before the mid barrier of iteration j+1.  Blocks -2 and -1 are zero-filled
// slots multiplied by zero P and dS; blocks past the sequence end read zeros
// and are masked.
#ifndef ATTN_BWD_DKDV_PP
#define ATTN_BWD_DKDV_PP 1  // 1: this kernel at d_qk = d_v <= 128, 0: the two-group split kernel
#endif
constexpr int kKvPrefetch = 4;                       // matrix-phase slots whose operands are read ahead

#ifndef ATTN_BWD_DKDV_KREG
#define ATTN_BWD_DKDV_KREG 1  // 1: each wave keeps its K rows in registers (the S products' B operands), 0: in LDS
#endif

// The lane's index within its wave, computed at the point of use: the asm
// keeps the compiler from holding it in a register across a loop (where it
// could be spilled and reloaded with a wait on every outstanding load).
__device__ __forceinline__ uint32_t lane_id_here() {
  uint32_t l = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
#endif
  return l;
}

template <int S, int NS, int NTR, int STEPS>
__device__ __forceinline__ void pin_kv_schedule() {
  constexpr int kMfma = 0x008, kDsRead = 0x100;
  if constexpr (S < NS) {
    // a dV / dK slot reads one transposed operand (two reads), an S / dP slot
    // an A and a B operand (two reads; one for S with K in registers)
    constexpr int t = S + kKvPrefetch;
    constexpr int reads = (ATTN_BWD_DKDV_KREG && t >= NTR && t < NTR + STEPS) ? 1 : 2;
    if constexpr (t < NS) __builtin_amdgcn_sched_group_barrier(kDsRead, reads, 0);
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    pin_kv_schedule<S + 1, NS, NTR, STEPS>();
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_pp_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "ping-pong dK/dV kernel: d_qk = d_v = 64 or 128");
  constexpr int STEPS = D / 16, BLKS = D / 32;
  constexpr int KV_ELEMS = kBlock * D;                            // K (then V) rows of the workgroup
  constexpr int QD_ELEMS = kRows * D;                             // one query block of Q (then dO)
  constexpr int ROWS_OFF = 2 * QD_ELEMS;                          // 64 LSE values, then 64 D values (fp32)
  constexpr int SLOT_ELEMS = (ROWS_OFF + 2 * 64 * 2 + 511) / 512 * 512;
  constexpr int kSlots = 5;
  constexpr int SLOTS_OFF = 2 * KV_ELEMS;
  constexpr int LOOP_ELEMS = SLOTS_OFF + kSlots * SLOT_ELEMS;
  constexpr int MERGE_ELEMS = kWaves * kWave * 2 * BLKS * 16 * 2; // group 1's dK^T and dV^T, fp32
  // a group-0 wave stages its output rows in its own merge region once it has read it
  static_assert(2 * kRows * (D + 8) <= kWave * 2 * BLKS * 16 * 2, "staging inside a wave's merge region");
  constexpr int LDS_ELEMS = LOOP_ELEMS > MERGE_ELEMS ? LOOP_ELEMS : MERGE_ELEMS;
  static_assert(LDS_ELEMS * 2 <= 160 * 1024, "LDS budget");
  constexpr int ROWS_REQ = 512 / D;                               // rows per 1 KB request
  constexpr int KV_REQ = KV_ELEMS / 512;                          // requests per K or V copy
  constexpr int KV_ISS = 2 * KV_REQ / (2 * kWaves);               // per wave, K and V
  constexpr int B_REQ = QD_ELEMS / 512;                           // requests per Q or dO block
  static_assert(B_REQ % kWaves == 0 && (2 * KV_REQ) % (2 * kWaves) == 0, "request split");
  constexpr int B_ISS = B_REQ / kWaves;                           // per wave per copy of a block
  constexpr int ISS = 2 * B_ISS + 1;                              // Q, dO, and one LSE or D request
  // matrix-phase slots: dV (hh, db), dK (hh, db), S (ks), dP (ks)
  constexpr int NDV = 2 * BLKS, NTR = 2 * NDV, NS = NTR + 2 * STEPS;
  constexpr int kDmaStride = NS / ISS;
  static_assert(kDmaStride >= 1, "DMAs per matrix phase");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[LDS_ELEMS];
  lds_u16_t* const lds = (lds_u16_t*)smem;
  auto slot = [&] __device__ (int i) __attribute__((always_inline)) { return lds + SLOTS_OFF + i * SLOT_ELEMS; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / kWaves, wv = wave % kWaves;
  const int lane = tid % kWave, g = lane / 32, lq = lane % 32;
  int h, b, blk;
  decode_block(p, false, h, b, blk);
  int seq0, L;
  seq_range(p, b, seq0, L);
  const int k0 = blk * kBlock;
  if (k0 >= L) return;                                            // uniform over the workgroup
  const int kw0 = k0 + wv * kRows;
  const int key = kw0 + lq;
  const bool key_valid = key < L;
  const int qstart = CAUSAL ? (k0 / kTile) * kTile : 0;
  const int nblk = (L - qstart + kRows - 1) / kRows;              // 32-query blocks
  const int niter = (nblk + 1) / 2;                               // iterations 0..niter
  const int64_t row = (int64_t)p.H * D;
  const uint32_t rowbytes = (uint32_t)(row * 2);
  const uint32_t seq_bytes = (uint32_t)((L - 1) * row * 2 + D * 2);
  const int T = total_tokens(p);
  const attn::u32x4_t q_rsrc = attn::make_rsrc(p.q + (int64_t)seq0 * row + (int64_t)h * D, seq_bytes);
  const attn::u32x4_t o_rsrc = attn::make_rsrc(p.dout + (int64_t)seq0 * row + (int64_t)h * D, seq_bytes);
  const attn::u32x4_t l_rsrc = attn::make_rsrc(p.lse + (int64_t)h * T + seq0, (uint32_t)L * 4u);
  const attn::u32x4_t d_rsrc = attn::make_rsrc(p.delta + (int64_t)h * T + seq0, (uint32_t)L * 4u);
  const float c = p.c;

  // K and V of the workgroup's keys into LDS (rows past L read zeros)
  {
    const uint32_t kv_bytes = (uint32_t)(L - 1 - k0) * rowbytes + (uint32_t)(D * 2);
    const attn::u32x4_t k_rsrc = attn::make_rsrc(p.k + (int64_t)(seq0 + k0) * row + (int64_t)h * D, kv_bytes);
    const attn::u32x4_t v_rsrc = attn::make_rsrc(p.v + (int64_t)(seq0 + k0) * row + (int64_t)h * D, kv_bytes);
#pragma unroll
    for (int i = 0; i < KV_ISS; ++i) {
      const int r = wave * KV_ISS + i, isv = r >= KV_REQ, rr = isv ? r - KV_REQ : r;
      const int e = rr * 512 + 8 * lane, krow = e / D, pos = (e % D) / 8;
      const uint32_t off = (uint32_t)krow * rowbytes + (uint32_t)(pos ^ RowSwz<D>::f(krow)) * 16u;
      attn::dma_chunk(isv ? v_rsrc : k_rsrc, off, 0u, lds + (isv ? KV_ELEMS : 0) + rr * 512);
    }
  }
  // per-lane offsets of this wave's K and V rows (B operands: row = key, not
  // the bit-swapped order), k-step ks
  int kvoff[STEPS];
#pragma unroll
  for (int ks = 0; ks < STEPS; ++ks) {
    const int r = wv * kRows + lq;
    kvoff[ks] = r * D + (((2 * ks + g) ^ RowSwz<D>::f(r)) * 8);
  }
  const ReadsP<D> rq(lane);                                       // Q, dO rows and Q^T, dO^T of a block

  // query-block DMAs: request rr of the Q or dO copy fills 1 KB block rr of
  // the slot (rows rr * ROWS_REQ on, in soffset); lane offsets depend on rr
  // mod (16 / ROWS_REQ) through the swizzle, and this wave's requests are
  // rr = wv * B_ISS + i
  uint32_t lane_off[B_ISS];
#pragma unroll
  for (int i = 0; i < B_ISS; ++i) {
    const int rr = wv * B_ISS + i, r = (8 * lane) / D, pos = (8 * lane % D) / 8;
    lane_off[i] = (uint32_t)r * rowbytes + (uint32_t)(pos ^ RowSwz<D>::f(rr * ROWS_REQ + r)) * 16u;
  }
  auto block_off = [&] __device__ (int bq) __attribute__((always_inline)) -> uint32_t {
    return bq < nblk ? (uint32_t)(qstart + bq * kRows) * rowbytes : seq_bytes;
  };
  // DMA d of this wave's share of block bq into slot dst: Q, dO, then the
  // LSE (waves 0, 2) or D (waves 1, 3) rows, 64 values from the block's first
  // row (only the first 32 are read)
  auto dma = [&] __device__ (int d, int bq, lds_u16_t* dst) __attribute__((always_inline)) {
    if (d < 2 * B_ISS) {
      const bool iso = d >= B_ISS;
      const int i = iso ? d - B_ISS : d, rr = wv * B_ISS + i;
      attn::dma_chunk(iso ? o_rsrc : q_rsrc, lane_off[i], block_off(bq) + (uint32_t)(rr * ROWS_REQ) * rowbytes,
                      dst + (iso ? QD_ELEMS : 0) + rr * 512);
    } else if (wv < 2) {
      const uint32_t r0 = bq < nblk ? (uint32_t)(qstart + bq * kRows) * 4u : (uint32_t)L * 4u;
      attn::dma_dword(wv == 0 ? l_rsrc : d_rsrc, r0 + 4u * lane_id_here(), dst + ROWS_OFF + wv * 128);
    }
  };

  f32x16_t dk[BLKS], dv[BLKS];
#pragma unroll
  for (int i = 0; i < BLKS; ++i) { dk[i] = f32x16_t{}; dv[i] = f32x16_t{}; }
  f32x16_t sacc = {}, pacc = {};
  u32x4_t pb[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
  u32x4_t dsb[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
  const f32x16_t zero = {};

  // A and B operands of slot s: dV / dK slots read block bprev transposed
  // (B is P or dS in registers), S / dP slots a row chunk of block bcur and
  // of this wave's K or V rows
  struct Ops { bf16x8_t a, b; };
  bf16x8_t kreg[STEPS];                                           // with ATTN_BWD_DKDV_KREG, after the prologue
  auto read_op = [&] __device__ (int s, const lds_u16_t* sprev, const lds_u16_t* scur) __attribute__((always_inline))
      -> Ops {
    Ops o;
    if (s < NTR) {
      const int isk = s >= NDV, q = isk ? s - NDV : s, hh = q / BLKS, db = q % BLKS;
      o.a = read_tr_p<D>(sprev + (isk ? 0 : QD_ELEMS), rq, db, 16 * hh);
      o.b = o.a;
    } else {
      const int q = s - NTR, isdp = q >= STEPS, ks = isdp ? q - STEPS : q;
      o.a = read_row_p<D>(scur + (isdp ? QD_ELEMS : 0), rq, ks, 0);
      if (ATTN_BWD_DKDV_KREG && !isdp) o.b = kreg[ks];
      else o.b = *(const lds_bf16x8_t*)(lds + (isdp ? KV_ELEMS : 0) + kvoff[ks]);
    }
    return o;
  };
  Ops op_pre[kKvPrefetch];
  auto prefetch = [&] __device__ (const lds_u16_t* sprev) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kKvPrefetch; ++s) op_pre[s] = read_op(s, sprev, sprev);
  };
  // matrix phase on blocks bprev (dV, dK) and bcur (S, dP); with DMA the
  // wave issues its share of block bnext into slot dst
  auto matrix = [&] __device__ (auto dma_tag, const lds_u16_t* sprev, const lds_u16_t* scur, int bnext,
                                lds_u16_t* dst) __attribute__((always_inline)) {
    constexpr bool DMA = decltype(dma_tag)::value;
    Ops op[NS];
#pragma unroll
    for (int s = 0; s < kKvPrefetch; ++s) op[s] = op_pre[s];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + kKvPrefetch < NS) op[s + kKvPrefetch] = read_op(s + kKvPrefetch, sprev, scur);
      if (s < NTR) {
        const int isk = s >= NDV, q = isk ? s - NDV : s, hh = q / BLKS, db = q % BLKS;
        if (isk) dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s].a, __builtin_bit_cast(bf16x8_t, dsb[hh]), dk[db], 0, 0, 0);
        else dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s].a, __builtin_bit_cast(bf16x8_t, pb[hh]), dv[db], 0, 0, 0);
      } else {
        const int q = s - NTR, isdp = q >= STEPS, ks = isdp ? q - STEPS : q;
        if (isdp) pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s].a, op[s].b, ks == 0 ? zero : pacc, 0, 0, 0);
        else sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s].a, op[s].b, ks == 0 ? zero : sacc, 0, 0, 0);
      }
      // a request after the last MFMA of each stride of slots (measured: mid-stride −0.5 %, first slot −1.5 %)
      if (DMA && s % kDmaStride == kDmaStride - 1 && s / kDmaStride < ISS) dma(s / kDmaStride, bnext, dst);
    }
    pin_kv_schedule<0, NS, NTR, STEPS>();
  };
  // VALU phase of block bq (S, dP in sacc, pacc; LSE and D rows in its slot)
  auto valu = [&] __device__ (int bq, const lds_u16_t* sq) __attribute__((always_inline)) {
    const lds_f32_t* const lse_s = (const lds_f32_t*)(sq + ROWS_OFF);
    const lds_f32_t* const d_s = lse_s + 64;
    const int q_base = qstart + bq * kRows;
    const bool masked = (q_base + kRows > L) || (kw0 + kRows > L) || (CAUSAL && kw0 + kRows - 1 > q_base) || bq < 0;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 16 * (r / 8) + 8 * g + (r % 8);
      x[r] = __builtin_fmaf(sacc[r], c, -lse_s[qi] * kLog2e);
    }
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int query = q_base + 16 * (r / 8) + 8 * g + (r % 8);
        if (!(key_valid && bq >= 0 && query < L && (!CAUSAL || key <= query))) x[r] = -__builtin_inff();
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 8 * hh + 2 * jj, qi = 16 * hh + 8 * g + 2 * jj;
        const float p0 = __builtin_amdgcn_exp2f(x[r]), p1 = __builtin_amdgcn_exp2f(x[r + 1]);
        pb[hh][jj] = pack_bf16x2(p0, p1);
        dsb[hh][jj] = pack_bf16x2(p0 * (pacc[r] - d_s[qi]), p1 * (pacc[r + 1] - d_s[qi + 1]));
      }
  };

  // Prologue: slots 3 and 4 (blocks -2, -1) zeros; blocks 0 and 1.
  for (int i = tid; i < 2 * SLOT_ELEMS / 8; i += kThreads2) ((lds_u32x4_t*)slot(3))[i] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int d = 0; d < ISS; ++d) {
    dma(d, 0 + grp, slot(grp));                                   // group 0: block 0, group 1: block 1
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
  if (ATTN_BWD_DKDV_KREG) {
#pragma unroll
    for (int ks = 0; ks < STEPS; ++ks) kreg[ks] = *(const lds_bf16x8_t*)(lds + kvoff[ks]);
  }
  using True = GroupTag<true>;
  using False = GroupTag<false>;
  auto run = [&] __device__ (auto grp_tag) __attribute__((always_inline)) {
    constexpr bool G0 = decltype(grp_tag)::value;
    int c0 = 0;                                                   // (2j) mod 5
    if (G0) prefetch(slot(3));                                    // matrix(0): block -2
    // not peeled: a peeled first iteration gets its own register assignment,
    // and at d = 128 the copies between the two spill registers
#pragma clang loop unroll(disable)
    for (int j = 0; j <= niter; ++j) {
      auto m5 = [&] __device__ (int a) __attribute__((always_inline)) { return a >= 5 ? a - 5 : a; };
      const int s_even = c0, s_odd = m5(c0 + 1), s_even_m2 = m5(c0 + 3), s_odd_m2 = m5(c0 + 4);
      const int s_even_p2 = m5(c0 + 2), s_odd_p2 = m5(c0 + 3);
      if (G0) {
        __builtin_amdgcn_s_setprio(1);
        matrix(True{}, slot(s_even_m2), slot(s_even), 2 * j + 2, slot(s_even_p2));
        __builtin_amdgcn_s_setprio(0);
        attn::barrier();
        valu(2 * j, slot(s_even));
        prefetch(slot(s_even));                                   // matrix(2j+2) starts with block 2j
        attn::dma_wait_barrier<0>();                              // block 2j+2 has landed
      } else {
        valu(2 * j - 1, slot(s_odd_m2));
        prefetch(slot(s_odd_m2));                                 // matrix(2j+1) starts with block 2j-1
        attn::dma_wait_barrier<0>();                              // block 2j+1 has landed
        __builtin_amdgcn_s_setprio(1);
        matrix(True{}, slot(s_odd_m2), slot(s_odd), 2 * j + 3, slot(s_odd_p2));
        __builtin_amdgcn_s_setprio(0);
        attn::barrier();
      }
      c0 = m5(c0 + 2);
    }
  };
  if (grp == 0) run(True{});
  else run(False{});
  attn::dma_wait_all();
  block_sync();
  // group 1's partial dK^T, dV^T -> LDS (16-byte pieces, lane-interleaved);
  // group 0 adds them and stores dK (times the scale) and dV
  lds_f32_t* const merge = (lds_f32_t*)lds + wv * (kWave * 2 * BLKS * 16);
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < BLKS; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4_t a = {dk[db][4 * q4], dk[db][4 * q4 + 1], dk[db][4 * q4 + 2], dk[db][4 * q4 + 3]};
        const f32x4_t v = {dv[db][4 * q4], dv[db][4 * q4 + 1], dv[db][4 * q4 + 2], dv[db][4 * q4 + 3]};
        *(__attribute__((address_space(3))) f32x4_t*)(merge + ((db * 4 + q4) * kWave + lane) * 4) = a;
        *(__attribute__((address_space(3))) f32x4_t*)(merge + (((BLKS + db) * 4 + q4) * kWave + lane) * 4) = v;
      }
  }
  block_sync();
  if (grp == 0) {
#pragma unroll
    for (int db = 0; db < BLKS; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4_t a = *(const __attribute__((address_space(3))) f32x4_t*)(merge + ((db * 4 + q4) * kWave + lane) * 4);
        const f32x4_t v = *(const __attribute__((address_space(3))) f32x4_t*)(merge + (((BLKS + db) * 4 + q4) * kWave + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[db][4 * q4 + e] += a[e];
          dv[db][4 * q4 + e] += v[e];
        }
      }
    // the wave's own merge region, read above, stages its dK and dV rows
    lds_u16_t* const stage = (lds_u16_t*)merge;
    store_rows<D>(dk, p.scale, stage, p.dk, (int64_t)seq0 + kw0, L - kw0, p.H, h, lane);
    store_rows<D>(dv, 1.0f, stage + kRows * (D + 8), p.dv, (int64_t)seq0 + kw0, L - kw0, p.H, h, lane);
  }
}

// ---- dK, dV with the work split over two wave groups: one workgroup of 8
// waves per block of 128 key rows.  Waves 0-3 (dV group) own 32 keys each and
// compute S = Q K^T, P and dV^T += dO^T P; waves 4-7 (dK group) own the same
// keys and compute dP = dO V^T, dS = P (dP - D) and dK^T += Q^T dS, taking P
// from the dV wave of their key slice through LDS (as bf16, lane for lane:
// both accumulators hold one key per lane and the same queries per
// register).  Each wave fits in 256 registers, so every SIMD holds one wave
// of each group and the matrix cores interleave them; each group runs 16
// MFMAs per 32-query block, the same 32 in total as one wave doing all four
// products.  One barrier per block separates P's writer from its reader:
//   dV group: ... | dV(b), S(b+1), P(b+1) -> LDS | dV(b+1), S(b+2) ...
//   dK group: ... | dS(b), dK(b), dP(b+1)       | dS(b+1), dK(b+1) ...
// P alternates between two LDS buffers, the Q/dO tiles between two more.
template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_split_kernel(BwdParams p) {
  constexpr int QK_STEPS = DQK / 16, V_STEPS = DV / 16, KBLK = DQK / 32, VBLK = DV / 32, QB = kTile / 32;
  constexpr int Q_ELEMS = kTile * DQK, O_ELEMS = kTile * DV;
  // Q is read row-wise (S) and transposed (dK), dO row-wise (dP) and
  // transposed (dV): each tile is stored once, in the row layout, which
  // serves both reads without bank conflicts.  Per buffer: Q, dO, then LSE
  // (log2 units) and D as fp32, padded to whole 1 KB blocks.
  constexpr int ROWS_OFF = Q_ELEMS + O_ELEMS;                           // LSE, D rows
  constexpr int TILE_ELEMS = (ROWS_OFF + 2 * kTile * 2 + 511) / 512 * 512;
  constexpr int P_ELEMS = kWaves * kWave * 16;                          // 32 x 32 bf16 per dV wave
  constexpr int STAGE_ELEMS = 2 * kWaves * kRows * ((DQK > DV ? DQK : DV) + 8);
  constexpr int WORK_ELEMS = 2 * TILE_ELEMS + 2 * P_ELEMS;
  constexpr int LDS_ELEMS = WORK_ELEMS > STAGE_ELEMS ? WORK_ELEMS : STAGE_ELEMS;
  static_assert(LDS_ELEMS * 2 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[LDS_ELEMS];
  lds_u16_t* const lds = (lds_u16_t*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool kgrp = wave >= kWaves;          // dK group
  const int wv = wave % kWaves;              // key slice of the wave within its group
  const int lane = tid % kWave, g = lane / 32, lq = lane % 32;
  int h, b, blk;
  decode_block(p, false, h, b, blk);
  int seq0, L;
  seq_range(p, b, seq0, L);
  const int k0 = blk * kBlock;
  if (k0 >= L) return;
  const int kw0 = k0 + wv * kRows;
  const int key = kw0 + lq;
  const bool key_valid = key < L;


  const Reads<DQK> rq(lane);
  const Reads<DV> ro(lane);
  const int qstart = CAUSAL ? (k0 / kTile) * kTile : 0;
  const int ntiles = (L - qstart + kTile - 1) / kTile;
  const int nblk = ntiles * QB;
  const int64_t qk_stride = (int64_t)p.H * DQK, v_stride = (int64_t)p.H * DV;
  const uint16_t* const qbase = p.q + (int64_t)seq0 * qk_stride + (int64_t)h * DQK;
  const uint16_t* const dobase = p.dout + (int64_t)seq0 * v_stride + (int64_t)h * DV;
  const int T = total_tokens(p);
  const float* const lse_h = p.lse + (int64_t)h * T + seq0;
  const float* const d_h = p.delta + (int64_t)h * T + seq0;

  const f32x16_t zero = {};

  auto buf = [&] __device__ (int t) __attribute__((always_inline)) { return lds + (t & 1) * TILE_ELEMS; };
  // Q and dO tiles are copied HBM/L2 -> LDS by buffer_load ... lds, every wave
  // issuing its share of the tile's 1 KB requests.  Request lane i writes the
  // 16 bytes at LDS position 8 i of its block, i.e. chunk `pos` of row `row`,
  // which holds the tile's chunk pos ^ f(row) of that row.  The buffer ranges
  // end after row L-1 of the sequence, so rows past its end read as zeros.
  constexpr int Q_REQ = Q_ELEMS / 512, O_REQ = O_ELEMS / 512;   // 1 KB requests per tile
  constexpr int REQ = Q_REQ + O_REQ;
  static_assert(Q_ELEMS % 512 == 0 && O_ELEMS % 512 == 0 && REQ % (2 * kWaves) == 0, "request split");
  constexpr int REQ_W = REQ / (2 * kWaves);                      // requests per wave per tile
  const uint32_t q_rowbytes = (uint32_t)(qk_stride * 2), o_rowbytes = (uint32_t)(v_stride * 2);
  const attn::u32x4_t q_rsrc = attn::make_rsrc(qbase, (uint32_t)((L - 1) * qk_stride * 2 + DQK * 2));
  const attn::u32x4_t o_rsrc = attn::make_rsrc(dobase, (uint32_t)((L - 1) * v_stride * 2 + DV * 2));
  auto issue_tile = [&] __device__ (int t) __attribute__((always_inline)) {
    lds_u16_t* const base = buf(t);
    const uint32_t q0t = (uint32_t)(qstart + t * kTile);
#pragma unroll
    for (int i = 0; i < REQ_W; ++i) {
      const int r = wave * REQ_W + i;                            // uniform
      const bool isq = r < Q_REQ;
      const int rr = isq ? r : r - Q_REQ;
      const int D = isq ? DQK : DV;
      const int e = rr * 512 + 8 * lane;                         // element of the tile (row-major, D per row)
      const int row = e / D, pos = (e % D) / 8;
      const int f = isq ? RowSwz<DQK>::f(row) : RowSwz<DV>::f(row);
      const uint32_t rowbytes = isq ? q_rowbytes : o_rowbytes;
      const uint32_t lane_off = (uint32_t)row * rowbytes + (uint32_t)(pos ^ f) * 16u;
      lds_u16_t* const dst = base + (isq ? 0 : Q_ELEMS) + rr * 512;
      attn::dma_chunk(isq ? q_rsrc : o_rsrc, lane_off, q0t * rowbytes, dst);
    }
  };
  // LSE and D of a tile's 64 rows go through registers (threads 0..63: LSE,
  // 64..127: D), loaded one tile ahead.  The LSE goes to log2 units only when
  // it is staged: an arithmetic use right after the load would make the wave
  // wait for every load in flight.
  float rowval = 0.0f;
  auto load_rows = [&] __device__ (int t) __attribute__((always_inline)) {
    const int r = qstart + t * kTile + (tid % kTile);
    if (tid < 2 * kTile) rowval = (r < L) ? (tid < kTile ? lse_h[r] : d_h[r]) : 0.0f;
  };
  auto stage_rows = [&] __device__ (int t) __attribute__((always_inline)) {
    if (tid < 2 * kTile) ((lds_f32_t*)(buf(t) + ROWS_OFF))[tid] = tid < kTile ? rowval * kLog2e : rowval;
  };
  // this lane's 32 bytes of the P block of key slice wv, buffer i, as two
  // 16-byte halves P_HALF apart: each half of all lanes is contiguous, so the
  // 16 lanes of a pass cover the 64 banks once
  constexpr int P_HALF = P_ELEMS / 2 / 8;                              // in 16-byte units
  auto pslot = [&] __device__ (int i) __attribute__((always_inline)) {
    return (lds_u32x4_t*)(lds + 2 * TILE_ELEMS + i * P_ELEMS + (wv * kWave + lane) * 8);
  };

  // Each group runs the same loop (and the same barriers) with its own
  // registers: the group is a compile-time parameter, so the dV group's
  // K operands and the dK group's six dK blocks are never allocated together.
  auto group_body = [&] __device__ (auto grp_tag) __attribute__((always_inline)) {
    constexpr bool KG = decltype(grp_tag)::value;     // dK group
    // dV group: K rows of its keys (B operand of S); dK group: V rows (of dP)
    constexpr int BSTEPS = KG ? V_STEPS : QK_STEPS;
    bf16x8_t breg[BSTEPS];
    if constexpr (KG) load_b_operand<DV>(breg, p.v, seq0 + key, p.H, h, g, key_valid);
    else load_b_operand<DQK>(breg, p.k, seq0 + key, p.H, h, g, key_valid);
    constexpr int ABLK = KG ? KBLK : VBLK;
    f32x16_t acc[ABLK];                      // dK^T blocks (dK group) or dV^T blocks (dV group)
#pragma unroll
    for (int i = 0; i < ABLK; ++i) acc[i] = f32x16_t{};

    // carried from a block's first half to its second, in the same registers:
    // the dK group's dP (16 floats) or the dV group's P (8 dwords of bf16 pairs)
    f32x16_t carry = zero;
    // The transposed A operands of the next block's dV (dO^T) or dK (Q^T)
    // products, read at the end of half_a: that block's rows are visible from
    // the barrier before half_a on (half_a reads them too), and a half_b that
    // starts with its operands in registers does not wait for LDS first.
    // At d_qk = 192 only the dV group has the registers for it (the dK group
    // would need 48 more beside its six dK blocks).
    constexpr bool PRE = (DQK <= 128 || !KG) && ATTN_BWD_PREFETCH;
    bf16x8_t pre[PRE ? 2 : 1][PRE ? ABLK : 1];
    auto prefetch = [&] __device__ (int nb) __attribute__((always_inline)) {
      if constexpr (PRE) {
        const int t = nb / QB, qb = nb % QB;
        const lds_u16_t* const base = buf(t);
  #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
  #pragma unroll
          for (int db = 0; db < ABLK; ++db)
            pre[hh][db] = KG ? read_tr<DQK>(base, rq, db, qb * 32 + 16 * hh)
                             : read_tr<DV>(base + Q_ELEMS, ro, db, qb * 32 + 16 * hh);
      }
    };
    // first half of block nb: dV group S, P -> LDS; dK group dP
    auto half_a = [&] __device__ (int nb) __attribute__((always_inline)) {
      const int t = nb / QB, qb = nb % QB;
      const lds_u16_t* const base = buf(t);
      if constexpr (!KG) {
        // operands read in groups of at most 8 k-steps (12 at d_qk = 192 would
        // not fit beside the accumulators)
        constexpr int CH = QK_STEPS > 8 ? QK_STEPS / 2 : QK_STEPS;
        f32x16_t s = zero;
  #pragma unroll
        for (int k0 = 0; k0 < QK_STEPS; k0 += CH) {
          bf16x8_t a_s[CH];
  #pragma unroll
          for (int i = 0; i < CH; ++i) a_s[i] = read_row<DQK>(base, rq, k0 + i, qb);
  #pragma unroll
          for (int i = 0; i < CH; ++i) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_s[i], breg[k0 + i], s, 0, 0, 0);
        }
        const lds_f32_t* const lse_s = (const lds_f32_t*)(base + ROWS_OFF);
        const int q0t = qstart + t * kTile;
        const bool masked = (q0t + kTile > L) || (kw0 + kRows > L) || (CAUSAL && kw0 + kRows - 1 > q0t);
        float x[16];
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qb * 32 + 16 * (r / 8) + 8 * g + (r % 8);
          x[r] = __builtin_fmaf(s[r], p.c, -lse_s[qi]);
        }
        if (masked) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int query = q0t + qb * 32 + 16 * (r / 8) + 8 * g + (r % 8);
            if (!(key_valid && query < L && (!CAUSAL || key <= query))) x[r] = -__builtin_inff();
          }
        }
        uint32_t pw[8];
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          pw[i] = pack_bf16x2(__builtin_amdgcn_exp2f(x[2 * i]), __builtin_amdgcn_exp2f(x[2 * i + 1]));
          carry[i] = __uint_as_float(pw[i]);
        }
        lds_u32x4_t* const slot = pslot(nb & 1);
        slot[0] = u32x4_t{pw[0], pw[1], pw[2], pw[3]};
        slot[P_HALF] = u32x4_t{pw[4], pw[5], pw[6], pw[7]};
      } else {
        bf16x8_t a_p[V_STEPS];
  #pragma unroll
        for (int vs = 0; vs < V_STEPS; ++vs) a_p[vs] = read_row<DV>(base + Q_ELEMS, ro, vs, qb);
        carry = zero;
  #pragma unroll
        for (int vs = 0; vs < V_STEPS; ++vs)
          carry = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_p[vs], breg[vs], carry, 0, 0, 0);
      }
      prefetch(nb);
    };
    // second half of block nb: dV group dV; dK group P from LDS, dS, dK
    auto half_b = [&] __device__ (int nb) __attribute__((always_inline)) {
      const int t = nb / QB, qb = nb % QB;
      const lds_u16_t* const base = buf(t);
      if constexpr (!KG) {
  #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t pw[4] = {__float_as_uint(carry[4 * hh]), __float_as_uint(carry[4 * hh + 1]),
                                  __float_as_uint(carry[4 * hh + 2]), __float_as_uint(carry[4 * hh + 3])};
          const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, pw);
          bf16x8_t a_v[VBLK];
  #pragma unroll
          for (int db = 0; db < VBLK; ++db)
            a_v[db] = PRE ? pre[PRE ? hh : 0][PRE ? db : 0] : read_tr<DV>(base + Q_ELEMS, ro, db, qb * 32 + 16 * hh);
  #pragma unroll
          for (int db = 0; db < VBLK; ++db) acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_v[db], bop, acc[db], 0, 0, 0);
        }
      } else {
        const lds_f32_t* const d_s = (const lds_f32_t*)(base + ROWS_OFF) + kTile;
        const lds_u32x4_t* const slot = pslot(nb & 1);
        const u32x4_t praw[2] = {slot[0], slot[P_HALF]};
  #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t dsb[4];
  #pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 8 * hh + 2 * jj;
            const int qi = qb * 32 + 16 * hh + 8 * g + 2 * jj;
            const uint32_t w = praw[hh][jj];
            dsb[jj] = pack_bf16x2(bf16_lo(w) * (carry[r] - d_s[qi]), bf16_hi(w) * (carry[r + 1] - d_s[qi + 1]));
          }
          const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, dsb);
          bf16x8_t a_k[KBLK];
  #pragma unroll
          for (int db = 0; db < KBLK; ++db)
            a_k[db] = PRE ? pre[PRE ? hh : 0][PRE ? db : 0]
                          : read_tr<DQK>(base, rq, db, qb * 32 + 16 * hh);
  #pragma unroll
          for (int db = 0; db < KBLK; ++db) acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_k[db], bop, acc[db], 0, 0, 0);
        }
      }
    };

    // Tiles: both buffers filled up front; tile u+1 goes into the buffer of tile
    // u-1 after barrier 2u (u >= 1), when every wave has finished block 2u-1:
    // its DMAs are issued right after that barrier and awaited before the next
    // one, so it is visible from barrier 2u+1 on, before block 2u+2 reads it.
    // The LSE and D rows follow the same schedule through registers, their
    // loads one tile ahead.
    issue_tile(0);
    load_rows(0);
    stage_rows(0);
    if (ntiles > 1) {
      issue_tile(1);
      load_rows(1);
      stage_rows(1);
    }
    if (ntiles > 2) load_rows(2);
    attn::dma_wait_all();
    block_sync();
    half_a(0);
    for (int nb = 0; nb < nblk; ++nb) {
      block_sync();
      const bool refill = nb % QB == 0 && nb >= QB && nb / QB + 1 < ntiles;
      if (refill) {
        const int u = nb / QB;
        stage_rows(u + 1);
        if (u + 2 < ntiles) load_rows(u + 2);
        issue_tile(u + 1);
      }
      half_b(nb);
      if (nb + 1 < nblk) half_a(nb + 1);
      if (refill) attn::dma_wait_all();        // tile u+1 has landed before the next barrier
    }
    block_sync();                           // the staging area overlaps the tile buffers
    lds_u16_t* const stage = lds + wave * kRows * ((DQK > DV ? DQK : DV) + 8);
    if constexpr (KG) {
      f32x16_t dk[KBLK];
  #pragma unroll
      for (int i = 0; i < KBLK; ++i) dk[i] = acc[i];
      store_rows<DQK>(dk, p.scale, stage, p.dk, (int64_t)seq0 + kw0, L - kw0, p.H, h, lane);
    } else {
      f32x16_t dv[VBLK];
  #pragma unroll
      for (int i = 0; i < VBLK; ++i) dv[i] = acc[i];
      store_rows<DV>(dv, 1.0f, stage, p.dv, (int64_t)seq0 + kw0, L - kw0, p.H, h, lane);
    }
  };
  if (kgrp) group_body(GroupTag<true>{});
  else group_body(GroupTag<false>{});
}

template <int DQK, int DV>
hipError_t launch_dims(const BwdParams& p, bool causal, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.N * p.H;   // at least T*H; the kernel stops at T*H
  constexpr int RPB = kThreads / (DV / 8);
  hipLaunchKernelGGL(bwd_delta_kernel<DV>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads), 0, s, p);
  const dim3 grid((unsigned)p.B * p.H * p.n_blocks);
  if constexpr (ATTN_BWD_DKDV_PP && DQK == DV && DQK <= 128) {
    if (causal) hipLaunchKernelGGL((bwd_dkdv_pp_kernel<DQK, true>), grid, dim3(kThreads2), 0, s, p);
    else hipLaunchKernelGGL((bwd_dkdv_pp_kernel<DQK, false>), grid, dim3(kThreads2), 0, s, p);
  } else {
    if (causal) hipLaunchKernelGGL((bwd_dkdv_split_kernel<DQK, DV, true>), grid, dim3(kThreads2), 0, s, p);
    else hipLaunchKernelGGL((bwd_dkdv_split_kernel<DQK, DV, false>), grid, dim3(kThreads2), 0, s, p);
  }
  const dim3 grid8((unsigned)(p.B * p.H * ((p.N + kDqBlock - 1) / kDqBlock)));
  if (causal) hipLaunchKernelGGL((bwd_dq_pp_kernel<DQK, DV, true>), grid8, dim3(kDqThreads), 0, s, p);
  else hipLaunchKernelGGL((bwd_dq_pp_kernel<DQK, DV, false>), grid8, dim3(kDqThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d_qk, int d_v, bool causal, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return launch_dims<64, 64>(p, causal, s);
  if (d_qk == 128 && d_v == 128) return launch_dims<128, 128>(p, causal, s);
  if (d_qk == 192 && d_v == 128) return launch_dims<192, 128>(p, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace attn_grad
