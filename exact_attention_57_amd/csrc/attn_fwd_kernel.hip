// Fused exact-attention forward kernels for gfx950 (CDNA4, MI355X).
//
// One workgroup = 8 wave64s (two per SIMD) = one query block of 256 rows of
// one (sequence, head); each wave owns 32 query rows for the whole key loop.
// Per key tile of 64 keys each wave computes
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
// Ping-pong schedule.  Waves 0-3 (group 0) and 4-7 (group 1) share the four
// SIMDs, one of each per SIMD.  Time is cut into phases separated by
// workgroup barriers; in a group's "matrix" phase for tile j it runs the
// output product of tile j-1 and the score product of tile j (all MFMA), in
// its "softmax" phase it runs the softmax of tile j (VALU).  Group 1 runs one
// phase behind group 0, so on every SIMD one wave feeds the matrix core while
// the other computes exponentials.
//
// LDS: three K and two V tile buffers (dense rows, XOR-swizzled 16-byte
// chunks), filled straight from L2/HBM by buffer_load ... lds requests that
// group 0 spreads over its matrix phase (V of tile j and K of tile j+2 in
// iteration j).
//
// Method sources (web pages on FlashAttention-4):
//  * tiling + online softmax with running max/sum: ainexis.cn deep dive,
//    background section and "horizontal extension" concept two; jsqmd news,
//    section two.
//  * overlap of matrix products with softmax and loads (one part multiplies
//    while another does softmax and another loads): jsqmd news section four,
//    item 2; newton.com.tw wiki "FlashAttention-4", core-technology section.
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
#include "attn_fwd_common.h"

namespace attn {

// LDS tile layouts.  Each 64-key tile is stored dense (row r = key k0 + r,
// R = d/8 chunks of 16 bytes per row); the chunk of column block c of row r
// sits at position c ^ f(r) within the row, so that
//  * K: the 16 rows one quarter-wave ds_read_b128 phase touches (same chunk,
//    16 consecutive rows) land in 16 distinct 4-bank groups;
//       f_K(r) = r mod 16          when R is a multiple of 16 (d = 128)
//       f_K(r) = (r/2) mod 8       when R = 8 or 24 (d = 64, 192: two rows
//                                  share a 64-bank window or alternate halves)
//  * V: the 4 rows x 4 chunks a half-wave ds_read_b64_tr_b16 touches cover 16
//    distinct 4-bank groups;
//       f_V(r) = 4 (r mod 4)       when R = 16
//       f_V(r) = 4 ((r/2) mod 2)   when R = 8
// Dense rows let each wave fill 1 KB of a tile with one buffer_load ... lds
// (lane i writes bytes 16i..16i+15 of the 1 KB block), no VGPR staging.
template <int D>
struct KSwz {
  static constexpr int R = D / 8;
  __device__ static int f(int r) { return (R % 16 == 0) ? (r & 15) : ((r >> 1) & 7); }
};
template <int D>
struct VSwz {
  static constexpr int R = D / 8;
  static_assert(R == 16 || R == 8, "V rows of 64 or 128 elements");
  __device__ static int f(int r) { return (R == 16) ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

template <int DQK, int DV, int BN>
struct TileLayout {
  static constexpr int K_ELEMS = BN * DQK;               // dense K tile
  static constexpr int V_ELEMS = BN * DV;                // dense V tile
  static constexpr int K_ISSUES = (K_ELEMS / 512) / kLoaders;   // 1 KB DMAs per loader wave per K tile
  static constexpr int V_ISSUES = (V_ELEMS / 512) / kLoaders;
  static constexpr int ISSUES = K_ISSUES + V_ISSUES;
  static_assert((K_ELEMS / 512) % kLoaders == 0 && (V_ELEMS / 512) % kLoaders == 0, "tile split");
  static constexpr int K_PERIOD = dma_period(DQK / 8, 16);
  static constexpr int V_PERIOD = dma_period(DV / 8, 4);
  static constexpr int K_OFFS = K_ISSUES < K_PERIOD ? K_ISSUES : K_PERIOD;   // lane offsets kept
  static constexpr int V_OFFS = V_ISSUES < V_PERIOD ? V_ISSUES : V_PERIOD;
  static constexpr int LDS_ELEMS = kKBufs * K_ELEMS + kVBufs * V_ELEMS;
  static_assert(LDS_ELEMS * 2 <= 160 * 1024, "LDS budget");
};

// Order of the matrix phase's instructions for the scheduler: per slot s the
// LDS reads of slot s + kPrefetch (one for a score-product slot, two
// transposing reads for an output-product slot) followed by the MFMA of
// slot s.  The reads of the first kPrefetch slots were issued at the end of
// the wave's previous phase.
constexpr int kPrefetch = ATTN_PREFETCH;
template <int S, int NS, int NQK>
__device__ __forceinline__ void pin_matrix_schedule() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  if constexpr (S < NS) {
    if constexpr (S + kPrefetch < NS) __builtin_amdgcn_sched_group_barrier(kDsRead, (S + kPrefetch < NQK) ? 1 : 2, 0);
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    pin_matrix_schedule<S + 1, NS, NQK>();
  }
}

// Block-sparse attention (SPARSE): a byte mask over 128 x 128 (query block,
// key block) pairs says which score blocks exist.  A workgroup's 256 query
// rows are two query blocks; it visits the key tiles of the union of their
// kept key blocks (one 128-key tile per block, or two 64-key tiles at
// d_qk = 192), in order, and a wave skips the tiles its own query block does
// not keep.  Up to 256 key blocks (N <= 32768) in four 64-bit words.
constexpr int kMaskBlock = 128;
constexpr int kMaskWords = 4;
constexpr int kNoTile = 1 << 20;

template <int DQK, int DV, bool CAUSAL, int NPOLY, bool SPARSE = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims");
  static_assert(!SPARSE || (kMaskBlock % block_n(DQK) == 0 && NPOLY == 0), "block-sparse: tiles inside mask blocks, hardware exp");
  constexpr int BN = block_n(DQK);               // keys per tile
  constexpr int KB = BN / 32;                      // 32-key blocks per tile
  using Lay = TileLayout<DQK, DV, BN>;
  constexpr int QK_STEPS = DQK / 16;             // MFMA k-steps for S^T
  constexpr int D_BLOCKS = DV / 32;              // 32-row blocks of O^T
  constexpr int RK = DQK / 8;                    // 16-byte chunks per K row
  constexpr int RV = DV / 8;                     // 16-byte chunks per V row

  __shared__ __attribute__((aligned(1024))) uint16_t smem[Lay::LDS_ELEMS];
  lds_u16_t* const lds = (lds_u16_t*)smem;
  auto kbuf = [&] __device__ (int i) __attribute__((always_inline)) { return lds + i * Lay::K_ELEMS; };
  auto vbuf = [&] __device__ (int i) __attribute__((always_inline)) {
    return lds + kKBufs * Lay::K_ELEMS + i * Lay::V_ELEMS;
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / 4;      // ping-pong group
  const int lane = tid % kWave;
  const int g = lane / 32;       // lane half
  const int lq = lane % 32;      // query column

  // Instrumented build: a record of kStampWords uint64 per workgroup after
  // the four counters of p.stats (when given), at the workgroup's linear grid
  // index:
  //   [0] real-time clock at entry, [1] at the end (wave 0; 100 MHz),
  //   [2] (XCC id << 32) | HW_ID of wave 0, [3] work item (h << 40 | b << 20 | query block),
  //   [4] tile-loop iterations, [5..7] wave 0's shader cycles in the prologue,
  //   the tile loop and the epilogue, [8..11] wave 0's cycles summed over the
  //   loop in its matrix phases, the barrier after them, its softmax phases
  //   (with the operand prefetch) and the barrier after those, [12..15] the
  //   same for wave 4 (the other group on the same SIMD).
  // The stamps wait for the counter reads, so this build runs a little slower.
  // It leaves the four counters alone: every wave adding to the same four
  // words at its end makes the workgroups that finish together (a round of
  // equal work items) queue on those atomics and leave their CUs late, which
  // would show up in the records as idle time between workgroups.
#if ATTN_STAMPS
  const uint64_t rt_start = realtime_now();
  const uint64_t cy_start = cycles_now();
  uint64_t ph[4] = {0, 0, 0, 0};
  uint64_t cy_loop0 = 0, cy_loop1 = 0;
  unsigned long long* const rec =
      p.stats ? p.stats + 4 + (int64_t)kStampWords * (blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z))
              : nullptr;
#endif

  // ---- work decode.  Longest-first schedule: a 1-D grid whose workgroups
  // the hardware deals to the 8 XCDs in turn (workgroup i to XCD i mod 8).
  // XCD x takes a contiguous run of a list ordered by (sequence, head) pair,
  // head-major so that every XCD sees every sequence length, and by query
  // block longest-first within a pair: the query blocks of a pair then run
  // side by side on one XCD and share its L2 for the pair's K and V tiles.
  // Natural schedule: blockIdx = (head, sequence, query block).
  const int W = p.H * p.B * p.n_qblocks;
  auto decode = [&] __device__ (int i, int& h, int& b, int& qblk) __attribute__((always_inline)) {
    const int x = i % kXcds, slot = i / kXcds;
    const int g = x * (W / kXcds) + min(x, W % kXcds) + slot;
    const int pair = g / p.n_qblocks;
    qblk = p.n_qblocks - 1 - (g - pair * p.n_qblocks);
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
  if (p.schedule == 0) {
    decode(blockIdx.x, h, b, qblk);
  } else {
    h = blockIdx.x;
    b = blockIdx.y;
    qblk = blockIdx.z;
  }
  int seq0, L;
  seq_range(b, seq0, L);
  const int T = p.cu_seqlens ? p.cu_seqlens[p.B] : p.B * p.N;
  const int q0 = qblk * kBlockM;
  if (q0 >= L) {  // uniform over the workgroup
#if ATTN_STAMPS
    if (rec && tid == 0) {
      rec[0] = rt_start;
      rec[1] = realtime_now();
      rec[2] = hardware_ids();
      rec[3] = ((uint64_t)h << 40) | ((uint64_t)b << 20) | (uint64_t)qblk;
      for (int i = 4; i < kStampWords; ++i) rec[i] = 0;
    }
#endif
    return;
  }
  const int kend = CAUSAL ? min(L, q0 + kBlockM) : L;
  const int ntiles = (kend + BN - 1) / BN;

  const int H = p.H;
  const int64_t qk_row = (int64_t)H * DQK;   // elements between consecutive tokens
  const int64_t v_row = (int64_t)H * DV;

  const int qw0 = q0 + kRowsPerWave * wave;   // first query row of this wave
  // last key tile with a key visible to some row of this wave
  const int t_last = CAUSAL ? min(ntiles - 1, (qw0 + kRowsPerWave - 1) / BN) : ntiles - 1;
  const int qrow = qw0 + lq;
  const bool row_valid = qrow < L;

  // ---- block-sparse: bitmaps (scalar registers, by ballot) of the kept key
  // blocks among the first nkb, for the union of the workgroup's two query
  // blocks (um) and for this wave's own block (own).  nact tiles are visited:
  // TPB per kept block, except past the last tile.
  constexpr int TPB = kMaskBlock / BN;               // tiles per mask block (1 or 2)
  uint64_t um[kMaskWords] = {};
  uint64_t own0 = 0, own1 = 0, own2 = 0, own3 = 0;   // named words: no indexed array in memory
  int nact = ntiles;
  if constexpr (SPARSE) {
    const int nb = p.mask_blocks;
    const uint8_t* const mrows = p.block_mask + (int64_t)(b * H + h) * nb * nb;
    const int r0 = 2 * qblk, r1 = 2 * qblk + 1;
    const int nkb = (ntiles + TPB - 1) / TPB;        // key blocks holding the first ntiles tiles
    nact = 0;
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) {
      const int kb = 64 * w + lane;
      const bool in = kb < nkb;
      const bool a = in && r0 < nb && mrows[(int64_t)r0 * nb + kb] != 0;
      const bool c = in && r1 < nb && mrows[(int64_t)r1 * nb + kb] != 0;
      const uint64_t ba = __builtin_amdgcn_ballot_w64(a), bc = __builtin_amdgcn_ballot_w64(c);
      um[w] = ba | bc;
      const uint64_t mine = (wave < kWaves / 2) ? ba : bc;
      if (w == 0) own0 = mine;
      if (w == 1) own1 = mine;
      if (w == 2) own2 = mine;
      if (w == 3) own3 = mine;
      nact += TPB * __builtin_popcountll(um[w]);
    }
    // the last key block holds one tile only when ntiles is odd (TPB = 2);
    // its word is selected in registers (a runtime index would move um to memory)
    if constexpr (TPB == 2) {
      const int last = nkb - 1;
      uint64_t lastw = 0;
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) lastw = (w == last / 64) ? um[w] : lastw;
      if ((ntiles & 1) && ((lastw >> (last % 64)) & 1ull)) nact -= 1;
    }
  }
  // smallest kept key block above kb (kNoTile if none)
  auto next_block = [&] __device__ (int kb) __attribute__((always_inline)) -> int {
    const int first = kb + 1;
    int res = kNoTile;
#pragma unroll
    for (int w = kMaskWords - 1; w >= 0; --w) {
      const int lo = first - 64 * w;
      uint64_t bits = um[w];
      if (lo >= 64) bits = 0;
      else if (lo > 0) bits &= ~0ull << lo;
      if (bits != 0) res = 64 * w + __builtin_ctzll(bits);
    }
    return res;
  };
  // next tile to visit after t (kNoTile if none; the identity order when
  // dense): the second tile of t's block, else the first of the next kept block
  auto next_tile = [&] __device__ (int t) __attribute__((always_inline)) -> int {
    if constexpr (!SPARSE) {
      return t + 1;
    } else {
      if (TPB == 2 && t >= 0 && (t & 1) == 0 && t + 1 < ntiles) return t + 1;
      const int kb = next_block(t < 0 ? -1 : t / TPB);
      return kb == kNoTile ? kNoTile : TPB * kb;
    }
  };
  static_assert(kMaskWords == 4, "own0..own3");
  auto own_keeps = [&] __device__ (int t) __attribute__((always_inline)) -> bool {
    const int kb = t / TPB;
    const uint64_t bits = kb < 64 ? own0 : kb < 128 ? own1 : kb < 192 ? own2 : own3;
    return ((bits >> (kb & 63)) & 1ull) != 0;
  };

  // ---- Q^T operand, resident for the whole key loop.  Lane (g, lq) holds
  // Q[qrow][16*ks + 8*g + i], i = 0..7, for every k-step ks.
  bf16x8_t qreg[QK_STEPS];
  {
    const uint32_t flip = p.neg_scale ? 0x80008000u : 0u;
    const int qr = min(qrow, L - 1);
    const uint16_t* qp = p.q + (int64_t)(seq0 + qr) * qk_row + (int64_t)h * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) {
      u32x4_t raw = *(const u32x4_t*)(qp + 16 * ks);
      raw ^= flip;
      qreg[ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  // ---- K/V tiles: HBM -> LDS with buffer_load ... lds.  The buffer range of
  // each of K and V starts at this (sequence, head) and ends after key L-1,
  // so keys past the sequence end read as zeros.
  const uint32_t k_rowbytes = (uint32_t)(qk_row * 2);
  const uint32_t v_rowbytes = (uint32_t)(v_row * 2);
  const void* const k_head = p.k + (int64_t)seq0 * qk_row + (int64_t)h * DQK;
  const void* const v_head = p.v + (int64_t)seq0 * v_row + (int64_t)h * DV;
  const uint32_t k_bytes = (uint32_t)((L - 1) * (int64_t)qk_row * 2 + DQK * 2);
  const uint32_t v_bytes = (uint32_t)((L - 1) * (int64_t)v_row * 2 + DV * 2);
  // lane byte offsets (within a tile) of the chunks this lane loads when its
  // wave is loader lw (group 1 computes them but issues no DMA); requests
  // past the pattern's period reuse them shifted by whole rows
  const int lw = wave % kLoaders;
  uint32_t koff[Lay::K_OFFS], voff[Lay::V_OFFS];
#pragma unroll
  for (int i = 0; i < Lay::K_OFFS; ++i) {
    const int slot = (lw * Lay::K_ISSUES + i) * 64 + lane;
    const int row = slot / RK, pos = slot % RK;
    koff[i] = (uint32_t)row * k_rowbytes + (uint32_t)(pos ^ KSwz<DQK>::f(row)) * 16u;
  }
#pragma unroll
  for (int i = 0; i < Lay::V_OFFS; ++i) {
    const int slot = (lw * Lay::V_ISSUES + i) * 64 + lane;
    const int row = slot / RV, pos = slot % RV;
    voff[i] = (uint32_t)row * v_rowbytes + (uint32_t)(pos ^ VSwz<DV>::f(row)) * 16u;
  }
  const uint32_t k_period_bytes = (uint32_t)(Lay::K_PERIOD * 64 / RK) * k_rowbytes;
  const uint32_t v_period_bytes = (uint32_t)(Lay::V_PERIOD * 64 / RV) * v_rowbytes;
  const u32x4_t k_rsrc = make_rsrc(k_head, k_bytes);
  const u32x4_t v_rsrc = make_rsrc(v_head, v_bytes);

  // L2 prefetch for the workgroup that starts next on this XCD (workgroup
  // blockIdx + next_stride of the 1-D grid): its Q rows and first 256 keys of
  // K, one 128-byte line per lane, issued by group 1 near the end of the key
  // loop.  The requests are LDS DMAs of one dword per lane into a K buffer
  // that is no longer read, so no register waits on them; they only warm the
  // XCD's L2 against the next workgroup's cold start.
  u32x4_t pq_rsrc = {0u, 0u, 0u, 0u}, pk_rsrc = {0u, 0u, 0u, 0u};
  bool prefetch_next = false;
  if (p.schedule == 0 && p.next_stride > 0 && (int)blockIdx.x + p.next_stride < W) {
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
  auto prefetch_l2 = [&] __device__ (lds_u16_t* garbage) __attribute__((always_inline)) {
    constexpr int LPR = (DQK * 2 + 127) / 128;          // 128-byte lines per row
    const int pw = wave - kWaves / 2;                   // 0..3 in group 1
#pragma unroll
    for (int n = 0; n < LPR; ++n) {
      const int li = (n * 4 + pw) * 64 + lane;          // line index over 256 rows
      const uint32_t off = (uint32_t)(li / LPR) * k_rowbytes + (uint32_t)(li % LPR) * 128u;
      dma_dword(pq_rsrc, off, garbage);
      dma_dword(pk_rsrc, off, garbage);
    }
  };
  // Byte offset of tile t in the K or V resource; a tile past the last one
  // starts at the resource's end, so its DMAs return zeros without touching
  // memory.
  auto k_tile = [&] __device__ (int t) __attribute__((always_inline)) -> uint32_t {
    return t < ntiles ? (uint32_t)(t * BN) * k_rowbytes : k_bytes;
  };
  auto v_tile = [&] __device__ (int t) __attribute__((always_inline)) -> uint32_t {
    return t < ntiles ? (uint32_t)(t * BN) * v_rowbytes : v_bytes;
  };
  // DMA d (0 <= d < ISSUES) of this loader's share of the V tile at byte
  // offset tv, then of the K tile at tk (V first: it is awaited one phase
  // earlier than K)
  auto dma = [&] __device__ (int d, uint32_t tk, uint32_t tv, lds_u16_t* kdst, lds_u16_t* vdst)
      __attribute__((always_inline)) {
    if (d < Lay::V_ISSUES) {
      dma_chunk(v_rsrc, voff[d % Lay::V_PERIOD], tv + (uint32_t)(d / Lay::V_PERIOD) * v_period_bytes,
                vdst + (lw * Lay::V_ISSUES + d) * 512);
    } else {
      const int e = d - Lay::V_ISSUES;
      dma_chunk(k_rsrc, koff[e % Lay::K_PERIOD], tk + (uint32_t)(e / Lay::K_PERIOD) * k_period_bytes,
                kdst + (lw * Lay::K_ISSUES + e) * 512);
    }
  };

  // K rows are read in the order sigma(m) = m with bits 2 and 3 swapped: then
  // accumulator registers 0..7 (and 8..15) of a 32-key block hold 8
  // consecutive keys -- exactly the B-operand slots of the second product.
  // Per k-step LDS element offsets of this lane's K chunk (row sigma(lq)).
  int kread[QK_STEPS];
  {
    const int sig = (lq & ~0xC) | ((lq & 4) << 1) | ((lq & 8) >> 1);
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) kread[ks] = sig * DQK + (((2 * ks + g) ^ KSwz<DQK>::f(sig)) * 8);
  }
  // ds_read_b64_tr_b16 source addressing for the V^T operand: in each group of
  // 16 lanes, lane s reads 4 consecutive d-values of key row s/4; the
  // transpose hands lane i the values of 4 consecutive keys at d-column i.
  // Rows read are 4-aligned blocks plus s/4, so f_V depends on s/4 only.
  int vread[D_BLOCKS];
  {
    const int lg = lane / 16;
    const int sl = lane % 16;
    const int vrow = 8 * (lg / 2) + sl / 4;
#pragma unroll
    for (int db = 0; db < D_BLOCKS; ++db) {
      const int d = db * 32 + 16 * (lg % 2) + 4 * (sl % 4);
      vread[db] = vrow * DV + (((d / 8) ^ VSwz<DV>::f(vrow)) * 8) + (d % 8);
    }
  }

  // ---- per-wave state: S^T of the tile between its two phases and its raw
  // row max, P^T as bf16 B operands (zero before the first softmax), O^T
  // accumulators, running max (log2 units) and lane-partial row sum
  f32x16_t sacc[KB];
  float mx_raw = -__builtin_inff();
  u32x4_t pb[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) pb[kb][hh] = u32x4_t{0u, 0u, 0u, 0u};
  f32x16_t oacc[D_BLOCKS];
#pragma unroll
  for (int db = 0; db < D_BLOCKS; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -__builtin_inff();
  float l_part = 0.0f;
  const float c = p.c;
  const float tau = p.tau;
  // uniform: kept in an SGPR (a VGPR copy can be spilled and reloaded)
  const float tau_dec =
      __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __builtin_fmaxf(tau, 0.0f))));
  uint32_t n_considered = 0, n_taken = 0, n_tiles = 0;

  // Row max of S^T over the tile: lane-local over its 32 keys, then with the
  // partner lane holding the other half of the row.
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
  // One matrix phase as a single stream of MFMA slots: first the score
  // product S^T = K_t Q^T (slots (ks, kb)), then the output product
  // O^T += V_{t-1}^T P_{t-1}^T (slots (kb, hh, db), db fastest, so neighbours
  // accumulate into different blocks).  Under the output product's MFMAs the
  // wave takes the row max of S_t, a chain of dependent VALU operations that
  // would otherwise stall the softmax phase.  The LDS operand of slot s + kPrefetch is read before
  // the MFMA of slot s, and pin_matrix_schedule fixes that order, so each read
  // has several MFMAs (32 cycles each) to return; the operands of the first
  // kPrefetch slots are read (prefetch) at the end of the wave's previous
  // phase, so the stream starts without waiting for LDS.
  constexpr int NPV = KB * 2 * D_BLOCKS;
  constexpr int NQK = QK_STEPS * KB;
  constexpr int NS = NPV + NQK;
  static_assert(kPrefetch <= NQK, "prefetched slots are score-product slots");
  // A loader wave spreads its DMAs over its matrix phase, one every
  // kDmaStride slots, so the requests of the four loaders trickle into the
  // memory pipeline instead of queueing behind each other.
  constexpr int kDmaStride = NS / Lay::ISSUES;
  static_assert(kDmaStride >= 1, "DMAs per matrix phase");
  // A operand of slot s: for the output product two transposing reads give
  // V^T rows db*32.. at keys kb*32 + 16hh + (0..7); for the score product
  // one 16-byte read gives K row sigma(lq) of key block kb at k-step ks.
  auto read_op = [&] __device__ (int s, const lds_u16_t* vt, const lds_u16_t* kt) __attribute__((always_inline))
      -> bf16x8_t {
    if (s < NQK) {
      const int ks = s / KB, kb = s % KB;
      return *(const lds_bf16x8_t*)(kt + kread[ks] + kb * 32 * DQK);
    }
    const int q = s - NQK, kb = q / (2 * D_BLOCKS), hh = (q / D_BLOCKS) % 2, db = q % D_BLOCKS;
    const lds_u16_t* vr = vt + vread[db] + (kb * 32 + 16 * hh) * DV;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vr));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vr + 4 * DV));
    const i16x4_t both[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8_t, both);
  };
  bf16x8_t op_pre[kPrefetch];
  auto prefetch = [&] __device__ (const lds_u16_t* vt, const lds_u16_t* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) op_pre[s] = read_op(s, vt, kt);
  };
  // vt, kt: V tile of the output product and K tile of the score product;
  // with DMA, this loader's requests for K tile tk -> kdst and V tile tv ->
  // vdst are issued along the way.
  auto matrix = [&] __device__ (auto dma_tag, const lds_u16_t* vt, const lds_u16_t* kt, uint32_t tk, uint32_t tv,
                                lds_u16_t* kdst, lds_u16_t* vdst) __attribute__((always_inline)) {
    constexpr bool DMA = decltype(dma_tag)::value;
    bf16x8_t op[NS];
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) op[s] = op_pre[s];
    const f32x16_t zero = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + kPrefetch < NS) op[s + kPrefetch] = read_op(s + kPrefetch, vt, kt);
      if (s < NQK) {
        const int ks = s / KB, kb = s % KB;
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s], qreg[ks], ks == 0 ? zero : sacc[kb], 0, 0, 0);
      } else {
        const int q = s - NQK, kb = q / (2 * D_BLOCKS), hh = (q / D_BLOCKS) % 2, db = q % D_BLOCKS;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[s], __builtin_bit_cast(bf16x8_t, pb[kb][hh]),
                                                           oacc[db], 0, 0, 0);
      }
      if (DMA && s % kDmaStride == kDmaStride / 2 && s / kDmaStride < Lay::ISSUES)
        dma(s / kDmaStride, tk, tv, kdst, vdst);
    }
    mx_raw = row_max();
    // keep the row max in this phase: left alone, the compiler sinks it to
    // its first use, in the softmax phase
    asm volatile("" : "+v"(mx_raw));
    pin_matrix_schedule<0, NS, NQK>();
  };

  // Does the softmax of tile t need masking for this wave?
  auto needs_mask = [&] __device__ (int t) __attribute__((always_inline)) {
    const int k0 = t * BN;
    return (k0 + BN > L) || (CAUSAL && k0 + BN - 1 > qw0);
  };

  // ---- phases.  Iteration j (0 <= j <= ntiles) has two phases separated by
  // barriers.  Group 0: phase 1 = matrix(j): S[j] = K[j] Q^T, O += P[j-1]
  // V[j-1], issuing the DMAs of V[j] and K[j+2]; phase 2 = softmax(j).  Group
  // 1 runs one phase behind: phase 1 = softmax(j-1), phase 2 = matrix(j).
  // K[t] lives in K buffer t mod 3, V[t] in V buffer t mod 2 (V[-1] is the
  // zero-filled V buffer 1).  The loaders wait for V[j] before the end
  // barrier of iteration j and for K[j+2] before the mid barrier of
  // iteration j+1, so every tile is complete before any wave reads or
  // prefetches it; the buffers the DMAs of iteration j refill (K[j-1],
  // V[j-2]) were last read in iteration j-1.
  // Softmax of tile t (in sacc): masks, row max, conditional rescale of O and
  // l, P = exp2(c s - m) as bf16 B operands, and the row sums.
  auto softmax = [&] __device__ (int t) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      if (!own_keeps(t)) {                        // this wave's query block skips tile t
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) pb[kb][hh][jj] = 0u;
        return;
      }
    }
    const int k0 = t * BN;
    // Row max of the tile (raw logits; c > 0 so max commutes with scaling),
    // computed by the matrix phase; a masked tile masks S and takes it again.
    // Keeping the mask a separate branch leaves one path through the O
    // rescale below.
    float mx = mx_raw;
    if (needs_mask(t)) {
      const int lim = CAUSAL ? min(L - 1, qrow) : (L - 1);   // last visible key
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 16 * (r / 8) + 8 * g + (r % 8);
          if (key > lim) sacc[kb][r] = -__builtin_inff();
        }
      mx = row_max();
    }
    const float m_tile = (mx == -__builtin_inff()) ? mx : mx * c;
    // Rescale when the tile max exceeds the running max by more than tau
    // (log2 units).  tau < 0 asks for the classic rule, rescaling whenever
    // the max grows; a tile whose max did not grow would be rescaled by
    // exp2(0) = 1, an exact no-op, so both rules are taken here as
    // "m_tile > m_run + max(tau, 0)".  On the first tile m_run = -inf, so
    // every lane rescales its still-zero O and l (alpha = 0).
    const bool need = m_tile > m_run + tau_dec;
    // rescale statistics as wave totals (scalar registers)
    const bool counted = !SPARSE && row_valid && g == 0 && t >= 1 && t <= t_last;
    n_considered += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(counted));
    n_taken += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(counted && (need || tau < 0.0f)));
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? __builtin_fmaxf(m_run, m_tile) : m_run;
      const float alpha = need ? exp2_hw(m_run - m_new) : 1.0f;
#pragma unroll
      for (int db = 0; db < D_BLOCKS; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = oacc[db][r];
          scale_in_place(x, alpha);
          oacc[db][r] = x;
        }
      l_part *= alpha;
      m_run = m_new;
    }
    // P = exp2(c s - m) in fp32 (all FMAs before the exponentials, so no exp
    // waits on the FMA just before it), then bf16 B operands and the row sum.
    // Block-sparse rows can reach a tile with no visible key before any
    // other (m = -inf, every s = -inf): x must then be -inf, not NaN.
    const float neg_m = (SPARSE && m_run == -__builtin_inff()) ? 0.0f : -m_run;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = __builtin_fmaf(sacc[kb][r], c, neg_m);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[kb][r] = ((r % 8) < NPOLY / 2) ? exp2_poly(sacc[kb][r]) : exp2_hw(sacc[kb][r]);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          pb[kb][hh][jj] = pack_bf16x2(sacc[kb][8 * hh + 2 * jj], sacc[kb][8 * hh + 2 * jj + 1]);
    float acc[4] = {sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3]};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 4 : 0); r < 16; ++r) acc[r % 4] += sacc[kb][r];
    l_part += (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };

  // Every iteration runs the same matrix code, so the O accumulators keep
  // one register assignment: at j = 0 the output product multiplies zero P
  // with the zero-filled V buffer, and at j = ntiles the score product of a
  // stale K buffer is computed and dropped; DMAs past the last tile fill a
  // free buffer with zeros.  Causal tiles past a wave's diagonal go through the
  // softmax fully masked (P = 0, no rescale), which leaves O, l and m exactly
  // as skipping them would.
  auto run = [&] __device__ (auto grp_tag) __attribute__((always_inline)) {
    constexpr int G = decltype(grp_tag)::value;
    int b0 = 0;                                  // j mod 3
    // tiles number j-1, j, j+1, j+2 of the visiting order (tile j itself when dense)
    int t_prev = -1, t_cur = next_tile(-1);
    int t_n1 = next_tile(t_cur), t_n2 = next_tile(t_n1);
    if (G == 0) prefetch(vbuf(1), kbuf(0));      // operands of matrix(0)
    for (int j = 0; j <= nact; ++j) {
      const int bm1 = (b0 == 0) ? 2 : b0 - 1;    // (j - 1) mod 3 = (j + 2) mod 3
      const int bp1 = (b0 == 2) ? 0 : b0 + 1;    // (j + 1) mod 3
      const int vc = j & 1, vp = vc ^ 1;         // V buffers of V[j] and V[j-1]
#if ATTN_STAMPS
      uint64_t c0 = cycles_now(), c1;
#define ATTN_PHASE(i) (c1 = cycles_now(), ph[i] += c1 - c0, c0 = c1)
#else
#define ATTN_PHASE(i) ((void)0)
#endif
      if (G == 0) {
        if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(ATTN_SETPRIO);
        matrix(True{}, vbuf(vp), kbuf(b0), k_tile(t_n2), v_tile(t_cur), kbuf(bm1), vbuf(vc));
        if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
        ATTN_PHASE(0);
        dma_wait_barrier<Lay::ISSUES>();         // K[j+1] has landed
        ATTN_PHASE(1);
        if (j < nact) softmax(t_cur);
        prefetch(vbuf(vc), kbuf(bp1));           // operands of matrix(j+1)
        ATTN_PHASE(2);
        dma_wait_barrier<Lay::K_ISSUES>();       // V[j] has landed
        ATTN_PHASE(3);
      } else {
        if (prefetch_next && j == nact - 1) prefetch_l2(kbuf(bm1));
        if (j >= 1 && j - 1 < nact) softmax(t_prev);
        prefetch(vbuf(vp), kbuf(b0));            // operands of matrix(j)
        ATTN_PHASE(2);
        barrier();
        ATTN_PHASE(3);
        if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(ATTN_SETPRIO);
        matrix(False{}, vbuf(vp), kbuf(b0), 0u, 0u, kbuf(bm1), vbuf(vc));
        if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
        ATTN_PHASE(0);
        barrier();
        ATTN_PHASE(1);
      }
#undef ATTN_PHASE
      n_tiles += (j < nact && (SPARSE || j <= t_last)) ? 1u : 0u;
      b0 = bp1;
      t_prev = t_cur;
      t_cur = t_n1;
      t_n1 = t_n2;
      t_n2 = next_tile(t_n2);
    }
  };
  // Prologue: V buffer 1 is read (times P = 0) by matrix(0); the loaders fetch
  // K[0] and K[1] and wait for them before the first barrier.
  for (int i = tid; i < Lay::V_ELEMS / 8; i += kThreads) ((lds_u32x4_t*)vbuf(1))[i] = u32x4_t{0u, 0u, 0u, 0u};
  if (grp == 0) {
    const int t0 = next_tile(-1), t1 = next_tile(t0);
#pragma unroll
    for (int d = Lay::V_ISSUES; d < Lay::ISSUES; ++d) dma(d, k_tile(t0), 0u, kbuf(0), vbuf(0));
#pragma unroll
    for (int d = Lay::V_ISSUES; d < Lay::ISSUES; ++d) dma(d, k_tile(t1), 0u, kbuf(1), vbuf(0));
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
#if ATTN_STAMPS
  cy_loop0 = cycles_now();
#endif
  if (grp == 0) run(Grp0{});
  else run(Grp1{});
  dma_wait_all();   // the last iteration's DMAs land before the LDS is reused
#if ATTN_STAMPS
  cy_loop1 = cycles_now();
#endif

  // ---- epilogue: O = O^T / l (bf16), LSE = (m + log2 l) ln 2.  A lane holds
  // its query row's outputs in 8-byte pieces, so storing from registers would
  // scatter every store over 32 rows; the wave instead stages its 32 x d_v
  // tile in LDS (rows padded by 16 bytes) and writes whole rows back, four
  // rows of d_v = 128 per 16-byte-per-lane store.  The tiles' LDS is free once
  // every loader's last DMAs have landed.
  barrier();
  const float l_tot = sum_with_partner(l_part);
  // a block-sparse row that saw no key: O = 0 (and LSE = -inf + log 0 = -inf)
  const float inv = (SPARSE && l_tot == 0.0f) ? 0.0f : 1.0f / l_tot;
  constexpr int OS = DV + 8;                       // staged row stride (elements)
  lds_u16_t* const ost = lds + wave * kRowsPerWave * OS;
#pragma unroll
  for (int db = 0; db < D_BLOCKS; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2_t w;
      w.x = pack_bf16x2(oacc[db][4 * jj + 0] * inv, oacc[db][4 * jj + 1] * inv);
      w.y = pack_bf16x2(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
      *(__attribute__((address_space(3))) u32x2_t*)(ost + lq * OS + db * 32 + 8 * jj + 4 * g) = w;
    }
  {
    constexpr int CPR = DV / 8;                      // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                    // rows per store
    const int c = lane % CPR;
#pragma unroll
    for (int i = 0; i < kRowsPerWave / RPI; ++i) {
      const int r = i * RPI + lane / CPR;
      const u32x4_t w = *(const lds_u32x4_t*)(ost + r * OS + c * 8);
      if (qw0 + r < L) *(u32x4_t*)(p.o + (int64_t)(seq0 + qw0 + r) * H * DV + (int64_t)h * DV + c * 8) = w;
    }
  }
  if (row_valid && g == 0)
    p.lse[(int64_t)h * T + seq0 + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.693147180559945309f;

#if ATTN_STAMPS
  if (rec && lane == 0) {
    if (wave == 0) {
      rec[0] = rt_start;
      rec[2] = hardware_ids();
      rec[3] = ((uint64_t)h << 40) | ((uint64_t)b << 20) | (uint64_t)qblk;
      rec[4] = (uint64_t)nact + 1;
      rec[5] = cy_loop0 - cy_start;
      rec[6] = cy_loop1 - cy_loop0;
      rec[7] = cycles_now() - cy_loop1;
      for (int i = 0; i < 4; ++i) rec[8 + i] = ph[i];
      rec[1] = realtime_now();
    } else if (wave == kWaves / 2) {
      for (int i = 0; i < 4; ++i) rec[12 + i] = ph[i];
    }
  }
#endif
  if (!ATTN_STAMPS && p.stats) {
    // wave totals -> one atomic per counter per wave
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
  const dim3 grid = (p.schedule == 0) ? dim3(p.H * p.B * p.n_qblocks) : dim3(p.H, p.B, p.n_qblocks);
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
  static_assert(kMaskBlock % block_n(DQK) == 0, "tiles inside mask blocks");
  if (p.block_mask) {
    if (npoly != 0) return hipErrorInvalidValue;
    const dim3 grid = (p.schedule == 0) ? dim3(p.H * p.B * p.n_qblocks) : dim3(p.H, p.B, p.n_qblocks);
    if (causal) hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, true, 0, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, false, 0, true>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
  return causal ? launch_poly<DQK, DV, true>(p, npoly, s) : launch_poly<DQK, DV, false>(p, npoly, s);
}

int query_block_rows() { return kBlockM; }
int keys_per_tile(int d_qk) { return block_n(d_qk); }
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
