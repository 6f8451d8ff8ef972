// Device-side pieces shared by the bf16 and FP8 forward kernels (and the
// backward dQ kernel's LDS DMAs): wave and
// workgroup geometry, cross-lane reductions, the LDS DMA requests with their
// wait-state padding, buffer resources and the phase barriers.
#ifndef EXACT_ATTENTION_57_AMD_ATTN_FWD_COMMON_H
#define EXACT_ATTENTION_57_AMD_ATTN_FWD_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef ATTN_DMA_NOP
#define ATTN_DMA_NOP 4   // s_nop operand in front of each LDS DMA (4: five wait states)
#endif
#define ATTN_STR2(x) #x
#define ATTN_STR(x) ATTN_STR2(x)
#ifndef ATTN_PREFETCH
#define ATTN_PREFETCH 4  // matrix-phase LDS operands read ahead of their MFMA
#endif
#ifndef ATTN_SETPRIO
#define ATTN_SETPRIO 1  // issue priority of the wave in its matrix phase (0: no change)
#endif
// Race-check build (1): every workgroup barrier first waits for all of the
// wave's memory traffic (LDS DMAs and LDS reads included) and is passed
// twice, so no DMA, LDS access or phase overlaps a barrier.  Its outputs must
// equal the default build's bit for bit; a tile read before its DMA landed, or
// a buffer refilled while still being read, would make them differ.
#ifndef ATTN_RACE_CHECK
#define ATTN_RACE_CHECK 0
#endif
// Instrumented build (1): the forward kernels write a timing record per
// workgroup after the four counters of attn_fwd_opts.stats (real-time start
// and end, hardware ids, per-phase cycle sums; see attn_fwd_kernel.hip).
#ifndef ATTN_STAMPS
#define ATTN_STAMPS 0
#endif

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

// Cubic p(r) = 1 + C1 r + C2 r^2 + C3 r^3 minimising max |p(r)/2^r - 1| on
// [0, 1] (relative minimax, max error 8.56e-5), rounded to fp32.  Derived by
// gen_exp2_coeffs.py in this directory (a linear program on a dense grid).
constexpr float kExp2C1 = 0x1.63e66ap-1f;   // 0.695117295
constexpr float kExp2C2 = 0x1.d236c6p-3f;   // 0.227643535
constexpr float kExp2C3 = 0x1.3babb0p-4f;   // 0.0770680308

constexpr int kWave = 64;
constexpr int kWaves = 8;              // two per SIMD: one per ping-pong group
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kRowsPerWave * kWaves;   // query rows per workgroup
// Keys per tile: 128 where the registers allow it (d_qk <= 128), else 64
// (96 also fits at d_qk = 192 but measured no faster, and the block-sparse
// kernel needs tiles that divide its 128-key mask blocks).
// Larger tiles halve the per-tile cost of the phase barriers and the
// softmax's row-wide steps.
#ifndef ATTN_BLOCK_N_SMALL_D
#define ATTN_BLOCK_N_SMALL_D 128
#endif
#ifndef ATTN_BLOCK_N_LARGE_D
#define ATTN_BLOCK_N_LARGE_D 64
#endif
constexpr int block_n(int d_qk) { return d_qk <= 128 ? ATTN_BLOCK_N_SMALL_D : ATTN_BLOCK_N_LARGE_D; }
constexpr int kXcds = 8;                         // MI355X: 8 XCDs, each with its own L2

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

// x *= a, in the register that holds x.  The O accumulators are rescaled
// only on the rare tiles whose row max grew; writing the product back into
// the same register keeps the allocator from copying all of O on the common
// path that skips the multiply.  (Every MFMA that wrote x completed before
// the barrier that precedes any rescale.)
__device__ __forceinline__ void scale_in_place(float& x, float a) {
  asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x) : "v"(a));
}

// Two fp32 values -> two bf16 (round to nearest even) in one dword, low first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Tiles are filled by the four group-0 waves, during their matrix phases.
constexpr int kLoaders = kWaves / 2;
constexpr int kKBufs = 3;                // K tile buffers in LDS
constexpr int kVBufs = 2;                // V tile buffers in LDS

// Smallest number p of consecutive 1 KB DMA requests (64 chunks of 16 bytes)
// after which a loader's chunk pattern repeats: a whole number of rows of R
// chunks that is also a multiple of the swizzle period.  Request i then uses
// the lane offset of request i mod p, shifted by whole rows.
constexpr int dma_period(int R, int swizzle_rows) {
  for (int p = 1; p < 64; ++p)
    if ((p * 64) % R == 0 && ((p * 64 / R) % swizzle_rows) == 0) return p;
  return 64;
}

// One buffer_load_dwordx4 ... lds request: copies, for every lane, the
// 16-byte chunk at byte offset lane_off + tile_off (from the resource base) to
// bytes 16*lane .. 16*lane+15 of the 1 KB LDS block at dst.  Offsets past the
// resource's byte count read as zeros.
//
// The request is inline assembly so that the compiler does not track it: it
// cannot tell which LDS buffer a DMA writes, and would make every later LDS
// read of the wave wait for all DMAs in flight.  Completion is awaited
// explicitly (dma_wait_barrier) before the barrier that precedes the tile's
// first read.  The host compilation pass only needs the kernels' launch stubs
// and sees an empty body.
__device__ __forceinline__ void dma_chunk(const u32x4_t& rsrc, uint32_t lane_off, uint32_t tile_off,
                                          lds_u16_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  // s_nop ATTN_DMA_NOP: the compiler's hazard checks do not look inside
  // inline assembly, and a VMEM instruction may read an SGPR only five wait
  // states after a VALU instruction wrote it (v_readlane reloads of spilled
  // SGPRs, v_readfirstlane); an LDS DMA needs one after the M0 write.  The
  // default 4 (five wait states) is always safe; the build uses 0 only for a
  // compilation whose assembly it has checked for both hazards.
  asm volatile("s_nop " ATTN_STR(ATTN_DMA_NOP) "\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "{m0}"(m0), "v"(lane_off), "s"(rsrc), "s"(tile_off)
               : "memory");
#endif
}

// One buffer_load_dword ... lds request (4 bytes per lane into the 256-byte
// LDS block at dst), used only to pull lines into L2.
__device__ __forceinline__ void dma_dword(const u32x4_t& rsrc, uint32_t lane_off, lds_u16_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  // the same wait states as dma_chunk
  asm volatile("s_nop " ATTN_STR(ATTN_DMA_NOP) "\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "{m0}"(m0), "v"(lane_off), "s"(rsrc)
               : "memory");
#endif
}

// Buffer resource for a byte range starting at base: raw (unswizzled)
// addressing, no stride, num_records = nbytes, so that reads at or past
// nbytes return zeros.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(nbytes);
  r.w = 0x00020000u;
  return r;
}

// Workgroup barriers of the phase schedule.  The memory clobber keeps the
// compiler from moving LDS accesses across them.  No LDS wait is needed
// before a barrier: every LDS read is either consumed by an MFMA of the same
// phase (so it has returned) or reads a buffer that is not refilled for
// another iteration.
__device__ __forceinline__ void barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
#if ATTN_RACE_CHECK
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier\n\ts_barrier" ::: "memory");
#else
  asm volatile("s_barrier" ::: "memory");
#endif
#endif
}
// Wait until at most N of this wave's DMAs are in flight, then barrier: the
// older DMAs have landed in LDS and, once every loader has waited, are
// visible to all waves.
template <int N>
__device__ __forceinline__ void dma_wait_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
#if ATTN_RACE_CHECK
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier\n\ts_barrier" ::: "memory");
#else
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
#endif
#endif
}
__device__ __forceinline__ void dma_wait_all() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

// Clocks of the instrumented build: s_memtime counts shader clock cycles,
// s_memrealtime a constant-rate (100 MHz) clock common to the whole chip.
__device__ __forceinline__ uint64_t cycles_now() {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_s_memtime();
#else
  return 0;
#endif
}
__device__ __forceinline__ uint64_t realtime_now() {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_s_memrealtime();
#else
  return 0;
#endif
}
// (XCC id << 32) | HW_ID (CU, SIMD, shader array and engine of this wave)
__device__ __forceinline__ uint64_t hardware_ids() {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t hw = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));    // HW_REG_HW_ID, 32 bits
  const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11));  // HW_REG_XCC_ID, 16 bits
  return ((uint64_t)xcc << 32) | hw;
#else
  return 0;
#endif
}
constexpr int kStampWords = 16;   // uint64 per workgroup record of the instrumented build

struct True { static constexpr bool value = true; };
struct False { static constexpr bool value = false; };
struct Grp0 { static constexpr int value = 0; };
struct Grp1 { static constexpr int value = 1; };

}  // namespace attn

#endif
