// Internal interface between the C-ABI entry points and the HIP kernels.
#ifndef EXACT_ATTENTION_57_AMD_ATTN_FWD_KERNEL_H
#define EXACT_ATTENTION_57_AMD_ATTN_FWD_KERNEL_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attn {

// Kernel arguments (validated by the entry points before any launch).
struct FwdParams {
  const uint16_t* q;          // bf16 [T, H, d_qk]
  const uint16_t* k;          // bf16 [T, H, d_qk]
  const uint16_t* v;          // bf16 [T, H, d_v]
  uint16_t* o;                // bf16 [T, H, d_v]
  float* lse;                 // fp32 [H, T]
  const int32_t* cu_seqlens;  // device int32 [B+1], or nullptr for fixed length N
  int B, H, N;
  int n_qblocks;              // ceil(N / query_block_rows())
  float c;                    // |scale| * log2(e), at least 1e-30
  int neg_scale;              // 1: scale < 0, Q is negated on load (exact)
  float tau;                  // rescale threshold in log2 units; < 0: always rescale
  int schedule;               // 0: longest-first, 1: natural order
  int next_stride;            // 1-D grid distance to the workgroup that starts next on the
                              // same XCD (the CU count), whose inputs are prefetched; 0: none
  unsigned long long* stats;  // optional device counters [4]
  const uint8_t* block_mask;  // optional device uint8 [B, H, mask_blocks, mask_blocks]: 128 x 128
                              // (query block, key block) pairs kept (nonzero) or skipped
  int mask_blocks;            // ceil(N / 128)
};

// FP8 forward: q, k, v hold OCP E4M3 bytes; S = scale * q_descale * k_descale * Q K^T
// and O = v_descale * P V / l.
struct Fp8Params {
  const uint8_t* q;           // e4m3 [T, H, d_qk]
  const uint8_t* k;           // e4m3 [T, H, d_qk]
  const uint8_t* v;           // e4m3 [T, H, d_v]
  uint16_t* o;                // bf16 [T, H, d_v]
  float* lse;                 // fp32 [H, T]
  const int32_t* cu_seqlens;  // device int32 [B+1], or nullptr for fixed length N
  int B, H, N;
  int n_qblocks;              // ceil(N / query_block_rows())
  float c;                    // |scale| * q_descale * k_descale * log2(e), at least 1e-30
  int neg_scale;              // 1: scale < 0, Q is negated on load (exact)
  float o_scale;              // v_descale
  float tau;                  // rescale threshold in log2 units, 0 <= tau <= 8 (P <= 256 < 448)
  int next_stride;            // as in FwdParams
};

int query_block_rows();
int keys_per_tile(int d_qk);
int rows_per_wave();
hipError_t launch_fwd(const FwdParams& p, int d_qk, int d_v, bool causal, int npoly, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8Params& p, int d_qk, int d_v, bool causal, hipStream_t s);
hipError_t launch_exp2_debug(const float* x, float* y, int n, int use_poly, hipStream_t s);

}  // namespace attn

#endif
