// Internal interface between the C-ABI backward entry point and its HIP kernels.
#ifndef EXACT_ATTENTION_57_AMD_ATTN_BWD_KERNEL_H
#define EXACT_ATTENTION_57_AMD_ATTN_BWD_KERNEL_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attn_grad {

// Kernel arguments (validated by the entry point before any launch).
struct BwdParams {
  const uint16_t* q;          // bf16 [T, H, d_qk]
  const uint16_t* k;          // bf16 [T, H, d_qk]
  const uint16_t* v;          // bf16 [T, H, d_v]
  const uint16_t* o;          // bf16 [T, H, d_v]   forward output
  const uint16_t* dout;       // bf16 [T, H, d_v]   gradient of the output
  const float* lse;           // fp32 [H, T]        forward LSE (natural log)
  uint16_t* dq;               // bf16 [T, H, d_qk]
  uint16_t* dk;               // bf16 [T, H, d_qk]
  uint16_t* dv;               // bf16 [T, H, d_v]
  float* delta;               // fp32 [H, T]        workspace: D = rowsum(dO * O)
  const int32_t* cu_seqlens;  // device int32 [B+1], or nullptr for fixed length N
  int B, H, N;                // T (total tokens) is B*N, or cu_seqlens[B] read on the device
  int n_blocks;               // ceil(N / block_rows())
  float scale;                // softmax scale
  float c;                    // scale * log2(e)
};

int block_rows();             // key rows per dK/dV workgroup (the dQ kernel takes 256 query rows each)
hipError_t launch_bwd(const BwdParams& p, int d_qk, int d_v, bool causal, hipStream_t s);

}  // namespace attn_grad

#endif
