// Argument checks and launch of the backward pass, shared by the entry points
// that take the D workspace from the caller (attn_bwd) and from the library's
// static scratch array (attn_bwd_noalloc).
#ifndef EXACT_ATTENTION_57_AMD_ATTN_API_INTERNAL_H
#define EXACT_ATTENTION_57_AMD_ATTN_API_INTERNAL_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attn_internal {

constexpr int kNothingToDo = 1;   // bwd_check: valid arguments and N == 0

// Every check of attn_bwd's arguments, in its order, before any HIP call;
// the D workspace pointer is checked only when with_delta.  Returns ATTN_OK,
// kNothingToDo or a negative attn_status.
int bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              const void* dq, const void* dk, const void* dv, const float* delta, bool with_delta,
              const int32_t* cu_seqlens, int B, int H, int N, int d_qk, int d_v, float scale);

// The three backward kernels on `stream` (arguments already checked).
int bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, float* delta, const int32_t* cu_seqlens, int B, int H, int N,
               int d_qk, int d_v, float scale, int causal, hipStream_t stream);

}  // namespace attn_internal

#endif
