// Allocation-free backward pass: attn_bwd with its D workspace (the row terms
// D_i = dO_i . O_i, fp32 [H, T]) in a static device array of this library
// instead of a caller-supplied buffer, for callers that cannot allocate device
// memory (work under stream capture, serving loops or harnesses that forbid
// allocation).  The kernels are attn_bwd's.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code its name only identifies the symbol; the device address of the
// current GPU's copy comes from hipGetSymbolAddress, taken once per device on
// the first call there and kept, and only that address reaches the kernels.
// Calls on one GPU share its copy: calls that overlap in time on that GPU
// (different streams, or different threads) race on it.  Nothing in it needs
// to start at zero: the D pass writes every row the later kernels read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn.h"
#include "attn_api_internal.h"

namespace {

constexpr int64_t kScratchFloats = ATTN_NOALLOC_MAX_ROWS;   // 64 MiB of fp32 per GPU

__device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch`, looked up once per
// device; nullptr if the device or the symbol cannot be resolved.
float* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens, int B,
                                int H, int N, int d_qk, int d_v, float scale, int causal, hipStream_t stream) {
  const int st = attn_internal::bwd_check(q, k, v, o, dout, lse, dq, dk, dv, nullptr, false, cu_seqlens, B, H, N,
                                          d_qk, d_v, scale);
  if (st != ATTN_OK) return st == attn_internal::kNothingToDo ? ATTN_OK : st;
  // D has H * T rows, T = B * N at most
  if ((int64_t)H * B * N > kScratchFloats) return ATTN_ERR_SCRATCH;
  float* const delta = scratch_on_current_device();
  if (delta == nullptr) return ATTN_ERR_LAUNCH;
  return attn_internal::bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, delta, cu_seqlens, B, H, N, d_qk, d_v, scale,
                                   causal, stream);
}
