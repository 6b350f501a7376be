// tv_tree_attention_noalloc: tv_tree_attention with its workspace in a
// file-scope device array instead of caller or library allocations, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that forbid allocation).  Each device holds its own copy of
// the array (a code-object global) until the process ends; its address on a
// device is looked up once, with that device current, and only that address
// is handed to kernels and copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tv_internal.h"

namespace {

static __device__ __align__(256) char scratch[TV_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

// Zero n words: the merge counters must start each call at zero (a kernel
// rather than a memset node, so the call can be captured into a graph).
__global__ void clear_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

tv_status tv_tree_attention_noalloc(const tv_attn_desc* desc, const tv_attn_ptrs* ptrs,
                                    int32_t* dev_err, hipStream_t stream) {
  void* ws = scratch_on_current_device();
  if (!ws) return TV_ERR_DEVICE;
  tv::AttnPlan plan{};
  bool empty = false;
  const tv_status st = tv::prepare_attention(desc, ptrs, ws, &plan, &empty);
  if (st != TV_OK || empty) return st;
  if (plan.ws_bytes() > (size_t)TV_ATTN_NOALLOC_SCRATCH_BYTES) return TV_ERR_WORKSPACE;
  const int words = (int)(plan.ws_sync_bytes / sizeof(uint32_t));
  hipLaunchKernelGGL(clear_words, dim3(8), dim3(256), 0, stream, static_cast<uint32_t*>(ws), words);
  if (hipGetLastError() != hipSuccess) return TV_ERR_LAUNCH;
  return tv::launch_attention(*desc, plan, *ptrs, ws, dev_err, stream) == hipSuccess ? TV_OK
                                                                                     : TV_ERR_LAUNCH;
}
