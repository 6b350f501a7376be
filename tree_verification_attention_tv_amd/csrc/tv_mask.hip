// Ancestor-or-self bitmask of a draft tree (SpecBlock App. A.2: a node sees
// its on-path ancestors and itself, never other branches).
//
// One workgroup per sequence.  The parent array is staged in LDS and
// validated first; then thread i walks from node i to the root, setting one
// bit per visited node in its own LDS row, and the finished [N][W] block is
// written out with coalesced stores.  N <= 256 keeps a row in 8 words.
#include "tv_device.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxWords = TV_MAX_NODES / 32;

__global__ __launch_bounds__(kThreads) void build_mask_kernel(const int32_t* __restrict__ parents,
                                                             int n, int words,
                                                             uint32_t* __restrict__ mask,
                                                             int32_t* __restrict__ depth,
                                                             int32_t* __restrict__ dev_err) {
  __shared__ int par[TV_MAX_NODES];
  __shared__ uint32_t rows[TV_MAX_NODES * kMaxWords];
  __shared__ int bad;

  const int b = blockIdx.x;
  const int i = threadIdx.x;
  if (i == 0) bad = 0;
  for (int k = i; k < n * words; k += kThreads) rows[k] = 0u;
  __syncthreads();

  if (i < n) {
    const int p = parents[(int64_t)b * n + i];
    par[i] = p;
    const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
    if (!ok) bad = 1;  // benign race: every writer stores 1
  }
  __syncthreads();

  if (i < n) {
    int d = 0;
    uint32_t* row = rows + i * words;
    row[i >> 5] |= 1u << (i & 31);
    if (!bad) {
      // parents precede children, so the walk strictly decreases and ends
      for (int j = par[i]; j >= 0; j = par[j]) {
        row[j >> 5] |= 1u << (j & 31);
        ++d;
      }
    }
    if (depth) depth[(int64_t)b * n + i] = d;
  }
  __syncthreads();

  uint32_t* out = mask + (int64_t)b * n * words;
  for (int k = i; k < n * words; k += kThreads) out[k] = rows[k];
  if (i == 0 && bad) raise_err(dev_err, TV_DERR_BAD_PARENT);
}

}  // namespace

hipError_t launch_build_mask(const int32_t* parents, int batch, int n, uint32_t* mask,
                             int32_t* depth, int32_t* dev_err, hipStream_t stream) {
  const int words = (n + 31) / 32;
  hipLaunchKernelGGL(build_mask_kernel, dim3(batch), dim3(kThreads), 0, stream, parents, n, words,
                     mask, depth, dev_err);
  return hipGetLastError();
}

}  // namespace tv
