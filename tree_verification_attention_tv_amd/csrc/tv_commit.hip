// Commit of the accepted path's K/V rows into the cache (SpecBlock App. A.5:
// the longest accepted prefix is committed before the next iteration).
//
// One workgroup per (sequence, layer) copies (accept_len + 1) * Hkv * 2 rows
// with 16-byte vector moves; the layers' tensors lie at fixed strides from
// layer 0's.  The sequence's prefix length is read once by thread 0 before
// any write, and the layer-0 workgroup's thread 0 writes the new length after
// its copy, so with a single layer new_prefix_len may alias prefix_len (with
// several, another layer's workgroup may start after that write, so the host
// refuses the alias).  Layer 0 alone reports the (shared) error bits.
#include "tv_device.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;  // copy items per thread in flight

__global__ __launch_bounds__(kThreads) void commit_kernel(
    const uint4* __restrict__ k_tree, const uint4* __restrict__ v_tree,
    const int32_t* __restrict__ path, const int32_t* __restrict__ accept_len,
    const int32_t* prefix_len, int32_t* new_prefix_len, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int64_t seq_stride_vec, int cap, int n, int hkv, int vec_per_row,
    int64_t tree_layer_vec, int64_t cache_layer_vec, int32_t* __restrict__ dev_err) {
  __shared__ int s_prefix, s_len, s_ok;
  __shared__ int s_node[TV_MAX_NODES];
  const int b = blockIdx.x;
  const int layer = blockIdx.y;
  const int t = threadIdx.x;
  k_tree += layer * tree_layer_vec;
  v_tree += layer * tree_layer_vec;
  k_cache += layer * cache_layer_vec;
  v_cache += layer * cache_layer_vec;
  int32_t* const err_out = layer == 0 ? dev_err : nullptr;
  // One round trip for every small input: the path entries are read before
  // accept_len is known (t < n is always in bounds).
  const int node_t = t < n ? path[(int64_t)b * n + t] : 0;
  if (t == 0) {
    const int p = prefix_len[b];
    const int a = accept_len[b];
    int ok = 1;
    if (p < 0 || p > cap) {
      raise_err(err_out, TV_DERR_BAD_PREFIX);
      ok = 0;
    } else if (a < 0 || a >= n) {
      raise_err(err_out, TV_DERR_BAD_PATH);
      ok = 0;
    } else if ((int64_t)p + a + 1 > cap) {
      raise_err(err_out, TV_DERR_CAPACITY);
      ok = 0;
    }
    s_prefix = p;
    s_len = a;
    s_ok = ok;
  }
  __syncthreads();
  const int a = s_len;
  if (s_ok && t <= a) {
    s_node[t] = node_t;
    if (node_t < 0 || node_t >= n) {
      raise_err(err_out, TV_DERR_BAD_PATH);
      s_ok = 0;  // benign race: every writer stores 0
    }
  }
  __syncthreads();
  if (s_ok) {
    const int p = s_prefix;
    const int per_row = vec_per_row;
    const int items = (a + 1) * hkv * per_row;
    const uint4* kt = k_tree + (int64_t)b * n * hkv * per_row;
    const uint4* vt = v_tree + (int64_t)b * n * hkv * per_row;
    uint4* kc = k_cache + b * seq_stride_vec;
    uint4* vc = v_cache + b * seq_stride_vec;
    // batches of kBatch items per thread: all loads, then all stores
    auto locate = [&](int it, int64_t& src, int64_t& dst) {
      const int c = it % per_row;
      const int rh = it / per_row;
      const int h = rh % hkv;
      const int r = rh / hkv;
      src = ((int64_t)s_node[r] * hkv + h) * per_row + c;
      dst = ((int64_t)h * cap + p + r) * per_row + c;
    };
    for (int it0 = t; it0 < items; it0 += kBatch * kThreads) {
      uint4 kx[kBatch], vx[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int it = min(it0 + u * kThreads, items - 1);  // clamped: always a valid item
        int64_t src, dst;
        locate(it, src, dst);
        kx[u] = kt[src];
        vx[u] = vt[src];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int it = it0 + u * kThreads;
        if (it < items) {
          int64_t src, dst;
          locate(it, src, dst);
          kc[dst] = kx[u];
          vc[dst] = vx[u];
        }
      }
    }
  }
  if (t == 0 && layer == 0) new_prefix_len[b] = s_ok ? s_prefix + a + 1 : s_prefix;
}

}  // namespace

hipError_t launch_commit(const void* k_tree, const void* v_tree, const int32_t* path,
                         const int32_t* accept_len, const int32_t* prefix_len,
                         int32_t* new_prefix_len, void* k_cache, void* v_cache,
                         int64_t seq_stride, int cap, int batch, int n, int hkv, int d,
                         int layers, int64_t tree_layer_stride, int64_t cache_layer_stride,
                         int32_t* dev_err, hipStream_t stream) {
  const int vec_per_row = d / 8;  // 8 bf16 per 16-byte vector
  hipLaunchKernelGGL(commit_kernel, dim3(batch, layers), dim3(kThreads), 0, stream,
                     (const uint4*)k_tree, (const uint4*)v_tree, path, accept_len, prefix_len,
                     new_prefix_len, (uint4*)k_cache, (uint4*)v_cache, seq_stride / 8, cap, n, hkv,
                     vec_per_row, tree_layer_stride / 8, cache_layer_stride / 8, dev_err);
  return hipGetLastError();
}

}  // namespace tv
