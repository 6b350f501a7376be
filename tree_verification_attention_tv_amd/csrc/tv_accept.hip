// Greedy (temperature-0) acceptance of a verified draft tree.
//
// Sources: SpecBlock Sec. 4 (greedy decoding), App. A.5 (longest accepted
// prefix is committed), App. E (one bonus token from the target); papernotes
// on SpecBlock, key design 3 (valid-prefix recurrence: a position stays
// valid only while every earlier prediction matched the target's argmax).
//
// Two kernels:
//  1. vocab_argmax_kernel: one workgroup per (row chunk, logits row).  Each
//     thread streams 16-byte vectors of its chunk, keeps the first index of
//     its running maximum, and the workgroup reduces (value, index) pairs
//     with "larger value, then smaller index" -- a total order, so the
//     result does not depend on the reduction order.  Partials go to the
//     workspace.  This is the HBM-bound part (B*N*V logits).
//  2. path_walk_kernel: one workgroup per sequence.  Thread i finishes row
//     i's argmax from the partials and tests its own edge,
//     draft[i] == argmax[parent(i)]; the result is packed with the parent
//     index in LDS.  Then thread i walks from node i to the root, one LDS
//     read per level, and stops at the first rejected edge; the deepest
//     accepted node (lowest index on ties) is found with one max-reduction
//     of depth * 65536 + (65535 - i), and its root path is written out.
#include "tv_device.h"

#include <float.h>

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte bf16 vectors per thread per chunk (fp32: twice as many)

// Optional commit done by the walk (tv_greedy_accept_commit); k_cache == null: none
struct CommitArgs {
  const uint4* k_tree;
  const uint4* v_tree;
  const int32_t* prefix_len;
  int32_t* new_prefix_len;
  uint4* k_cache;
  uint4* v_cache;
  int64_t seq_stride_vec;
  int cap, hkv, vec_per_row;
  int64_t tree_layer_vec, cache_layer_vec;  // 16-byte vectors between layers
};

struct ValIdx {
  float v;
  int i;
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int CTRL>
__device__ __forceinline__ void dpp_take(ValIdx& a) {
  // row rotation: every lane of a 16-lane row sees another lane of the row
  const float ov = __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(a.v), __float_as_int(a.v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(a.i, a.i, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, a.v, a.i)) {
    a.v = ov;
    a.i = oi;
  }
}

__device__ __forceinline__ void swap_take16(ValIdx& a) {
  const auto v = __builtin_amdgcn_permlane16_swap(__float_as_uint(a.v), __float_as_uint(a.v), false, false);
  const auto i = __builtin_amdgcn_permlane16_swap((unsigned)a.i, (unsigned)a.i, false, false);
  // each lane now holds its own value and its partner row's in (v[0], v[1])
  ValIdx x{__uint_as_float(v[0]), (int)i[0]}, y{__uint_as_float(v[1]), (int)i[1]};
  a = better(y.v, y.i, x.v, x.i) ? y : x;
}

__device__ __forceinline__ void swap_take32(ValIdx& a) {
  const auto v = __builtin_amdgcn_permlane32_swap(__float_as_uint(a.v), __float_as_uint(a.v), false, false);
  const auto i = __builtin_amdgcn_permlane32_swap((unsigned)a.i, (unsigned)a.i, false, false);
  ValIdx x{__uint_as_float(v[0]), (int)i[0]}, y{__uint_as_float(v[1]), (int)i[1]};
  a = better(y.v, y.i, x.v, x.i) ? y : x;
}

// every lane gets the wave's (largest value, smallest index) pair: row
// rotations by 8, 4, 2, 1 (DPP), then the gfx950 row swaps across rows.
// The order is total, so the result does not depend on the combining order.
__device__ __forceinline__ ValIdx wave_argmax(ValIdx a) {
  dpp_take<0x128>(a);
  dpp_take<0x124>(a);
  dpp_take<0x122>(a);
  dpp_take<0x121>(a);
  swap_take16(a);
  swap_take32(a);
  return a;
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}

// wave-wide max of a float and min of an int (every lane gets the result):
// row rotations by 8, 4, 2, 1, then the row swaps
__device__ __forceinline__ float wave_max_f(float x) {
  x = fmaxf(x, __int_as_float(dpp_i<0x128>(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_i<0x124>(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_i<0x122>(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_i<0x121>(__float_as_int(x))));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ int wave_min_i(int x) {
  x = min(x, dpp_i<0x128>(x));
  x = min(x, dpp_i<0x124>(x));
  x = min(x, dpp_i<0x122>(x));
  x = min(x, dpp_i<0x121>(x));
  const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = min((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return min((int)b[0], (int)b[1]);
}

__device__ __forceinline__ unsigned wave_max_u(unsigned x) {
  x = max(x, (unsigned)dpp_i<0x128>((int)x));
  x = max(x, (unsigned)dpp_i<0x124>((int)x));
  x = max(x, (unsigned)dpp_i<0x122>((int)x));
  x = max(x, (unsigned)dpp_i<0x121>((int)x));
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(b[0], b[1]);
}

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 x) {
  return (float)x;
}
template <>
__device__ __forceinline__ float to_f32<float>(float x) {
  return x;
}

// VEC elements of T per 16-byte load
template <typename T, bool kVector>
__global__ __launch_bounds__(kThreads) void vocab_argmax_kernel(const T* __restrict__ logits,
                                                               int64_t vocab, int64_t row_stride,
                                                               int64_t chunk_len, int chunks,
                                                               float* __restrict__ part_v,
                                                               int* __restrict__ part_i) {
  constexpr int VEC = 16 / sizeof(T);
  const int chunk = blockIdx.x;
  const int64_t row = blockIdx.y;
  const T* src = logits + row * row_stride;
  const int64_t begin = (int64_t)chunk * chunk_len;
  int64_t end = begin + chunk_len;
  if (end > vocab) end = vocab;

  float bv = -INFINITY;
  int bi = INT32_MAX;
  auto take = [&](float f, int64_t k) {
    // scanning in increasing index: a strict '>' keeps the first occurrence
    if (f > bv || bi == INT32_MAX) {
      bv = f;
      bi = (int)k;
    }
  };
  if (kVector) {
    typedef T vec_t __attribute__((ext_vector_type(VEC)));
    // All of the thread's loads are issued before any is used, so the chunk
    // costs one memory round trip.  Vector u of thread t covers elements
    // begin + (u * kThreads + t) * VEC .. +VEC-1 (coalesced for each u).
    // chunk_len <= kThreads * 8 * kUnroll = kThreads * VEC * U elements, so
    // U vectors per thread cover the chunk; only the last chunk is ragged
    // (elements past its end read as -inf and are never chosen).
    constexpr int U = kUnroll * 8 / VEC;
    vec_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t base = begin + ((int64_t)u * kThreads + threadIdx.x) * VEC;
      if (base + VEC <= end) {
        x[u] = *reinterpret_cast<const vec_t*>(src + base);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[u][e] = base + e < end ? src[base + e] : (T)(-INFINITY);
      }
    }
    // Two passes over the registers: the workgroup's largest value first
    // (a max per element), then, only in the threads that hold it, the
    // first index equal to it (values compare as reals, -0 == +0).  A
    // running (value, index) update per element would cost three times the
    // VALU work.
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) m = fmaxf(m, to_f32<T>(x[u][e]));
    __shared__ float s_max[kThreads / kWave];
    const int w = threadIdx.x / kWave;
    const float wm = wave_max_f(m);
    if ((threadIdx.x & (kWave - 1)) == 0) s_max[w] = wm;
    __syncthreads();
    float big = s_max[0];
#pragma unroll
    for (int k = 1; k < kThreads / kWave; ++k) big = fmaxf(big, s_max[k]);
    int first = INT32_MAX;
    if (m == big) {
#pragma unroll
      for (int u = U - 1; u >= 0; --u) {
        const int64_t base = begin + ((int64_t)u * kThreads + threadIdx.x) * VEC;
#pragma unroll
        for (int e = VEC - 1; e >= 0; --e)
          if (to_f32<T>(x[u][e]) == big && base + e < end) first = (int)(base + e);
      }
    }
    __shared__ int s_first[kThreads / kWave];
    const int wf = wave_min_i(first);
    if ((threadIdx.x & (kWave - 1)) == 0) s_first[w] = wf;
    __syncthreads();
    if (threadIdx.x == 0) {
      int f = s_first[0];
      for (int k = 1; k < kThreads / kWave; ++k) f = min(f, s_first[k]);
      part_v[row * chunks + chunk] = big;
      part_i[row * chunks + chunk] = f;
    }
    return;
  } else {
    for (int64_t k = begin + threadIdx.x; k < end; k += kThreads) take(to_f32<T>(src[k]), k);
  }

  ValIdx a = wave_argmax(ValIdx{bv, bi});
  __shared__ float sv[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sv[wave] = a.v;
    si[wave] = a.i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / kWave; ++w)
      if (better(sv[w], si[w], a.v, a.i)) {
        a.v = sv[w];
        a.i = si[w];
      }
    part_v[row * chunks + chunk] = a.v;
    part_i[row * chunks + chunk] = a.i;
  }
}

__global__ __launch_bounds__(kThreads) void path_walk_kernel(
    const float* __restrict__ part_v, const int* __restrict__ part_i, int chunks,
    const int32_t* __restrict__ parents, const int32_t* __restrict__ draft, int n,
    int32_t* __restrict__ target_argmax, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ accept_path, int32_t* __restrict__ bonus, int32_t* __restrict__ dev_err,
    CommitArgs cm) {
  __shared__ int par[TV_MAX_NODES];
  __shared__ int s_path[TV_MAX_NODES];
  __shared__ int s_prefix, s_ok;
  __shared__ int amax[TV_MAX_NODES];
  __shared__ int link[TV_MAX_NODES];  // node j: its parent (low 16 bits), its edge accepted (bit 16)
  __shared__ int bad;
  __shared__ unsigned red[kThreads / kWave];

  const int b = blockIdx.x;
  // With several layers, one workgroup per (sequence, layer): each walks the
  // (small) tree itself and copies its own layer's rows; layer 0 writes the
  // acceptance outputs, the new prefix length and the error bits.
  const bool lead = blockIdx.y == 0;
  const int i = threadIdx.x;
  if (i == 0) bad = 0;
  __syncthreads();
  int p_commit = 0;  // the commit's prefix length, loaded with the partials
  int my_par = -1, my_tok = 0;
  if (i < n) {
    const int64_t row = (int64_t)b * n + i;
    const int p = parents[row];
    my_par = p;
    my_tok = draft[row];
    if (i == 0 && cm.k_cache) p_commit = cm.prefix_len[b];
    // chunk partials in groups of 8, all loads of a group in flight at once
    float bv = -INFINITY;
    int bi = INT32_MAX;
    for (int c0 = 0; c0 < chunks; c0 += 8) {
      float v[8];
      int k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = c0 + u < chunks;
        v[u] = in ? part_v[row * chunks + c0 + u] : -INFINITY;
        k[u] = in ? part_i[row * chunks + c0 + u] : INT32_MAX;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (better(v[u], k[u], bv, bi)) {
          bv = v[u];
          bi = k[u];
        }
    }
    amax[i] = bi;
    if (lead) target_argmax[row] = bi;
    par[i] = p;
    const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
    if (!ok) bad = 1;
  }
  __syncthreads();

  // Each edge is tested once (node i's token against its parent's argmax)
  // and its result packed with the parent index, so that the up-walks below
  // take one LDS read per level.
  const bool edge = i < n && (i == 0 || (!bad && my_tok == amax[my_par]));
  if (i < n && !bad) link[i] = (i == 0 ? 0 : my_par) | ((int)edge << 16);
  __syncthreads();
  // key = depth << 16 | (0xFFFF - i) for accepted nodes, 0 otherwise; the
  // root is always accepted so the maximum is never 0.  A node is accepted
  // when every edge on its root path is; the walk stops at the first
  // rejected one (parents precede children, so it always ends).
  unsigned key = 0;
  if (i < n) {
    if (bad) {
      key = (i == 0) ? 0xFFFFu : 0u;
    } else {
      bool acc = edge;
      int d = i > 0 ? 1 : 0;
      int j = i > 0 ? my_par : 0;
      while (acc && j > 0) {
        const int w = link[j];
        acc = (w >> 16) != 0;
        j = w & 0xFFFF;
        ++d;
      }
      if (acc) key = ((unsigned)d << 16) | (unsigned)(0xFFFF - i);
    }
  }
  key = wave_max_u(key);
  if ((i & (kWave - 1)) == 0) red[i / kWave] = key;
  __syncthreads();
  unsigned best = red[0];
  for (int w = 1; w < kThreads / kWave; ++w) best = red[w] > best ? red[w] : best;
  const int end_node = 0xFFFF - (int)(best & 0xFFFFu);
  const int depth = (int)(best >> 16);

  int32_t* path = accept_path + (int64_t)b * n;
  if (lead && i < n && i > depth) path[i] = -1;
  int32_t* const err_out = lead ? dev_err : nullptr;
  if (i == 0) {
    int j = end_node;
    for (int k = depth; k >= 0; --k) {
      if (lead) path[k] = j;
      s_path[k] = j;
      j = par[j];
    }
    if (lead) {
      accept_len[b] = depth;
      bonus[b] = amax[end_node];
    }
    if (bad) raise_err(err_out, TV_DERR_BAD_PARENT);
    if (cm.k_cache) {
      // the commit's checks (tv_commit_kv): the path is valid by construction
      const int p = p_commit;
      int ok = 1;
      if (p < 0 || p > cm.cap) {
        raise_err(err_out, TV_DERR_BAD_PREFIX);
        ok = 0;
      } else if ((int64_t)p + depth + 1 > cm.cap) {
        raise_err(err_out, TV_DERR_CAPACITY);
        ok = 0;
      }
      s_prefix = p;
      s_ok = ok;
    }
  }
  if (!cm.k_cache) return;
  __syncthreads();
  // copy the accepted nodes' K/V rows into the cache, 16 bytes per item
  const int p = s_prefix;
  if (s_ok) {
    const int per_row = cm.vec_per_row, hkv = cm.hkv;
    const int items = (depth + 1) * hkv * per_row;
    const int64_t lt = blockIdx.y * cm.tree_layer_vec, lc = blockIdx.y * cm.cache_layer_vec;
    const uint4* __restrict__ kt = cm.k_tree + lt + (int64_t)b * n * hkv * per_row;
    const uint4* __restrict__ vt = cm.v_tree + lt + (int64_t)b * n * hkv * per_row;
    uint4* __restrict__ kc = cm.k_cache + lc + b * cm.seq_stride_vec;
    uint4* __restrict__ vc = cm.v_cache + lc + b * cm.seq_stride_vec;
#pragma unroll 4
    for (int it = i; it < items; it += kThreads) {
      const int c = it % per_row, rh = it / per_row;
      const int h = rh % hkv, r = rh / hkv;
      const int64_t src = ((int64_t)s_path[r] * hkv + h) * per_row + c;
      const int64_t dst = ((int64_t)h * cm.cap + p + r) * per_row + c;
      kc[dst] = kt[src];
      vc[dst] = vt[src];
    }
  }
  if (i == 0 && lead) cm.new_prefix_len[b] = s_ok ? p + depth + 1 : p;
}

}  // namespace

AcceptPlan plan_accept(int batch, int n, int64_t vocab) {
  AcceptPlan p;
  // ~32 KB of bf16 per workgroup: enough bytes in flight per CU without
  // starving rows with few chunks.
  const int64_t per_pass = (int64_t)kThreads * 8;
  int64_t chunk = per_pass * kUnroll;
  if (chunk > vocab) chunk = ((vocab + per_pass - 1) / per_pass) * per_pass;
  if (chunk < per_pass) chunk = per_pass;
  p.chunk_len = chunk;
  p.chunks = (int)((vocab + chunk - 1) / chunk);
  const size_t rows = (size_t)batch * n;
  p.ws_bytes = rows * p.chunks * (sizeof(float) + sizeof(int)) + 256;
  return p;
}

hipError_t launch_accept(const void* logits, tv_dtype dt, int64_t vocab, int64_t row_stride,
                         const int32_t* parents, const int32_t* draft, int batch, int n,
                         int32_t* target_argmax, int32_t* accept_len, int32_t* accept_path,
                         int32_t* bonus, void* workspace, const AcceptPlan& plan,
                         int32_t* dev_err, hipStream_t stream, const CommitTarget* commit) {
  const size_t rows = (size_t)batch * n;
  float* part_v = reinterpret_cast<float*>(workspace);
  int* part_i = reinterpret_cast<int*>(
      reinterpret_cast<char*>(workspace) + ((rows * plan.chunks * sizeof(float) + 255) / 256) * 256);
  const dim3 grid(plan.chunks, (unsigned)rows);
  const uintptr_t addr = reinterpret_cast<uintptr_t>(logits);
  if (dt == TV_BF16) {
    const bool vec = (addr % 16 == 0) && (row_stride % 8 == 0);
    if (vec)
      hipLaunchKernelGGL((vocab_argmax_kernel<bf16, true>), grid, dim3(kThreads), 0, stream,
                         (const bf16*)logits, vocab, row_stride, plan.chunk_len, plan.chunks,
                         part_v, part_i);
    else
      hipLaunchKernelGGL((vocab_argmax_kernel<bf16, false>), grid, dim3(kThreads), 0, stream,
                         (const bf16*)logits, vocab, row_stride, plan.chunk_len, plan.chunks,
                         part_v, part_i);
  } else {
    const bool vec = (addr % 16 == 0) && (row_stride % 4 == 0);
    if (vec)
      hipLaunchKernelGGL((vocab_argmax_kernel<float, true>), grid, dim3(kThreads), 0, stream,
                         (const float*)logits, vocab, row_stride, plan.chunk_len, plan.chunks,
                         part_v, part_i);
    else
      hipLaunchKernelGGL((vocab_argmax_kernel<float, false>), grid, dim3(kThreads), 0, stream,
                         (const float*)logits, vocab, row_stride, plan.chunk_len, plan.chunks,
                         part_v, part_i);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CommitArgs cm{};
  int layers = 1;
  if (commit) {
    layers = commit->layers;
    cm.tree_layer_vec = commit->tree_layer_stride / 8;
    cm.cache_layer_vec = commit->cache_layer_stride / 8;
    cm.k_tree = (const uint4*)commit->k_tree;
    cm.v_tree = (const uint4*)commit->v_tree;
    cm.prefix_len = commit->prefix_len;
    cm.new_prefix_len = commit->new_prefix_len;
    cm.k_cache = (uint4*)commit->k_cache;
    cm.v_cache = (uint4*)commit->v_cache;
    cm.seq_stride_vec = commit->seq_stride / 8;
    cm.cap = commit->cap;
    cm.hkv = commit->hkv;
    cm.vec_per_row = commit->d / 8;
  }
  hipLaunchKernelGGL(path_walk_kernel, dim3(batch, layers), dim3(kThreads), 0, stream, part_v, part_i,
                     plan.chunks, parents, draft, n, target_argmax, accept_len, accept_path, bonus,
                     dev_err, cm);
  return hipGetLastError();
}

}  // namespace tv
