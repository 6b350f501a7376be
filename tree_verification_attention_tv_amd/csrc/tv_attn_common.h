// Definitions shared by the tree-attention kernels (tv_attention.hip: the
// 16-row split kernel and the combine; tv_attn_wide.hip: the 32-row kernel).
#pragma once

#include "tv_device.h"

#include <math.h>

namespace tv {
namespace attn {

constexpr int kTile = 32;        // tokens per KV tile
constexpr int kMinChunk = 128;   // minimum prefix slots per split
constexpr float kSumMax = 1.2676506e30f;  // 2^100: largest accepted row sum

typedef short i16x4 __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const bf16* q;
  const bf16* k_tree;
  const bf16* v_tree;
  const bf16* k_cache;
  const bf16* v_cache;
  const int32_t* prefix_len;
  const uint32_t* mask;      // null: built from `parents` by the tree workgroups
  const int32_t* parents;    // [batch][n] when mask is null
  uint32_t* mask_out;        // optional outputs of the in-kernel build (as tv_build_tree_mask)
  int32_t* depth_out;
  const int32_t* block_idx;
  const int32_t* n_blocks;
  bf16* part_o;     // [batch][nparts][hkv][rows][D], normalised by the row's own sum
  float2* part_ml;  // [batch][nparts][hkv][rows]: (reference max, row sum)
  int32_t* dev_err;
  bf16* out;
  float* lse;
  int64_t seq_stride;
  int batch, n, hq, hkv, grp, cap, words;
  int block_size, block_shift, max_blocks, max_prefix;  // block_shift < 0: not a power of 2
  int chunk, splits, row_groups, rows;
  int tree_sep, nparts;  // tree in its own workgroup (split index `splits`); partials per sequence
  float c;  // softmax scale * log2(e)
  // In-launch combine (32-row kernel): the workgroups past the nsplit_wg
  // split workgroups merge the partials, ncw_unit per (sequence, kv head),
  // rpw rows per wave.  sync[u] counts the split workgroups of unit u that
  // have written their partials, sync[batch * hkv + u] the finished merges.
  int* sync;
  int nsplit_wg, ncw_unit, rpw;
};

// Verified-prefix length of sequence b, clamped to what the grid covers.
// A workgroup-uniform int32 read through the scalar cache (constant address
// space): its wait is on lgkmcnt, so it never drains the tile requests in
// flight, which the vector-memory counter also counts.  The arrays read
// this way (prefix lengths, list lengths) are not written by the kernel.
__device__ __forceinline__ int load_uniform(const int32_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ int clamped_prefix(const AttnArgs& a, int b, int* err) {
  int p = load_uniform(a.prefix_len + b);
  const int lim = a.max_blocks ? a.cap : min(a.cap, a.max_prefix);
  if (p < 0 || p > lim) {
    *err |= TV_DERR_BAD_PREFIX;
    p = p < 0 ? 0 : lim;
  }
  return p;
}

// Number of prefix slots of sequence b: prefix rows in full mode, listed
// blocks times block size in partial mode.
__device__ __forceinline__ int prefix_slots(const AttnArgs& a, int b, int p, int* err) {
  if (a.max_blocks == 0) return p;
  int nb = load_uniform(a.n_blocks + b);
  if (nb < 0 || nb > a.max_blocks) {
    *err |= TV_DERR_BAD_BLOCK;
    nb = nb < 0 ? 0 : a.max_blocks;
  }
  return nb * a.block_size;
}


// Workgroup barrier for LDS hand-off only.  __syncthreads() would also wait
// for every outstanding global load of the wave (vmcnt(0)), which would
// drain the tile prefetches the pipeline keeps in flight across barriers.
// Here each wave only waits for its own LDS accesses (lgkmcnt(0)); the
// signal fences keep the compiler from moving memory operations across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: lgkmcnt(0), vmcnt/expcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap permutes: after swapping, the two results of each
// swap hold the value of a lane and of its partner.
__device__ __forceinline__ float xsum16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float xmax16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---- LDS DMA -----------------------------------------------------------------
// global_load_lds_dwordx4: each lane loads 16 bytes from its own address and
// the wave's 64 results land contiguously in LDS at M0 (lane i at M0 + 16 i).
// Issued through inline asm so that the compiler neither reorders it nor
// inserts its own (conservative) waits; completion is tracked by hand with
// vmcnt, which counts these loads like any other vector-memory load.
__device__ __forceinline__ void dma16(uint32_t lds_addr, const void* gptr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_addr), "v"(gptr)
               : "memory");
}

// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
__device__ __forceinline__ void dma16s(uint32_t lds_addr, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

constexpr int kRing = 4;        // LDS ring slots (tiles)
constexpr int kBlkCache = 1024; // block ids of one split staged in LDS

__device__ __forceinline__ float xmax_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xsum_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Partial stores and loads.  COH = true: device-coherent 8-byte accesses
// (agent-scope relaxed atomics, which bypass the non-coherent cache levels),
// for partials that are merged inside the launch that writes them: a writer
// then needs only its stores to have completed (s_waitcnt vmcnt(0)) before
// it signals, instead of a write-back of its whole L2.
typedef unsigned long long u64;
template <bool COH>
__device__ __forceinline__ void store_ml(float2* p, float2 v) {
  if constexpr (COH)
    __hip_atomic_store(reinterpret_cast<u64*>(p), __builtin_bit_cast(u64, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool COH>
__device__ __forceinline__ float2 load_ml(const float2* p) {
  if constexpr (COH)
    return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<const u64*>(p), __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT));
  else
    return *p;
}
typedef u64 u64x2 __attribute__((ext_vector_type(2)));
template <bool COH>
__device__ __forceinline__ void store_o(bf16* p, bf16x8 v) {
  if constexpr (COH) {
    const u64x2 w = __builtin_bit_cast(u64x2, v);
    __hip_atomic_store(reinterpret_cast<u64*>(p), w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<u64*>(p) + 1, w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *reinterpret_cast<bf16x8*>(p) = v;
  }
}
template <bool COH>
__device__ __forceinline__ bf16x8 load_o(const bf16* p) {
  if constexpr (COH) {
    u64x2 w;
    w[0] = __hip_atomic_load(reinterpret_cast<const u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[1] = __hip_atomic_load(reinterpret_cast<const u64*>(p) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_bit_cast(bf16x8, w);
  } else {
    return *reinterpret_cast<const bf16x8*>(p);
  }
}

// Partial stores of the split work: device-coherent when the merge runs in
// the same launch (sync set), plain otherwise -- coherent stores also write
// through to memory, which doubles the partials' HBM write traffic
// (measured with WRITE_SIZE).
__device__ __forceinline__ void store_part_ml(const AttnArgs& a, float2* p, float2 v) {
  if (a.sync) store_ml<true>(p, v);
  else store_ml<false>(p, v);
}
__device__ __forceinline__ void store_part_o(const AttnArgs& a, bf16* p, bf16x8 v) {
  if (a.sync) store_o<true>(p, v);
  else store_o<false>(p, v);
}

// Merge the split partials of NR (sequence, node, head) rows -- rowid =
// (b * n + i) * hq + h, negative for none -- by the wave of `lane`: with
// weights w_s = 2^(m_s - m) l_s, m = max m_s, the output is
// sum w_s o_s / sum w_s (o_s already divided by l_s) and the log-sum-exp is
// m + log2(sum w_s), in natural-log units.  Lane t C + c (C = D/8 chunks of
// 8 elements, T = 64/C) folds the partials k = t, t+T, ... for elements
// 8c..8c+7 into a running (max, sum, output), U partials per row with their
// loads in flight together (the rows' loads too), and the T running states
// are merged across lanes in a fixed order.
template <int D, int NR, bool COH>
__device__ __forceinline__ void combine_rows(const AttnArgs& a, const int64_t (&rowid)[NR], int lane) {
  constexpr int C = D / 8;
  constexpr int T = 64 / C;
  constexpr int U = 8 / NR;  // 8 partial loads in flight per lane
  const int c = lane % C;
  const int t = lane / C;
  // Every split writes a partial for every row (an empty one, m = -inf,
  // where it sees no key), so all of them are merged and the prefix length
  // is not needed here: the partial loads are the only memory round trip.
  const int cnt = a.nparts;
  const int64_t stride = (int64_t)a.hkv * a.rows;  // partial rows between splits
  int64_t p0[NR];
  float mx[NR], l[NR], acc[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    // 32-bit index arithmetic (the row count fits; 64-bit divisions are
    // long instruction sequences in front of the loads)
    const uint32_t id = rowid[r] < 0 ? 0u : (uint32_t)rowid[r];
    const uint32_t bi = id / (uint32_t)a.hq;
    const int h = (int)(id - bi * (uint32_t)a.hq);
    const uint32_t bq = bi / (uint32_t)a.n;
    const int i = (int)(bi - bq * (uint32_t)a.n);
    const int b = (int)bq;
    const int g = h / a.grp;
    p0[r] = ((int64_t)b * a.nparts * a.hkv + g) * a.rows + i * a.grp + h % a.grp;
    mx[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }
  for (int k0 = t; k0 < cnt; k0 += T * U) {
    float2 ml[NR][U];
    bf16x8 ov[NR][U];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * T;
        if (k < cnt && rowid[r] >= 0) {
          const int64_t pi = p0[r] + k * stride;
          ml[r][u] = load_ml<COH>(a.part_ml + pi);
          ov[r][u] = load_o<COH>(a.part_o + pi * D + 8 * c);
        } else {
          ml[r][u] = make_float2(-INFINITY, 0.f);
          ov[r][u] = bf16x8{};
        }
      }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float mb = mx[r];
#pragma unroll
      for (int u = 0; u < U; ++u) mb = fmaxf(mb, ml[r][u].x);
      if (mb == -INFINITY) continue;
      const float sc = mx[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx[r] - mb);
      l[r] *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // an empty partial (m = -inf) weighs 0 and its output is not read
        const float w = ml[r][u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[r][u].x - mb) * ml[r][u].y;
        l[r] += w;
        if (w != 0.f) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] = __builtin_fmaf(w, (float)ov[r][u][e], acc[r][e]);
        }
      }
      mx[r] = mb;
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    // merge the T states of a chunk (lanes c, c + C, ...)
#pragma unroll
    for (int off = C; off < 64; off <<= 1) {
      const float mo = __shfl_xor(mx[r], off);
      const float lo = __shfl_xor(l[r], off);
      float ao[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ao[e] = __shfl_xor(acc[r][e], off);
      const float mn = fmaxf(mx[r], mo);
      if (mn != -INFINITY) {
        const float r0 = mx[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx[r] - mn);
        const float r1 = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
        l[r] = l[r] * r0 + lo * r1;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = acc[r][e] * r0 + ao[e] * r1;
      }
      mx[r] = mn;
    }
    if (t != 0 || rowid[r] < 0) continue;
    bf16x8 res;
    float lse_v;
    if (mx[r] == -INFINITY) {
      res = bf16x8{};
      lse_v = -INFINITY;
    } else {
      const float inv = 1.f / l[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = (bf16)(acc[r][e] * inv);
      lse_v = (mx[r] + log2f(l[r])) * 0.69314718055994530942f;
    }
    *reinterpret_cast<bf16x8*>(a.out + rowid[r] * D + 8 * c) = res;
    if (c == 0 && a.lse) a.lse[rowid[r]] = lse_v;
  }
}

// ---- merge inside the launch ------------------------------------------------
// The grid of a schedule holds nsplit_wg split workgroups, then ncw_unit
// merge workgroups per (sequence, kv head) unit u = b * hkv + g.  A split
// workgroup, once its partials are stored, adds 1 to sync[u]; the merge
// workgroups of u wait until sync[u] counts all nparts * row_groups of them,
// merge NW * rpw rows each, and count themselves in sync[batch * hkv + u];
// the last one resets both counters to zero for the next call.  Merge
// workgroups follow every split workgroup in dispatch order, so their wait
// depends only on workgroups already running or done; it is bounded all the
// same (TV_DERR_SYNC past the bound).
constexpr unsigned kSpinLimit = 1u << 22;  // polls of the merge wait, s_sleep 2 apart

template <int D, int NW>
__device__ __forceinline__ void merge_role(const AttnArgs& a, int j) {
  const int units_bg = a.batch * a.hkv;
  const int u = j % units_bg;
  const int slice = j / units_bg;
  const int mb = u / a.hkv, mg = u % a.hkv;
  if (threadIdx.x == 0) {
    const int target = a.nparts * a.row_groups;
    // The partials are read with device-coherent loads after the barrier
    // below, so relaxed polls suffice (an acquire would also invalidate
    // this XCD's L2 under the split workgroups still streaming).
    int v = __hip_atomic_load(&a.sync[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (unsigned it = 0; v < target && it < kSpinLimit; ++it) {
      __builtin_amdgcn_s_sleep(2);
      v = __hip_atomic_load(&a.sync[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (v < target) raise_err(a.dev_err, TV_DERR_SYNC);
  }
  __syncthreads();
  const int wv = threadIdx.x >> 6;
  const int r0 = (slice * NW + wv) * a.rpw;  // first row of this wave: node * grp + head in group
  auto rowid_of = [&](int r) -> int64_t {
    if (r >= a.rows || r >= r0 + a.rpw) return -1;
    const int i = r / a.grp;
    return ((int64_t)mb * a.n + i) * a.hq + mg * a.grp + (r - i * a.grp);
  };
  for (int q = 0; q < a.rpw; q += 2) {
    const int64_t ids[2] = {rowid_of(r0 + q), rowid_of(r0 + q + 1)};
    combine_rows<D, 2, true>(a, ids, threadIdx.x & 63);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(&a.sync[units_bg + u], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == a.ncw_unit - 1) {
      __hip_atomic_store(&a.sync[u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.sync[units_bg + u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// A split workgroup of unit u has stored its partials.  They went out as
// device-coherent stores: once they have completed (vmcnt 0 in every wave,
// then the barrier) the merge's coherent loads see them on any XCD.  A
// release fence would instead write back this XCD's whole L2, which
// stretches the tail of the split workgroups still running by tens of
// microseconds (measured at the 60000-token prefix).
__device__ __forceinline__ void split_done(const AttnArgs& a, int u) {
  vm_wait<0>();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(&a.sync[u], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// launch of the 32-row kernel (tv_attn_wide.hip): grid of (splits + tree_sep)
// * batch * kv heads * row groups workgroups, `rt` 32-row tiles per wave
hipError_t launch_wide(const AttnArgs& a, int head_dim, int rt, unsigned grid, hipStream_t stream);

}  // namespace attn
}  // namespace tv
