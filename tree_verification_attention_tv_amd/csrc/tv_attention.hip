// Tree-masked GQA attention for the verify forward of a draft tree.
//
// Sources: SpecBlock App. A.2 (a node sees the verified prefix, its on-path
// ancestors and itself); SpecPV Sec. 3.2 (a selected subset of KV blocks is
// attended as one continuous segment); "Dynamic Speculative Decoding",
// Roofline analysis (decode attention is bandwidth-bound; a tree of N
// proposed tokens multiplies the arithmetic intensity by N).
//
// Design (gfx950):
//  * One workgroup (4 waves) per (sequence, kv head, row group, split).  It
//    holds every query row of its kv head -- n_nodes x group rows -- so each
//    K/V tile is read from HBM once and reused by all rows (AI = rows
//    FLOP/byte).  Each wave owns RB blocks of 16 rows.
//  * The prefix (full rows, or the listed blocks) is cut into `splits`
//    contiguous ranges; the tree block is one more split whose tiles are
//    masked with the packed ancestor bits.  A combine kernel merges the
//    (max, sum, unnormalised output) partials in fixed order.
//  * K/V tiles of 32 tokens are staged in LDS (double buffered, padded rows
//    against bank conflicts).  S^T = K Q^T and O^T += V^T P^T run on
//    v_mfma_f32_16x16x32_bf16: the S^T accumulator layout puts one query row
//    per lane column, so the softmax row statistics are mostly in-register
//    and need two cross-lane steps; P^T is re-packed to bf16 straight from
//    the accumulator registers as the B operand of the PV product.
//  * Online softmax in fp32 in the log2 domain (scale * log2 e folded into
//    one FMA before v_exp_f32); masked scores are -inf; rescaling of the
//    output accumulators is skipped when no row maximum moved.
#include "tv_internal.h"

#include <math.h>

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;        // tokens per KV tile
constexpr int kMinChunk = 64;    // minimum prefix slots per split

struct AttnArgs {
  const bf16* q;
  const bf16* k_tree;
  const bf16* v_tree;
  const bf16* k_cache;
  const bf16* v_cache;
  const int32_t* prefix_len;
  const uint32_t* mask;
  const int32_t* block_idx;
  const int32_t* n_blocks;
  float* part_o;
  float2* part_ml;
  int32_t* dev_err;
  bf16* out;
  float* lse;
  int64_t seq_stride;
  int batch, n, hq, hkv, grp, cap, words;
  int block_size, max_blocks, max_prefix;
  int chunk, splits, row_groups, rows;
  float c;  // softmax scale * log2(e)
};

// Verified-prefix length of sequence b, clamped to what the grid covers.
__device__ __forceinline__ int clamped_prefix(const AttnArgs& a, int b, int* err) {
  int p = a.prefix_len[b];
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
  int nb = a.n_blocks[b];
  if (nb < 0 || nb > a.max_blocks) {
    *err |= TV_DERR_BAD_BLOCK;
    nb = nb < 0 ? 0 : a.max_blocks;
  }
  return nb * a.block_size;
}

// Cache row behind prefix slot u (< slots), or -1 when the slot is empty
// (past the prefix, or in an invalid / clipped block).
__device__ __forceinline__ int slot_row(const AttnArgs& a, int b, int p, int u, int* err) {
  if (a.max_blocks == 0) return u < p ? u : -1;
  const int blk = a.block_idx[(int64_t)b * a.max_blocks + u / a.block_size];
  if (blk < 0 || (int64_t)blk * a.block_size >= p) {
    *err |= TV_DERR_BAD_BLOCK;
    return -1;
  }
  const int row = blk * a.block_size + u % a.block_size;
  return row < p ? row : -1;
}

__device__ __forceinline__ float wave_max_cols(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_cols(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int D, int RB>
__global__ __launch_bounds__(kThreads, 1) void attn_split_kernel(AttnArgs a) {
  constexpr int DC = D / 32;               // k-steps of the QK^T product
  constexpr int DB = D / 16;               // 16-wide output blocks of PV
  constexpr int KSTR = D + 8;              // LDS row stride (elements), K
  constexpr int VSTR = D + 16;             // LDS row stride (elements), V
  constexpr int VPR = D / 8;               // 16-byte vectors per row
  constexpr int LOADS = kTile * VPR / kThreads;
  static_assert(LOADS >= 1 && kTile * VPR % kThreads == 0, "tile / thread mismatch");

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][kTile * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][kTile * VSTR];
  __shared__ uint32_t svalid[2];

  const int s = blockIdx.x;
  const int g = blockIdx.y / a.row_groups;
  const int rg = blockIdx.y % a.row_groups;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;   // MFMA column (query row within a block)
  const int grp4 = lane >> 4;  // lane group 0..3
  const bool tree = (s == a.splits);

  int err = 0;
  const int p_len = clamped_prefix(a, b, &err);
  const int slots = prefix_slots(a, b, p_len, &err);
  int begin, end;
  if (tree) {
    begin = 0;
    end = a.n;
  } else {
    begin = s * a.chunk;
    end = min(begin + a.chunk, slots);
  }
  if (err && s == 0 && g == 0 && rg == 0 && tid == 0) raise_err(a.dev_err, err);
  err = 0;
  if (begin >= end) return;  // uniform over the workgroup

  const int row0 = rg * (64 * RB) + wave * (16 * RB);
  const bool active = row0 < a.rows;

  // Q^T fragments (B operand of S^T = K Q^T): column = query row, 8 d per lane
  bf16x8 qf[RB][DC];
#pragma unroll
  for (int mb = 0; mb < RB; ++mb) {
    const int m = row0 + 16 * mb + col;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (m < a.rows) {
        const int i = m / a.grp;
        const int h = g * a.grp + m % a.grp;
        qf[mb][dc] = *reinterpret_cast<const bf16x8*>(
            a.q + (((int64_t)b * a.n + i) * a.hq + h) * D + 32 * dc + 8 * grp4);
      } else {
        qf[mb][dc] = bf16x8{};
      }
    }
  }

  f32x4 o[RB][DB];
  float mrun[RB], lrun[RB];
#pragma unroll
  for (int mb = 0; mb < RB; ++mb) {
    mrun[mb] = -INFINITY;
    lrun[mb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[mb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const bf16* kbase;
  const bf16* vbase;
  int64_t row_elems;  // elements between consecutive tokens in the source
  if (tree) {
    kbase = a.k_tree + ((int64_t)b * a.n * a.hkv + g) * D;
    vbase = a.v_tree + ((int64_t)b * a.n * a.hkv + g) * D;
    row_elems = (int64_t)a.hkv * D;
  } else {
    kbase = a.k_cache + b * a.seq_stride + (int64_t)g * a.cap * D;
    vbase = a.v_cache + b * a.seq_stride + (int64_t)g * a.cap * D;
    row_elems = D;
  }

  uint4 kreg[LOADS], vreg[LOADS];
  uint32_t vbits_next = 0;

  auto token_row = [&](int u) -> int {  // source row of slot/token u, -1 if empty
    if (u >= end) return -1;
    return tree ? u : slot_row(a, b, p_len, u, &err);
  };

  auto load_tile = [&](int t0) {
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const int idx = tid + ld * kThreads;
      const int r = idx / VPR;
      const int cv = idx % VPR;
      const int row = token_row(t0 + r);
      if (row >= 0) {
        kreg[ld] = *reinterpret_cast<const uint4*>(kbase + row * row_elems + cv * 8);
        vreg[ld] = *reinterpret_cast<const uint4*>(vbase + row * row_elems + cv * 8);
      } else {
        kreg[ld] = uint4{0u, 0u, 0u, 0u};
        vreg[ld] = uint4{0u, 0u, 0u, 0u};
      }
    }
    const bool v = lane < kTile && token_row(t0 + lane) >= 0;
    vbits_next = (uint32_t)__ballot(v);
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const int idx = tid + ld * kThreads;
      const int r = idx / VPR;
      const int cv = idx % VPR;
      *reinterpret_cast<uint4*>(&Ks[buf][r * KSTR + cv * 8]) = kreg[ld];
      *reinterpret_cast<uint4*>(&Vs[buf][r * VSTR + cv * 8]) = vreg[ld];
    }
    if (tid == 0) svalid[buf] = vbits_next;
  };

  const int ntiles = (end - begin + kTile - 1) / kTile;
  load_tile(begin);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int t0 = begin + it * kTile;
    if (it + 1 < ntiles) load_tile(t0 + kTile);

    if (active) {
      // ---- S^T = K Q^T for 32 tokens x RB*16 rows -------------------------
      f32x4 sacc[2][RB];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int mb = 0; mb < RB; ++mb) sacc[tb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              &Ks[buf][(tb * 16 + col) * KSTR + 32 * dc + 8 * grp4]);
#pragma unroll
          for (int mb = 0; mb < RB; ++mb)
            sacc[tb][mb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[mb][dc], sacc[tb][mb], 0, 0, 0);
        }
      }

      // ---- masking --------------------------------------------------------
      const uint32_t vbits = svalid[buf];
      if (tree || vbits != 0xFFFFFFFFu) {
#pragma unroll
        for (int mb = 0; mb < RB; ++mb) {
          uint32_t allow = vbits;
          if (tree) {
            const int m = row0 + 16 * mb + col;
            const uint32_t w =
                m < a.rows ? a.mask[((int64_t)b * a.n + m / a.grp) * a.words + t0 / kTile] : 0u;
            allow &= w;
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = tb * 16 + 4 * grp4 + r;
              if (!((allow >> t) & 1u)) sacc[tb][mb][r] = -INFINITY;
            }
        }
      }

      // ---- online softmax, P^T packed to bf16 -----------------------------
      bf16x8 pb[RB];
#pragma unroll
      for (int mb = 0; mb < RB; ++mb) {
        float mx = sacc[0][mb][0];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[tb][mb][r]);
        mx = wave_max_cols(mx);
        const float mnew = fmaxf(mrun[mb], mx * a.c);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrun[mb] - muse);
        float psum = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tb][mb][r], a.c, -muse));
            psum += pv;
            pb[mb][tb * 4 + r] = (bf16)pv;
          }
        lrun[mb] = lrun[mb] * alpha + psum;
        mrun[mb] = mnew;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) o[mb][db] *= alpha;
        }
      }

      // ---- O^T += V^T P^T ---------------------------------------------------
      // k-slot j of lane group q holds token 4q+j (j<4) or 16+4q+(j-4): the
      // tokens this lane already owns in the S^T accumulators.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16* vcol = &Vs[buf][16 * db + col];
        bf16x8 vf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vf[j] = vcol[(4 * grp4 + j) * VSTR];
          vf[4 + j] = vcol[(16 + 4 * grp4 + j) * VSTR];
        }
#pragma unroll
        for (int mb = 0; mb < RB; ++mb)
          o[mb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[mb], o[mb][db], 0, 0, 0);
      }
    }

    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }
  if (err) raise_err(a.dev_err, err);

  if (!active) return;
#pragma unroll
  for (int mb = 0; mb < RB; ++mb) {
    const float l = wave_sum_cols(lrun[mb]);
    const int m = row0 + 16 * mb + col;
    if (m < a.rows) {
      const int i = m / a.grp;
      const int h = g * a.grp + m % a.grp;
      const int64_t pi = (((int64_t)b * (a.splits + 1) + s) * a.n + i) * a.hq + h;
      float* dst = a.part_o + pi * D + 4 * grp4;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = o[mb][db];
      if (grp4 == 0) a.part_ml[pi] = make_float2(mrun[mb], l);
    }
  }
}

// Merge the split partials of one (sequence, node, head): m = max m_s,
// l = sum 2^(m_s - m) l_s, o = sum 2^(m_s - m) o_s / l.  Fixed split order.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnArgs a) {
  constexpr int Q4 = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)a.batch * a.n * a.hq * Q4;
  if (gid >= total) return;
  const int dq = (int)(gid % Q4);
  const int64_t rowid = gid / Q4;  // (b * n + i) * hq + h
  const int h = (int)(rowid % a.hq);
  const int64_t bi = rowid / a.hq;
  const int i = (int)(bi % a.n);
  const int b = (int)(bi / a.n);

  int err = 0;
  const int p_len = clamped_prefix(a, b, &err);
  const int slots = prefix_slots(a, b, p_len, &err);
  const int ns = (slots + a.chunk - 1) / a.chunk;
  const int64_t base = (int64_t)b * (a.splits + 1);
  auto pidx = [&](int s) { return ((base + s) * a.n + i) * a.hq + h; };

  float m = a.part_ml[pidx(a.splits)].x;
  for (int s = 0; s < ns; ++s) m = fmaxf(m, a.part_ml[pidx(s)].x);

  bf16x4 res;
  float lse_v;
  if (m == -INFINITY) {
    res = bf16x4{};
    lse_v = -INFINITY;
  } else {
    float l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s <= ns; ++s) {
      const int ss = (s == ns) ? a.splits : s;
      const int64_t pi = pidx(ss);
      const float2 ml = a.part_ml[pi];
      const float w = __builtin_amdgcn_exp2f(ml.x - m);
      l += w * ml.y;
      const f32x4 ov = *reinterpret_cast<const f32x4*>(a.part_o + pi * D + 4 * dq);
      acc += w * ov;
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = (bf16)(acc[e] * inv);
    lse_v = (m + log2f(l)) * 0.69314718055994530942f;
  }
  *reinterpret_cast<bf16x4*>(a.out + rowid * D + 4 * dq) = res;
  if (dq == 0 && a.lse) a.lse[rowid] = lse_v;
}

template <int D, int RB>
void launch_split(const AttnArgs& args, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_split_kernel<D, RB>), grid, dim3(kThreads), 0, stream, args);
}

template <int D>
void launch_split_rb(int rb, const AttnArgs& args, dim3 grid, hipStream_t stream) {
  switch (rb) {
    case 1: launch_split<D, 1>(args, grid, stream); break;
    case 2: launch_split<D, 2>(args, grid, stream); break;
    case 3: launch_split<D, 3>(args, grid, stream); break;
    default: launch_split<D, 4>(args, grid, stream); break;
  }
}

}  // namespace

AttnPlan plan_attention(const tv_attn_desc& d, int cu_count) {
  AttnPlan p{};
  const int grp = d.n_q_heads / d.n_kv_heads;
  p.rows = d.n_nodes * grp;
  p.row_groups = (p.rows + 255) / 256;
  const int per_group = (p.rows + p.row_groups - 1) / p.row_groups;
  p.row_blocks = (per_group + 63) / 64;
  if (p.row_blocks < 1) p.row_blocks = 1;
  p.prefix_slots = d.max_blocks ? d.max_blocks * d.block_size : d.max_prefix_len;
  const int units = d.batch * d.n_kv_heads * p.row_groups;
  int splits;
  if (d.num_splits > 0) {
    splits = d.num_splits;
  } else {
    splits = (cu_count + units - 1) / units;
    const int cap = (p.prefix_slots + kMinChunk - 1) / kMinChunk;
    if (splits > cap) splits = cap;
    if (splits < 1) splits = 1;
  }
  int chunk = p.prefix_slots > 0 ? (p.prefix_slots + splits - 1) / splits : kTile;
  chunk = ((chunk + kTile - 1) / kTile) * kTile;
  p.chunk = chunk;
  p.splits = p.prefix_slots > 0 ? (p.prefix_slots + chunk - 1) / chunk : 1;
  const size_t parts = (size_t)d.batch * (p.splits + 1) * d.n_nodes * d.n_q_heads;
  p.ws_o_bytes = ((parts * d.head_dim * sizeof(float) + 255) / 256) * 256;
  p.ws_ml_bytes = ((parts * sizeof(float2) + 255) / 256) * 256;
  return p;
}

hipError_t launch_attention(const tv_attn_desc& d, const AttnPlan& plan, const tv_attn_ptrs& p,
                            void* workspace, int32_t* dev_err, hipStream_t stream) {
  AttnArgs a{};
  a.q = (const bf16*)p.q;
  a.k_tree = (const bf16*)p.k_tree;
  a.v_tree = (const bf16*)p.v_tree;
  a.k_cache = (const bf16*)p.k_cache;
  a.v_cache = (const bf16*)p.v_cache;
  a.prefix_len = p.prefix_len;
  a.mask = p.mask;
  a.block_idx = p.block_idx;
  a.n_blocks = p.n_blocks;
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float2*>(reinterpret_cast<char*>(workspace) + plan.ws_o_bytes);
  a.dev_err = dev_err;
  a.out = (bf16*)p.out;
  a.lse = p.lse;
  a.seq_stride = d.cache_seq_stride ? d.cache_seq_stride
                                    : (int64_t)d.n_kv_heads * d.cache_capacity * d.head_dim;
  a.batch = d.batch;
  a.n = d.n_nodes;
  a.hq = d.n_q_heads;
  a.hkv = d.n_kv_heads;
  a.grp = d.n_q_heads / d.n_kv_heads;
  a.cap = d.cache_capacity;
  a.words = (d.n_nodes + 31) / 32;
  a.block_size = d.max_blocks ? d.block_size : 1;
  a.max_blocks = d.max_blocks;
  a.max_prefix = d.max_prefix_len;
  a.chunk = plan.chunk;
  a.splits = plan.splits;
  a.row_groups = plan.row_groups;
  a.rows = plan.rows;
  const float scale = d.softmax_scale > 0.f ? d.softmax_scale : 1.f / sqrtf((float)d.head_dim);
  a.c = scale * 1.44269504088896340736f;

  const dim3 grid(plan.splits + 1, d.n_kv_heads * plan.row_groups, d.batch);
  if (d.head_dim == 128)
    launch_split_rb<128>(plan.row_blocks, a, grid, stream);
  else
    launch_split_rb<64>(plan.row_blocks, a, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t total = (int64_t)d.batch * d.n_nodes * d.n_q_heads * (d.head_dim / 4);
  const dim3 cgrid((unsigned)((total + kThreads - 1) / kThreads));
  if (d.head_dim == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tv
