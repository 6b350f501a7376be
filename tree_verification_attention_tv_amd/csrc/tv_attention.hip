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
//    K/V tile is read from HBM once and reused by all rows (rows FLOP/byte).
//    Each wave owns RB blocks of 16 rows.
//  * The prefix (full rows, or the listed blocks) is cut into `splits`
//    contiguous ranges; the tree block is one more split whose tiles are
//    masked with the packed ancestor bits.  A combine kernel merges the
//    (max, sum, unnormalised output) partials in a fixed order.
//  * 32-token K/V tiles flow HBM -> registers -> LDS through a 3-slot LDS
//    ring with two register stages, so two tiles are in flight per CU.  LDS
//    rows are padded (K: D+8, V: D+16 elements) so that the 16-byte K reads
//    and the 8-byte transposing V reads below are free of bank conflicts,
//    and every operand address is a per-lane base plus an immediate.
//  * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16.  The
//    S^T accumulator gives every lane one query row and four tokens, so row
//    statistics need two cross-lane steps; P^T is packed to bf16 straight
//    from those registers as the B operand of the PV product, and the V^T
//    A operand comes from ds_read_b64_tr_b16 (two per operand).
//  * Software pipeline: QK of tile i+1 is issued before the softmax of tile
//    i, so MFMA work overlaps the VALU softmax.
//  * Softmax in fp32, log2 domain (scale * log2 e folded into one FMA
//    before v_exp_f32).  Each row's reference max is fixed at the first tile
//    in which the row sees a key, so the hot loop never rescales the output
//    accumulators: later scores above the reference only make p > 1, which
//    fp32 accumulates exactly enough (p is also exact in bf16's 8-bit
//    exponent).  If a row's sum leaves [1, 2^100] or an output is not
//    finite, the split is recomputed with the exact row max from a QK-only
//    pre-pass (p <= 1 then).  Masked scores are -inf.
#include "tv_internal.h"

#include <math.h>

#include <type_traits>

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;        // tokens per KV tile
constexpr int kSlots = 3;        // LDS ring slots
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
  int block_size, block_shift, max_blocks, max_prefix;  // block_shift < 0: not a power of 2
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

// Hide a per-tile LDS base from loop-invariant code motion so operand
// addresses stay "base + immediate" instead of one register each.
#define LDSP(T) __attribute__((address_space(3))) T*
template <typename T>
__device__ __forceinline__ void opaque(__attribute__((address_space(3))) T*& p) {
  asm volatile("" : "+v"(p));
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap permutes: after swapping, the two results of each
// swap hold the value of a lane and of its partner.
__device__ __forceinline__ float xmax16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float xsum16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int RB, bool PARTIAL>
__global__ __launch_bounds__(kThreads, 1) void attn_split_kernel(AttnArgs a) {
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int DC = D / 32;                // k-steps of the QK^T product
  constexpr int DB = D / 16;                // 16-wide output blocks of PV
  constexpr int KSTR = D + 8;               // LDS row stride of K (elements)
  constexpr int VSTR = D + 16;              // LDS row stride of V (elements)
  constexpr int RSTEP = kThreads / CH;      // rows covered by one load step
  constexpr int LOADS = kTile / RSTEP;      // 16-byte loads per thread per tensor per tile
  static_assert(LOADS >= 1 && kTile % RSTEP == 0, "tile / thread mismatch");

  __shared__ __attribute__((aligned(16))) bf16 Ks[kSlots][kTile * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kSlots][kTile * VSTR];
  __shared__ uint32_t svalid[kSlots];
  __shared__ uint32_t smask[TV_MAX_NODES * (TV_MAX_NODES / 32)];  // tree rows of this WG

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

  const int wg_row0 = rg * (64 * RB);
  const int row0 = wg_row0 + wave * (16 * RB);
  const bool active = row0 < a.rows;

  // ---- tree rows' mask words staged in LDS -------------------------------
  const int node0 = wg_row0 / a.grp;
  if (tree) {
    const int node1 = min(a.n, (wg_row0 + 64 * RB + a.grp - 1) / a.grp);
    const int cnt = (node1 - node0) * a.words;
    const uint32_t* src = a.mask + ((int64_t)b * a.n + node0) * a.words;
    for (int k = tid; k < cnt; k += kThreads) smask[k] = src[k];
  }

  // ---- Q^T fragments (B operand of S^T = K Q^T) ----------------------------
  bf16x8 qf[RB][DC];
#pragma unroll
  for (int mb = 0; mb < RB; ++mb) {
    const int m = row0 + 16 * mb + col;
    const bool real = m < a.rows;
    const int i = real ? m / a.grp : 0;
    const int h = g * a.grp + (real ? m - i * a.grp : 0);
    const bf16* qrow = a.q + (((int64_t)b * a.n + i) * a.hq + h) * D + 8 * grp4;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[mb][dc] = real ? *reinterpret_cast<const bf16x8*>(qrow + 32 * dc) : bf16x8{};
  }

  // ---- source rows --------------------------------------------------------
  const bf16* kbase;
  const bf16* vbase;
  int row_elems;
  if (tree) {
    kbase = a.k_tree + ((int64_t)b * a.n * a.hkv + g) * D;
    vbase = a.v_tree + ((int64_t)b * a.n * a.hkv + g) * D;
    row_elems = a.hkv * D;
  } else {
    kbase = a.k_cache + b * a.seq_stride + (int64_t)g * a.cap * D;
    vbase = a.v_cache + b * a.seq_stride + (int64_t)g * a.cap * D;
    row_elems = D;
  }
  const int lrow = tid / CH;         // first tile row this thread loads
  const int lcol = (tid % CH) * 8;   // its column (elements)
  const int32_t* blist = PARTIAL ? a.block_idx + (int64_t)b * a.max_blocks : nullptr;

  // source row of slot u (caller guarantees u < end), -1 when empty
  auto partial_row = [&](int u) -> int {
    const int bi = a.block_shift >= 0 ? (u >> a.block_shift) : (u / a.block_size);
    const int blk = blist[bi];
    if (blk < 0 || (int64_t)blk * a.block_size >= p_len) {
      err |= TV_DERR_BAD_BLOCK;
      return -1;
    }
    const int row = blk * a.block_size + (u - bi * a.block_size);
    return row < p_len ? row : -1;
  };

  // ---- staging: registers -> LDS ring --------------------------------------
  uint4 kreg[2][LOADS], vreg[2][LOADS];
  uint32_t vb_reg[2] = {0u, 0u};

  auto load_tile = [&](int st, int t0) {
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const int u = t0 + lrow + ld * RSTEP;
      int row = u < end ? u : -1;
      if (PARTIAL && !tree && row >= 0) row = partial_row(u);
      if (row >= 0) {
        const int64_t off = (int64_t)row * row_elems + lcol;
        kreg[st][ld] = *reinterpret_cast<const uint4*>(kbase + off);
        vreg[st][ld] = *reinterpret_cast<const uint4*>(vbase + off);
      } else {
        kreg[st][ld] = uint4{0u, 0u, 0u, 0u};
        vreg[st][ld] = uint4{0u, 0u, 0u, 0u};
      }
    }
    uint32_t vb;
    if (PARTIAL && !tree) {
      const int u = t0 + lane;
      const bool v = lane < kTile && u < end && partial_row(u) >= 0;
      vb = (uint32_t)__ballot(v);
    } else {
      const int cnt = end - t0;
      vb = cnt >= kTile ? 0xFFFFFFFFu : ((1u << cnt) - 1u);
    }
    vb_reg[st] = vb;
  };

  auto store_tile = [&](int st, int slot) {
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const int r = lrow + ld * RSTEP;
      *reinterpret_cast<uint4*>(&Ks[slot][r * KSTR + lcol]) = kreg[st][ld];
      *reinterpret_cast<uint4*>(&Vs[slot][r * VSTR + lcol]) = vreg[st][ld];
    }
    if (tid == 0) svalid[slot] = vb_reg[st];
  };

  // ---- per-tile math --------------------------------------------------------
  // S^T for one tile: sacc[tb][mb][r] = score of token tb*16 + 4*grp4 + r,
  // row row0 + 16*mb + col.  Masked entries are -inf.
  auto qk_tile = [&](int slot, int tile_idx, f32x4 (&sacc)[2][RB]) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int mb = 0; mb < RB; ++mb) sacc[tb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    LDSP(const bf16) kt = (LDSP(const bf16))&Ks[slot][col * KSTR + 8 * grp4];
    opaque(kt);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 kf = *(LDSP(const bf16x8))(kt + tb * 16 * KSTR + 32 * dc);
#pragma unroll
        for (int mb = 0; mb < RB; ++mb)
          sacc[tb][mb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[mb][dc], sacc[tb][mb], 0, 0, 0);
      }
    }
    const uint32_t vbits = svalid[slot];
    if (tree || vbits != 0xFFFFFFFFu) {
#pragma unroll
      for (int mb = 0; mb < RB; ++mb) {
        uint32_t allow = vbits;
        if (tree) {
          const int m = row0 + 16 * mb + col;
          allow &= m < a.rows ? smask[(m / a.grp - node0) * a.words + tile_idx] : 0u;
        }
        allow >>= 4 * grp4;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!((allow >> (16 * tb + r)) & 1u)) sacc[tb][mb][r] = -INFINITY;
      }
    }
  };

  f32x4 o[RB][DB];
  float mref[RB], lrun[RB];
  bool mset = false;  // wave-uniform: every real row of the wave has a reference

  // p = 2^(s*c - mref) of one tile for row block mb, packed as the PV B
  // operand.  The reference is taken from the first tile with a finite max.
  auto softmax_block = [&](f32x4 (&sacc)[2][RB], int mb) -> bf16x8 {
    if (!mset) {
      float mx = fmaxf(fmaxf(fmaxf(sacc[0][mb][0], sacc[0][mb][1]), fmaxf(sacc[0][mb][2], sacc[0][mb][3])),
                       fmaxf(fmaxf(sacc[1][mb][0], sacc[1][mb][1]), fmaxf(sacc[1][mb][2], sacc[1][mb][3])));
      mx = xmax16_32(mx) * a.c;
      mref[mb] = mref[mb] == -INFINITY ? mx : mref[mb];
    }
    const float muse = (mref[mb] == -INFINITY) ? 0.f : mref[mb];
    bf16x8 pb;
    float psum = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tb][mb][r], a.c, -muse));
        psum += pv;
        pb[tb * 4 + r] = (bf16)pv;
      }
    lrun[mb] += psum;
    return pb;
  };

  auto update_mset = [&]() {
    bool missing = false;
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) missing |= (row0 + 16 * mb + col < a.rows) && mref[mb] == -INFINITY;
    mset = !__ballot(missing);
  };

  // O^T += V^T P^T for one tile.  k-slot j of lane group q is token 4q+j
  // (j<4) or 16+4q+(j-4): the tokens the lane holds in the S^T registers.
  // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4
  // of the 8-byte chunks addressed by lanes 4k + i/4 (k = 0..3); lane
  // 4k + qq therefore addresses token (base + k), columns 4qq..4qq+3.
  auto pv_tile = [&](int slot, const bf16x8 (&pb)[RB]) {
    LDSP(bf16) vlo = (LDSP(bf16))&Vs[slot][(4 * grp4 + (col >> 2)) * VSTR + 4 * (col & 3)];
    opaque(vlo);
    LDSP(bf16) vhi = vlo + 16 * VSTR;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP(i16x4))(vlo + 16 * db));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP(i16x4))(vhi + 16 * db));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, both);
#pragma unroll
      for (int mb = 0; mb < RB; ++mb)
        o[mb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[mb], o[mb][db], 0, 0, 0);
    }
  };

  // ---- pipeline -------------------------------------------------------------
  // tile t lives in LDS slot t % 3; register stage (t & 1) carries tile t from
  // its global load (two iterations ahead) to its LDS store (one ahead).
  const int ntiles = (end - begin + kTile - 1) / kTile;

  auto run = [&]() {
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) {
      lrun[mb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[mb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    load_tile(0, begin);
    if (ntiles > 1) load_tile(1, begin + kTile);
    store_tile(0, 0);
    if (ntiles > 1) store_tile(1, 1);
    if (ntiles > 2) load_tile(0, begin + 2 * kTile);
    if (ntiles > 3) load_tile(1, begin + 3 * kTile);
    __syncthreads();

    f32x4 sA[2][RB], sB[2][RB];
    if (active) qk_tile(0, 0, sA);

    // one pipeline step; ST = register stage of tile it+2; scores of tile
    // it are in `cur`, tile it+1's go to `nxt`
    auto step = [&](auto st_tag, int it, f32x4 (&cur)[2][RB], f32x4 (&nxt)[2][RB]) {
      constexpr int ST = decltype(st_tag)::value;
      if (it + 2 < ntiles) {
        store_tile(ST, (it + 2) % kSlots);
        if (it + 4 < ntiles) load_tile(ST, begin + (it + 4) * kTile);
      }
      if (active) {
        if (it + 1 < ntiles) qk_tile((it + 1) % kSlots, it + 1, nxt);
        bf16x8 pb[RB];
#pragma unroll
        for (int mb = 0; mb < RB; ++mb) pb[mb] = softmax_block(cur, mb);
        if (!mset) update_mset();
        pv_tile(it % kSlots, pb);
      }
      __syncthreads();
    };
    for (int it = 0; it < ntiles; it += 2) {
      step(std::integral_constant<int, 0>{}, it, sA, sB);
      if (it + 1 < ntiles) step(std::integral_constant<int, 1>{}, it + 1, sB, sA);
    }
  };

#pragma unroll
  for (int mb = 0; mb < RB; ++mb) mref[mb] = -INFINITY;
  run();

  // ---- overflow check; exact two-pass recompute when needed --------------
  __shared__ int s_redo;
  if (tid == 0) s_redo = 0;
  __syncthreads();
  if (active) {
    bool bad = false;
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) {
      const float l = xsum16_32(lrun[mb]);
      bool fin = true;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) fin = fin && __builtin_isfinite(o[mb][db][e]);
      const bool real = row0 + 16 * mb + col < a.rows;
      bad |= real && mref[mb] != -INFINITY && !(l <= kSumMax && fin);
    }
    if (__ballot(bad) && lane == 0) s_redo = 1;
  }
  __syncthreads();
  if (s_redo) {
    // QK-only pre-pass for the exact row max (single-buffered, rare path)
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) mref[mb] = -INFINITY;
    for (int it = 0; it < ntiles; ++it) {
      load_tile(0, begin + it * kTile);
      store_tile(0, 0);
      __syncthreads();
      if (active) {
        f32x4 sc[2][RB];
        qk_tile(0, it, sc);
#pragma unroll
        for (int mb = 0; mb < RB; ++mb) {
          float mx = -INFINITY;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[tb][mb][r]);
          mref[mb] = fmaxf(mref[mb], xmax16_32(mx) * a.c);
        }
      }
      __syncthreads();
    }
    mset = true;
    run();
  }
  if (err) raise_err(a.dev_err, err);

  if (!active) return;
#pragma unroll
  for (int mb = 0; mb < RB; ++mb) {
    const float l = xsum16_32(lrun[mb]);
    const int m = row0 + 16 * mb + col;
    if (m < a.rows) {
      const int i = m / a.grp;
      const int h = g * a.grp + m % a.grp;
      const int64_t pi = (((int64_t)b * (a.splits + 1) + s) * a.n + i) * a.hq + h;
      float* dst = a.part_o + pi * D + 4 * grp4;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = o[mb][db];
      if (grp4 == 0) a.part_ml[pi] = make_float2(mref[mb], l);
    }
  }
}

// Merge the split partials of one (sequence, node, head): m = max m_s,
// l = sum 2^(m_s - m) l_s, o = sum 2^(m_s - m) o_s / l.  Fixed split order.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnArgs a) {
  constexpr int Q4 = D / 4;
  constexpr int U = 8;
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
  const int64_t stride = (int64_t)a.n * a.hq;  // partial rows between splits
  const int64_t p0 = (base * a.n + i) * a.hq + h;

  // splits 0..ns-1 then the tree split
  auto split_of = [&](int k) { return k < ns ? k : a.splits; };
  const int cnt = ns + 1;
  float m = -INFINITY;
  for (int k0 = 0; k0 < cnt; k0 += U) {
    float mv[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      mv[u] = (k0 + u < cnt) ? a.part_ml[p0 + split_of(k0 + u) * stride].x : -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) m = fmaxf(m, mv[u]);
  }

  bf16x4 res;
  float lse_v;
  if (m == -INFINITY) {
    res = bf16x4{};
    lse_v = -INFINITY;
  } else {
    float l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < cnt; k0 += U) {
      float2 ml[U];
      f32x4 ov[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k0 + u < cnt) {
          const int64_t pi = p0 + split_of(k0 + u) * stride;
          ml[u] = a.part_ml[pi];
          ov[u] = *reinterpret_cast<const f32x4*>(a.part_o + pi * D + 4 * dq);
        } else {
          ml[u] = make_float2(-INFINITY, 0.f);
          ov[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = __builtin_amdgcn_exp2f(ml[u].x - m);
        l += w * ml[u].y;
        acc += w * ov[u];
      }
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
  if (args.max_blocks)
    hipLaunchKernelGGL((attn_split_kernel<D, RB, true>), grid, dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, RB, false>), grid, dim3(kThreads), 0, stream, args);
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
  a.block_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == a.block_size) a.block_shift = sh;
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
