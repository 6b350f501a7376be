// SpecPV retrieval of KV blocks for partial verification ("SpecPV: Improving
// Self-Speculative Decoding for Long-Context Generation via Partial
// Verification", Sec. 3.2 "Partial Verification", App. C, App. D).
//
//  * summaries_kernel: element-wise max and min key of every 16-token (any
//    size) block, per KV head, kept as a bf16 cache [B][Hkv][nb][2][D].  One
//    wave per block; bf16 values compare exactly as order-mapped int16 with
//    packed 16-bit max/min.  HBM-bound: it reads the block's K rows once.
//  * Block score: the bound q.k <= sum_d max(q_d hi_d, q_d lo_d) over the
//    block's box [lo, hi].  With q+ = max(q, 0) and q- = min(q, 0) it is
//    [q+ | q-] . [hi | lo], a dot product of length 2D.
//      - mean and last are linear in q: the query rows of a KV group are
//        folded into one fp32 vector [sum q+ | sum q-] first, and each block
//        then costs one 2D-long dot product (score_linear_kernel, a GEMV
//        bound by the summary bytes).
//      - max needs every row's bound: [q+ | q-] (rows) times the summaries
//        (columns) is a bf16 GEMM on v_mfma_f32_16x16x32_bf16, exact
//        products with fp32 accumulation (score_max_kernel); the max over a
//        head's nodes is taken in registers and across lanes.
//    Both write per-KV-head partial scores; the selection sums them.
//  * select_kernel: one workgroup per sequence; thread t owns KPT consecutive
//    blocks and keeps their keys (order-mapped fp32 scores, the KV heads'
//    partial scores summed in head order) in registers.  The sinks and the
//    window are kept; the top-k of the rest come from a radix select over
//    the bits in which the candidates' keys differ (11-bit digits, LDS
//    histograms), equal keys taken in ascending block order; the list is
//    written ascending with workgroup prefix sums.
#include "tv_device.h"

namespace tv {
namespace {

constexpr int kSumThreads = 256;    // summaries: 4 waves, one block each
constexpr int kScoreThreads = 512;  // scoring: 8 waves
constexpr int kScoreWaves = kScoreThreads / kWave;
constexpr int kSelThreads = 1024;   // selection: one workgroup per sequence
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxRowTilesPerWave = 2;

typedef short s16x2 __attribute__((ext_vector_type(2)));

// ---- bf16 order keys ----------------------------------------------------------
// A bf16 bit pattern read as int16, with the 15 magnitude bits flipped when the
// sign is set, orders like the value (-0 just below +0).  The map is its own
// inverse.
__device__ __forceinline__ s16x2 bf16_key(uint32_t w) {
  const s16x2 v = __builtin_bit_cast(s16x2, w);
  return v ^ ((v >> (short)15) & (short)0x7FFF);
}
__device__ __forceinline__ uint32_t bf16_unkey(s16x2 k) {
  return __builtin_bit_cast(uint32_t, k ^ ((k >> (short)15) & (short)0x7FFF));
}

// fp32 order key (unsigned compare), with -0 folded onto +0 so that equal
// values get equal keys.
__device__ __forceinline__ uint32_t f32_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_unkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- cross-lane steps on DPP and the gfx950 row-swap permutes -------------------
// DPP controls: row_ror:n = 0x120 + n, row_shr:n = 0x110 + n, row_bcast:15 =
// 0x142, row_bcast:31 = 0x143.

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, 0xF, false);
}

// sum over the 16 lanes of each row, in every lane of the row
__device__ __forceinline__ float row_sum16(float x) {
  x += __uint_as_float(dpp_u<0x128>(0u, __float_as_uint(x)));
  x += __uint_as_float(dpp_u<0x124>(0u, __float_as_uint(x)));
  x += __uint_as_float(dpp_u<0x122>(0u, __float_as_uint(x)));
  x += __uint_as_float(dpp_u<0x121>(0u, __float_as_uint(x)));
  return x;
}

// sum over lane pairs of rows (0,1) and (2,3), in every lane of both rows
__device__ __forceinline__ float row_pair_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// min and max over the wave, in every lane
__device__ __forceinline__ void wave_minmax(uint32_t& mn, uint32_t& mx) {
#define TV_STEP(C)                                   \
  mn = min(mn, dpp_u<C>(0xFFFFFFFFu, mn));           \
  mx = max(mx, dpp_u<C>(0u, mx));
  TV_STEP(0x128) TV_STEP(0x124) TV_STEP(0x122) TV_STEP(0x121)
#undef TV_STEP
  auto a = __builtin_amdgcn_permlane16_swap(mn, mn, false, false);
  mn = min(a[0], a[1]);
  a = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
  mx = max(a[0], a[1]);
  a = __builtin_amdgcn_permlane32_swap(mn, mn, false, false);
  mn = min(a[0], a[1]);
  a = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
  mx = max(a[0], a[1]);
}

__device__ __forceinline__ int effective_prefix(const int32_t* prefix_len, int b, int limit) {
  const int p = prefix_len[b];
  return p < 0 ? 0 : (p > limit ? limit : p);
}

// ---- summaries ---------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kSumThreads) void summaries_kernel(
    const uint4* __restrict__ k_cache, int64_t seq_stride_vec, int cap, int bs, int nb_cap,
    int hkv, const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ first_token,
    uint4* __restrict__ summ, int32_t* __restrict__ dev_err) {
  constexpr int C = D / 8;   // 16-byte chunks per key row
  constexpr int R = 64 / C;  // rows per wave-wide load
  constexpr int U = 4;       // loads in flight per lane
  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = lane % C, r0 = lane / C;
  const int p_raw = prefix_len[b];
  const int f = first_token ? first_token[b] : 0;
  if (p_raw < 0 || p_raw > cap || f < 0 || f > p_raw) {
    if (blockIdx.x == 0 && g == 0 && threadIdx.x == 0) raise_err(dev_err, TV_DERR_BAD_PREFIX);
    return;
  }
  const int j0 = f / bs, j1 = (p_raw + bs - 1) / bs;  // j1 <= nb_cap since p <= cap
  const uint4* kseq = k_cache + b * seq_stride_vec + (int64_t)g * cap * C + c;
  uint4* sseq = summ + ((int64_t)b * hkv + g) * nb_cap * (2 * C);
  const s16x2 lowest = {(short)0x8000, (short)0x8000}, highest = {0x7FFF, 0x7FFF};
  for (int j = j0 + blockIdx.x * (kSumThreads / kWave) + wave; j < j1;
       j += gridDim.x * (kSumThreads / kWave)) {
    const int row0 = j * bs;
    const int rows = min(bs, p_raw - row0);
    s16x2 mx[4] = {lowest, lowest, lowest, lowest};
    s16x2 mn[4] = {highest, highest, highest, highest};
    for (int r = r0; r < rows; r += U * R) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (r + u * R < rows) v[u] = kseq[(int64_t)(row0 + r + u * R) * C];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (r + u * R < rows) {
          const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const s16x2 k = bf16_key(w[e]);
            mx[e] = __builtin_elementwise_max(mx[e], k);
            mn[e] = __builtin_elementwise_min(mn[e], k);
          }
        }
      }
    }
    // lanes with the same chunk c hold partial results for the same 8 values
#pragma unroll
    for (int off = C; off < kWave; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t om = __shfl_xor(__builtin_bit_cast(uint32_t, mx[e]), off);
        const uint32_t on = __shfl_xor(__builtin_bit_cast(uint32_t, mn[e]), off);
        mx[e] = __builtin_elementwise_max(mx[e], __builtin_bit_cast(s16x2, om));
        mn[e] = __builtin_elementwise_min(mn[e], __builtin_bit_cast(s16x2, on));
      }
    }
    // one 2*D*2-byte record per block: lanes r0 == 0 write the max, r0 == 1 the min
    if (r0 < 2) {
      const s16x2* src = r0 == 0 ? mx : mn;
      uint4 o;
      o.x = bf16_unkey(src[0]);
      o.y = bf16_unkey(src[1]);
      o.z = bf16_unkey(src[2]);
      o.w = bf16_unkey(src[3]);
      sseq[(int64_t)j * (2 * C) + r0 * C + c] = o;
    }
  }
}

// ---- scoring -----------------------------------------------------------------------

struct ScoreArgs {
  const uint16_t* q;       // [B][N][Hq][D]
  const uint4* summ;       // [B][Hkv][nb_cap][2][D] bf16
  const int32_t* prefix_len;
  float* part;             // [B][Hkv][part_stride]
  int n, hq, hkv, group, bs, nb_cap, part_stride, prefix_limit, chunk;
  int last_only;           // linear kernel: fold node n-1 only
};

template <int D>
__global__ __launch_bounds__(kScoreThreads) void score_linear_kernel(ScoreArgs a) {
  constexpr int C = D / 8;                  // 16-byte chunks per query row
  constexpr int SLOTS = kScoreThreads / C;  // query rows folded in parallel
  constexpr int L = 2 * D / 8;              // lanes per block record
  constexpr int BPL = kWave / L;            // blocks per wave-wide load
  constexpr int U = 8;                      // record loads in flight per lane
  constexpr int QU = 8;                     // query-row loads in flight per thread
  __shared__ float s_part[SLOTS][2 * D];
  __shared__ float s_qs[2 * D];
  const int b = blockIdx.z, g = blockIdx.y, t = threadIdx.x;
  const int p = effective_prefix(a.prefix_len, b, a.prefix_limit);
  const int nv = (p + a.bs - 1) / a.bs;
  const int j_begin = blockIdx.x * a.chunk;
  if (j_begin >= nv) return;  // uniform over the workgroup
  const int j_end = min(j_begin + a.chunk, nv);
  const int lane = t % kWave, wave = t / kWave;
  const int sub = lane / L, li = lane % L;
  const uint4* sg = a.summ + ((int64_t)b * a.hkv + g) * a.nb_cap * L;
  float* part = a.part + ((int64_t)b * a.hkv + g) * a.part_stride;

  // The first batch of block records does not depend on the queries: its
  // loads are in flight while the queries are folded.
  uint4 v[U];
  int jb = j_begin + wave * BPL * U;
  auto load_batch = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * BPL + sub;
      if (j < j_end) v[u] = sg[(int64_t)j * L + li];
    }
  };
  load_batch();

  // 1. [sum q+ | sum q-] over the folded rows of this KV group, fp32
  {
    const int c = t % C, slot = t / C;
    const int i0 = a.last_only ? a.n - 1 : 0;
    const int nrows = (a.n - i0) * a.group;
    float pos[8], neg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pos[e] = neg[e] = 0.f;
    const uint4* q4 = reinterpret_cast<const uint4*>(a.q);
    for (int r0 = slot; r0 < nrows; r0 += QU * SLOTS) {
      uint4 qv[QU];
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const int r = r0 + u * SLOTS;
        if (r < nrows) {
          const int i = i0 + r / a.group, h = g * a.group + r % a.group;
          qv[u] = q4[(((int64_t)b * a.n + i) * a.hq + h) * C + c];
        }
      }
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        if (r0 + u * SLOTS < nrows) {
          const uint32_t w[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
            pos[2 * e] += fmaxf(x0, 0.f);
            neg[2 * e] += fminf(x0, 0.f);
            pos[2 * e + 1] += fmaxf(x1, 0.f);
            neg[2 * e + 1] += fminf(x1, 0.f);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_part[slot][c * 8 + e] = pos[e];
      s_part[slot][D + c * 8 + e] = neg[e];
    }
    __syncthreads();
    for (int e = t; e < 2 * D; e += kScoreThreads) {
      float s = 0.f;
#pragma unroll 8
      for (int sl = 0; sl < SLOTS; ++sl) s += s_part[sl][e];
      s_qs[e] = s;
    }
    __syncthreads();
  }

  // 2. one dot product of length 2D per block
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = s_qs[li * 8 + e];
  while (true) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf16_lo(w[e]), qv[2 * e], acc);
        acc = fmaf(bf16_hi(w[e]), qv[2 * e + 1], acc);
      }
      acc = row_sum16(acc);
      if (L == 32) acc = row_pair_sum(acc);
      const int j = jb + u * BPL + sub;
      if (li == 0 && j < j_end) part[j] = acc;
    }
    jb += kScoreWaves * BPL * U;
    if (jb >= j_end) break;  // uniform over the wave
    load_batch();
  }
}

// bf16 pair -> (max(x,0), min(x,0)) pairs, exact bit selections
__device__ __forceinline__ void split_sign(uint32_t w, uint32_t& pos, uint32_t& neg) {
  const uint32_t m = ((w >> 15) & 0x00010001u) * 0xFFFFu;  // all ones in each negative half
  pos = w & ~m;
  neg = w & m;
}

template <int D>
__global__ __launch_bounds__(kScoreThreads) void score_max_kernel(ScoreArgs a) {
  constexpr int KS = 2 * D / 32;  // k-steps of 32 over [q+ | q-]
  constexpr int C = D / 8;
  constexpr int RPW = kMaxRowTilesPerWave;
  __shared__ uint32_t s_hmax[2][TV_MAX_SELECT_GROUP][16];  // per head, per column: key of the max
  const int b = blockIdx.z, g = blockIdx.y, t = threadIdx.x;
  const int p = effective_prefix(a.prefix_len, b, a.prefix_limit);
  const int nv = (p + a.bs - 1) / a.bs;
  const int j_begin = blockIdx.x * a.chunk;
  if (j_begin >= nv) return;
  const int j_end = min(j_begin + a.chunk, nv);
  const int lane = t % kWave, wave = t / kWave;
  const int col = lane % 16, quad = lane / 16;
  const int npad = (a.n + 15) & ~15;
  const int tiles = a.group * npad / 16;             // 16-row tiles of [q+ | q-]
  const int per_pass = kScoreWaves * RPW;
  const bool one_pass = tiles <= per_pass;
  for (int e = t; e < 2 * TV_MAX_SELECT_GROUP * 16; e += kScoreThreads) (&s_hmax[0][0][0])[e] = 0u;
  __syncthreads();

  const uint4* q4 = reinterpret_cast<const uint4*>(a.q);
  bf16x8 af[RPW][KS];
  // A operand of row tile rt: lane holds row rt*16 + col, k = ks*32 + 8*quad .. +7
  auto load_a = [&](int pass) {
#pragma unroll
    for (int m = 0; m < RPW; ++m) {
      const int rt = pass * per_pass + m * kScoreWaves + wave;
      const int row = rt * 16 + col;
      const int hl = row / npad, i = row % npad;
      const bool ok = rt < tiles && i < a.n;
      const int64_t base = (((int64_t)b * a.n + (ok ? i : 0)) * a.hq + g * a.group + (ok ? hl : 0)) * C;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int k = ks * 32 + 8 * quad;
        const int chunk = (k % D) / 8;
        uint4 v = ok ? q4[base + chunk] : uint4{0, 0, 0, 0};
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t ps, ng;
          split_sign(w[e], ps, ng);
          w[e] = k < D ? ps : ng;
        }
        af[m][ks] = __builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]});
      }
    }
  };
  if (one_pass) load_a(0);

  const uint4* sg = a.summ + ((int64_t)b * a.hkv + g) * a.nb_cap * (2 * C);
  float* part = a.part + ((int64_t)b * a.hkv + g) * a.part_stride;
  int buf = 0;
  for (int j0 = j_begin; j0 < j_end; j0 += 16, buf ^= 1) {
    // B operand: lane holds block j0 + col, k = ks*32 + 8*quad .. +7 of its record
    bf16x8 bfr[KS];
    const int jb = min(j0 + col, j_end - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bfr[ks] = __builtin_bit_cast(bf16x8, sg[(int64_t)jb * (2 * C) + ks * 4 + quad]);
    for (int pass = 0; pass * per_pass < tiles; ++pass) {
      if (!one_pass) load_a(pass);
#pragma unroll
      for (int m = 0; m < RPW; ++m) {
        const int rt = pass * per_pass + m * kScoreWaves + wave;
        if (rt >= tiles) continue;  // uniform over the wave
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m][ks], bfr[ks], acc, 0, 0, 0);
        // lane holds rows rt*16 + 4*quad + r of column col; all rows of a
        // tile belong to one head because npad is a multiple of 16
        const int row0 = rt * 16;
        const int hl = row0 / npad, i0 = row0 % npad + 4 * quad;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (i0 + r < a.n) mx = fmaxf(mx, acc[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (quad == 0) atomicMax(&s_hmax[buf][hl][col], f32_key(mx));
      }
    }
    __syncthreads();
    if (t < 16) {
      float s = 0.f;
      for (int hl = 0; hl < a.group; ++hl) {
        s += f32_unkey(s_hmax[buf][hl][t]);
        s_hmax[buf][hl][t] = 0u;
      }
      if (j0 + t < j_end) part[j0 + t] = s;
    }
  }
}

// ---- selection ---------------------------------------------------------------------

struct SelectArgs {
  const float* part;       // [B][Hkv][part_stride]
  float* scores;           // [B][nb_cap] or nullptr
  const int32_t* prefix_len;
  int32_t* block_idx;      // [B][max_blocks]
  int32_t* n_blocks;       // [B]
  int32_t* dev_err;
  int hkv, nb_cap, part_stride, bs, prefix_limit, cap, max_prefix;
  int n_sink, n_window, top_k, max_blocks;
  float count;             // divisor: query rows averaged
};

// inclusive prefix sum over the wave's 64 lanes: row_shr steps within each
// row of 16, then row_bcast:15 and row_bcast:31 carry row totals upward
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u<0x111>(0u, v);
  v += dpp_u<0x112>(0u, v);
  v += dpp_u<0x114>(0u, v);
  v += dpp_u<0x118>(0u, v);
  v += dpp_u<0x142, 0xA>(0u, v);
  v += dpp_u<0x143, 0xC>(0u, v);
  return v;
}

// Inclusive prefix sum over the workgroup in thread order; `total` gets the sum.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* s_wsum, uint32_t& total) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const uint32_t x = wave_incl_scan(v);
  if (lane == kWave - 1) s_wsum[w] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const uint32_t s = s_wsum[i];
    off += i < w ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return x + off;
}

// KPT consecutive blocks per thread (thread t owns blocks t*KPT ..), keys in
// registers.  KPT is a multiple of 4.
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_wsum[kSelWaves], s_wmin[kSelWaves], s_wmax[kSelWaves];
  __shared__ uint32_t s_bin, s_above;
  const int b = blockIdx.x, t = threadIdx.x;
  const int lane = t % kWave, wave = t / kWave;
  const int p_raw = a.prefix_len[b];
  if (t == 0 && (p_raw < 0 || p_raw > a.cap || p_raw > a.max_prefix))
    raise_err(a.dev_err, TV_DERR_BAD_PREFIX);
  const int p = p_raw < 0 ? 0 : (p_raw > a.prefix_limit ? a.prefix_limit : p_raw);
  const int nv = (p + a.bs - 1) / a.bs;
  const int j0 = t * KPT;
  const int lo = min(a.n_sink, nv);
  const int hi = max(nv - a.n_window, lo);

  // 1. scores: the KV heads' partial scores summed in head order, averaged
  uint32_t key[KPT];
#pragma unroll
  for (int u0 = 0; u0 < KPT; u0 += 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const bool any = j0 + u0 < nv;  // then j0+u0+3 < part_stride (a multiple of 4)
    constexpr int GB = KPT <= 16 ? 16 : 4;  // heads loaded together (registers)
    for (int g0 = 0; g0 < a.hkv; g0 += GB) {
      float4 v[GB];
#pragma unroll
      for (int gg = 0; gg < GB; ++gg)
        if (any && g0 + gg < a.hkv)
          v[gg] = *reinterpret_cast<const float4*>(
              a.part + ((int64_t)b * a.hkv + g0 + gg) * a.part_stride + j0 + u0);
#pragma unroll
      for (int gg = 0; gg < GB; ++gg)
        if (any && g0 + gg < a.hkv) {
          acc[0] += v[gg].x;
          acc[1] += v[gg].y;
          acc[2] += v[gg].z;
          acc[3] += v[gg].w;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = acc[e] / a.count;
      key[u0 + e] = f32_key(s);
      if (a.scores && j0 + u0 + e < nv) a.scores[(int64_t)b * a.nb_cap + j0 + u0 + e] = s;
    }
  }

  // 2. candidates [lo, hi): neither sink nor window
  const int ncand = hi - lo;
  const int k = min(a.top_k, ncand);
  const bool all_cand = k == ncand;
  const bool radix = k > 0 && !all_cand;
  uint32_t want_val = 0, need = 0;
  if (radix) {
    // leading bits shared by every candidate key need no pass
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int j = j0 + u;
      if (j >= lo && j < hi) {
        kmin = min(kmin, key[u]);
        kmax = max(kmax, key[u]);
      }
    }
    wave_minmax(kmin, kmax);
    if (lane == 0) {
      s_wmin[wave] = kmin;
      s_wmax[wave] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
      kmin = min(kmin, s_wmin[i]);
      kmax = max(kmax, s_wmax[i]);
    }
    const int cp = kmin == kmax ? 32 : __clz(kmin ^ kmax);
    uint32_t want_mask = cp == 0 ? 0u : (cp == 32 ? 0xFFFFFFFFu : (0xFFFFFFFFu << (32 - cp)));
    want_val = kmin & want_mask;
    uint32_t remaining = (uint32_t)k;
    for (int left = 32 - cp; left > 0;) {  // uniform over the workgroup
      const int bits = left < 11 ? left : 11;
      const int shift = left - bits;
      const int nbins = 1 << bits;
      for (int i = t; i < nbins; i += kSelThreads) s_hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int j = j0 + u;
        if (j >= lo && j < hi && (key[u] & want_mask) == want_val)
          atomicAdd(&s_hist[(key[u] >> shift) & (nbins - 1)], 1u);
      }
      __syncthreads();
      // bins from the top: thread t covers bins hb and hb - 1
      const int hb = nbins - 1 - 2 * t;
      const uint32_t c_hi = hb >= 0 ? s_hist[hb] : 0u;
      const uint32_t c_lo = hb >= 1 ? s_hist[hb - 1] : 0u;
      uint32_t tot;
      const uint32_t before = block_incl_scan(c_hi + c_lo, s_wsum, tot) - (c_hi + c_lo);
      if (before < remaining && remaining <= before + c_hi) {
        s_bin = (uint32_t)hb;
        s_above = before;
      } else if (before + c_hi < remaining && remaining <= before + c_hi + c_lo) {
        s_bin = (uint32_t)(hb - 1);
        s_above = before + c_hi;
      }
      __syncthreads();
      want_val |= s_bin << shift;
      want_mask |= (uint32_t)(nbins - 1) << shift;
      remaining -= s_above;
      left = shift;
      __syncthreads();
    }
    need = remaining;  // candidates with key == want_val still to take, lowest ids first
  }

  // 3. ascending output: sinks, window, keys above the threshold, and the
  //    first `need` candidates whose key equals it
  uint32_t neq = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int j = j0 + u;
    neq += (radix && j >= lo && j < hi && key[u] == want_val) ? 1u : 0u;
  }
  uint32_t tot_eq;
  uint32_t eq_rank = block_incl_scan(neq, s_wsum, tot_eq) - neq;
  static_assert(KPT <= 64, "selection flags are kept in one 64-bit mask");
  uint64_t sel = 0;
  uint32_t nsel = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int j = j0 + u;
    const bool cand = j >= lo && j < hi;
    bool s = j < nv && (!cand || all_cand);
    if (cand && radix) {
      if (key[u] > want_val) s = true;
      else if (key[u] == want_val) s = eq_rank++ < need;
    }
    sel |= (uint64_t)s << u;
    nsel += s;
  }
  uint32_t tot_sel;
  uint32_t pos = block_incl_scan(nsel, s_wsum, tot_sel) - nsel;
  int32_t* out = a.block_idx + (int64_t)b * a.max_blocks;
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if ((sel >> u) & 1u) {
      if (pos < (uint32_t)a.max_blocks) out[pos] = j0 + u;
      ++pos;
    }
  for (int i = (int)tot_sel + t; i < a.max_blocks; i += kSelThreads) out[i] = -1;
  if (t == 0) a.n_blocks[b] = (int32_t)min(tot_sel, (uint32_t)a.max_blocks);
}
}  // namespace

SelectPlan plan_select(const tv_select_desc& d, int cu_count) {
  SelectPlan p{};
  p.nb_cap = (d.cache_capacity + d.block_size - 1) / d.block_size;
  const int limit = d.max_prefix_len < d.cache_capacity ? d.max_prefix_len : d.cache_capacity;
  p.nb_max = (limit + d.block_size - 1) / d.block_size;
  // blocks per thread of the selection workgroup (keys live in registers)
  static_assert(32 * kSelThreads == TV_MAX_SELECT_BLOCKS, "selection capacity");
  p.kpt = p.nb_max <= 4 * kSelThreads ? 4 : p.nb_max <= 16 * kSelThreads ? 16
        : p.nb_max <= 32 * kSelThreads ? 32 : 0;
  // chunk of blocks per scoring workgroup: about one workgroup per CU, never
  // below 64 blocks (each workgroup also folds or loads the queries)
  const int64_t groups = (int64_t)d.batch * d.n_kv_heads;
  const int64_t want = groups > 0 ? (cu_count + groups - 1) / groups : 1;
  int chunk = (int)((p.nb_max + want - 1) / (want > 0 ? want : 1));
  chunk = chunk < 64 ? 64 : chunk;
  p.chunk = (chunk + 15) & ~15;
  p.chunks = p.nb_max > 0 ? (p.nb_max + p.chunk - 1) / p.chunk : 0;
  p.part_stride = (p.nb_cap + 3) & ~3;
  const size_t part = (size_t)d.batch * d.n_kv_heads * p.part_stride * sizeof(float);
  p.ws_part_bytes = (part + 255) & ~(size_t)255;
  return p;
}

hipError_t launch_summaries(const void* k_cache, int64_t seq_stride, int cap, int batch, int hkv,
                            int d, int bs, const int32_t* prefix_len, const int32_t* first_token,
                            int max_tokens, void* summaries, int32_t* dev_err,
                            hipStream_t stream) {
  const int nb_cap = (cap + bs - 1) / bs;
  int64_t blocks = (int64_t)(max_tokens + bs - 1) / bs + (first_token ? 1 : 0);
  if (blocks > nb_cap) blocks = nb_cap;
  if (blocks < 1) blocks = 1;
  const int64_t per_wg = kSumThreads / kWave;
  int64_t gx = (blocks + per_wg - 1) / per_wg;
  if (gx > 65535) gx = 65535;
  const dim3 grid((unsigned)gx, hkv, batch);
  if (d == 128)
    hipLaunchKernelGGL(summaries_kernel<128>, grid, dim3(kSumThreads), 0, stream,
                       (const uint4*)k_cache, seq_stride / 8, cap, bs, nb_cap, hkv, prefix_len,
                       first_token, (uint4*)summaries, dev_err);
  else
    hipLaunchKernelGGL(summaries_kernel<64>, grid, dim3(kSumThreads), 0, stream,
                       (const uint4*)k_cache, seq_stride / 8, cap, bs, nb_cap, hkv, prefix_len,
                       first_token, (uint4*)summaries, dev_err);
  return hipGetLastError();
}

hipError_t launch_select(const tv_select_desc& d, const SelectPlan& plan, const void* q,
                         const void* summaries, const int32_t* prefix_len, int32_t* block_idx,
                         int32_t* n_blocks, float* scores, void* workspace, int32_t* dev_err,
                         hipStream_t stream) {
  float* part = static_cast<float*>(workspace);
  const int limit = d.max_prefix_len < d.cache_capacity ? d.max_prefix_len : d.cache_capacity;
  const int group = d.n_q_heads / d.n_kv_heads;
  if (plan.chunks > 0) {
    ScoreArgs sa{};
    sa.q = static_cast<const uint16_t*>(q);
    sa.summ = static_cast<const uint4*>(summaries);
    sa.prefix_len = prefix_len;
    sa.part = part;
    sa.n = d.n_nodes;
    sa.hq = d.n_q_heads;
    sa.hkv = d.n_kv_heads;
    sa.group = group;
    sa.bs = d.block_size;
    sa.nb_cap = plan.nb_cap;
    sa.part_stride = plan.part_stride;
    sa.prefix_limit = limit;
    sa.chunk = plan.chunk;
    sa.last_only = d.reduction == TV_REDUCE_LAST;
    const dim3 grid(plan.chunks, d.n_kv_heads, d.batch);
    if (d.reduction == TV_REDUCE_MAX) {
      if (d.head_dim == 128)
        hipLaunchKernelGGL(score_max_kernel<128>, grid, dim3(kScoreThreads), 0, stream, sa);
      else
        hipLaunchKernelGGL(score_max_kernel<64>, grid, dim3(kScoreThreads), 0, stream, sa);
    } else {
      if (d.head_dim == 128)
        hipLaunchKernelGGL(score_linear_kernel<128>, grid, dim3(kScoreThreads), 0, stream, sa);
      else
        hipLaunchKernelGGL(score_linear_kernel<64>, grid, dim3(kScoreThreads), 0, stream, sa);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  SelectArgs a{};
  a.part = part;
  a.scores = scores;
  a.prefix_len = prefix_len;
  a.block_idx = block_idx;
  a.n_blocks = n_blocks;
  a.dev_err = dev_err;
  a.hkv = d.n_kv_heads;
  a.nb_cap = plan.nb_cap;
  a.part_stride = plan.part_stride;
  a.bs = d.block_size;
  a.prefix_limit = limit;
  a.cap = d.cache_capacity;
  a.max_prefix = d.max_prefix_len;
  a.n_sink = d.n_sink_blocks;
  a.n_window = d.n_window_blocks;
  a.top_k = d.top_k;
  a.max_blocks = d.max_blocks;
  a.count = d.reduction == TV_REDUCE_MEAN ? (float)d.n_nodes * (float)d.n_q_heads
                                          : (float)d.n_q_heads;
  if (plan.kpt == 4)
    hipLaunchKernelGGL(select_kernel<4>, dim3(d.batch), dim3(kSelThreads), 0, stream, a);
  else if (plan.kpt == 16)
    hipLaunchKernelGGL(select_kernel<16>, dim3(d.batch), dim3(kSelThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(select_kernel<32>, dim3(d.batch), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tv
