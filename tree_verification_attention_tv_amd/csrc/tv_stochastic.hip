// Stochastic (temperature > 0) acceptance of a verified draft tree.
//
// Sources: SpecPV Sec. 2 "Related Work" (speculative sampling is equivalent
// to sampling from the target; tree-structured candidates), SpecPV App. D
// and App. E and SpecBlock Sec. 4 (sampling at T = 0.6, 0.7, 1.0).  Random
// numbers: Philox-4x64-10 (Salmon et al., SC 2011) on counters, so every
// decision has a fixed uniform.
//
// Node u's target distribution is p_u = softmax(l_u / T), optionally
// filtered (SpecPV App. D: T 0.6, top-p 0.95, top-k 20; App. E: T 0.7 and
// 1.0, top-p 0.9): top-k keeps the tokens with fewer than k strictly larger
// logits, then top-p keeps, of those, the tokens whose strictly larger ones
// hold less than p of their mass, and the kept probabilities are
// renormalised.  Both keep every token at or above a logit threshold tau, so
// the filter is one value per row.  Drafts are point masses: at an accepted
// node the children are tried in ascending node index, child c (token x) is
// accepted with probability p_u(x) / R, R the mass not yet rejected at u (a
// token already rejected at u has probability 0).  When every child is
// rejected the bonus token is drawn from the residual by inverse CDF in
// vocabulary order.
//
// Kernels:
//  0. the filter's threshold tau (only with a filter), by radix selection
//     over order-preserving 32-bit keys of the logits (11-bit digits,
//     histograms in LDS): top-k by counts, then top-p by masses 2^((l - M) c)
//     in 2^-40 fixed point (integer sums, so the result does not depend on
//     the order of the atomics).  Top-k of at most 32 goes through
//     candidate lists: cand_collect_kernel, over 8192-element slices, keeps
//     each slice's elements at or above a lower bound of its top-k, then
//     filter_threshold_kernel, one workgroup per row, selects among them (or
//     searches the whole row when ties overflow a list).  Otherwise the
//     selection is spread over the same slices (sel_*_kernel): a launch per
//     digit, each adding its slices' histograms into the row's in global
//     memory.
//  1. softmax_stats_kernel: one workgroup per (row chunk, logits row), the
//     same streaming layout as the greedy argmax: each thread's 16-byte loads
//     are all in flight at once.  Per chunk it writes (m, s): the chunk's max
//     logit and sum_v 2^((l_v - m) c), c = log2(e) / T, summed in a fixed
//     order (thread, then DPP/lane tree, then waves in order), over the
//     tokens at or above the row's tau (after the spread selection, derived
//     here from its last histogram).  HBM-bound: the B*N*V logits are read
//     once.
//  2. stochastic_walk_kernel: one workgroup per sequence.  Every input of
//     the walk is fetched in parallel first, on separate waves: each node's
//     row statistics (M, Z), the probability of its draft token at its
//     parent (after a sibling scan four threads per node) and its uniform.
//     One thread then walks the tree out of LDS.  The bonus draw
//     finds its chunk from the chunk masses (minus the rejected tokens) and
//     scans that chunk's logits, loaded with 16-byte loads, with a
//     workgroup prefix sum.
#include "tv_device.h"

#include <limits.h>

#include <type_traits>

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;  // 16-byte vectors of bf16 per thread per chunk (fp32: twice as many)
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWalkThreads = 1024;  // walk kernel: 16 waves, four per SIMD
constexpr int kWalkWaves = kWalkThreads / kWave;
constexpr int kPer = 16;    // tokens per walk thread in the bonus scan: chunk_len <= kWalkThreads * kPer

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

// ---- cross-lane helpers (DPP row ops and the gfx950 row swaps) ---------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

// every lane gets the wave's maximum
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0x128>(-INFINITY, x));
  x = fmaxf(x, dpp_f<0x124>(-INFINITY, x));
  x = fmaxf(x, dpp_f<0x122>(-INFINITY, x));
  x = fmaxf(x, dpp_f<0x121>(-INFINITY, x));
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}

// every lane gets the wave's sum (a fixed tree: the same order every call)
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0x128>(0.f, x);
  x += dpp_f<0x124>(0.f, x);
  x += dpp_f<0x122>(0.f, x);
  x += dpp_f<0x121>(0.f, x);
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// inclusive prefix sum over the wave (row_shr steps, then row_bcast 15 / 31)
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp_f<0x111>(0.f, v);
  v += dpp_f<0x112>(0.f, v);
  v += dpp_f<0x114>(0.f, v);
  v += dpp_f<0x118>(0.f, v);
  v += dpp_f<0x142, 0xA>(0.f, v);
  v += dpp_f<0x143, 0xC>(0.f, v);
  return v;
}

// ---- Philox-4x64-10 ----------------------------------------------------------------
// 128-bit product of two 64-bit words from four 32x32 -> 64 products
__device__ __forceinline__ void mul_64x64(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
  const uint64_t a0 = (uint32_t)a, a1 = a >> 32, b0 = (uint32_t)b, b1 = b >> 32;
  const uint64_t p00 = a0 * b0, p01 = a0 * b1, p10 = a1 * b0, p11 = a1 * b1;
  const uint64_t mid = (p00 >> 32) + (uint32_t)p01 + (uint32_t)p10;
  hi = p11 + (p01 >> 32) + (p10 >> 32) + (mid >> 32);
  lo = (mid << 32) | (uint32_t)p00;
}

// Round: with products M0*c0 and M1*c2 (128-bit), the new state is
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
// advances by the Weyl increments between rounds.
__device__ __forceinline__ uint64_t philox_first_word(uint64_t c0, uint64_t c1, uint64_t c2,
                                                      uint64_t c3, uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll 1
  for (int r = 0; r < 10; ++r) {  // rolled: this kernel's code runs once per call
    uint64_t hi0, lo0, hi1, lo1;
    mul_64x64(M0, c0, hi0, lo0);
    mul_64x64(M1, c2, hi1, lo1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return c0;
}

// uniform in [0, 1) from the 24 high bits (exact in fp32)
__device__ __forceinline__ float philox_uniform(uint64_t step, uint64_t seq, uint64_t node,
                                                uint64_t slot, uint64_t k0, uint64_t k1) {
  return (float)(uint32_t)(philox_first_word(step, seq, node, slot, k0, k1) >> 40) * 0x1.0p-24f;
}

// ---- kernel 0: the filter's threshold -------------------------------------------------
constexpr int kFiltThreads = 1024;
constexpr int kFiltWaves = kFiltThreads / kWave;
constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;
constexpr float kFix = 1099511627776.0f;  // 2^40: masses in fixed point
constexpr int kCand = 4096;                // top-k candidate list in LDS
constexpr int kSliceCand = 256;            // candidates kept per (row, slice)

// Order-preserving key of a logit: larger value, larger key; -0 and +0 share
// the key of +0 (they compare equal).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave 0 over a descending scan of the 2^bits bins: the largest bin d with
// above + sum(hist[d..]) >= target (target = frac * total when frac > 0),
// and the mass strictly above it (*s_sel = -1 when even the whole range
// falls short); *s_total gets the histogram's total.
__device__ void select_bin(const unsigned long long* hist, int nbins, unsigned long long above,
                           double target, double frac, int* s_sel,
                           unsigned long long* s_above, unsigned long long* s_total) {
  const int lane = threadIdx.x;  // wave 0 only
  // bins per lane (lane 0 the top ones); with fewer bins than lanes, one
  // bin per lane and the lanes past them empty
  const int per = nbins >= kWave ? nbins / kWave : 1;
  const int hi = nbins - 1 - lane * per;
  unsigned long long mine = 0;
  for (int j = 0; j < per && hi - j >= 0; ++j) mine += hist[hi - j];
  // inclusive scan in lane order (descending bins)
  unsigned long long incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const unsigned long long total = __shfl(incl, kWave - 1);
  if (lane == 0) *s_total = total;
  if (frac > 0.0) target = frac * (double)total;
  const bool cross = (double)(above + incl) >= target;
  const uint64_t ball = __ballot(cross);
  if (ball == 0) {
    if (lane == 0) {
      *s_sel = -1;
      *s_above = above + total;
    }
    return;
  }
  const int l = __builtin_ctzll(ball);
  if (lane == l) {
    unsigned long long run = above + incl - mine;
    int d = hi;
    for (int j = 0; j < per && hi - j >= 0; ++j) {
      d = hi - j;
      if ((double)(run + hist[d]) >= target) break;
      run += hist[d];
    }
    *s_sel = d;
    *s_above = run;
  }
}

// ---- kernel 0': the filter's threshold by radix selection spread over the row ------------
// The same selection as above (top-k by counts, then top-p by 2^-40 fixed-point
// masses), with every pass a launch of its own over (slice, row) workgroups:
// each builds its slice's histogram of the pass's digit in LDS and adds the
// nonzero bins into the row's histogram in global memory (integer atomics:
// the sums do not depend on their order).  At the start of the next pass
// every workgroup of the row derives the chosen bin from that histogram
// itself; the row's first workgroup records the state for the pass after.  A
// first launch takes the slice maxima (the masses are relative to the row
// maximum) and clears the row's histograms; the statistics kernel after the
// last pass turns the final state into tau.  Keys here map -0 and +0 to one key (2^31 plus the value's
// integer-ordered bits), so a threshold at zero keeps both.
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelVecs = 4;    // 16-byte vectors per thread and slice
constexpr int kSelPasses = 6;  // top-k digits, then top-p digits: 3 each at most

// A row's selection before one pass: the range of keys still searched is
// key & fixed == prefix.
struct SelState {
  uint32_t prefix, fixed;
  uint32_t tau_k;            // the top-k threshold key, once found (else 0)
  int32_t whole;             // top-p: the range holds less than the target, kept whole
  unsigned long long above;  // count or mass of the keys above the range
  double target;             // the count or mass the descending sum has to reach
};

struct SelArgs {
  const void* logits;
  int64_t vocab, row_stride;
  int slices;              // slices of kSelThreads * kSelVecs vectors per row
  int top_k, nk, np;       // nk / np: digits of the top-k / top-p selection (0: off)
  float top_p, c2;
  float* slice_max;          // [rows][slices]
  unsigned long long* hist;  // [rows][kSelPasses][kBins]
  SelState* state;           // [rows][kSelPasses]
  float* tau;                // [rows]
};

// order-preserving key of fp32 bits u: 2^31 + (u's sign-magnitude value as a
// two's complement integer), so that -0 and +0 share 2^31
__device__ __forceinline__ uint32_t sel_key(uint32_t u) {
  const uint32_t s = (uint32_t)((int32_t)u >> 31);
  return (u ^ (s | 0x80000000u)) - s;
}

__device__ __forceinline__ float sel_key_value(uint32_t k) {
  return __uint_as_float(k >= 0x80000000u ? k & 0x7FFFFFFFu : 0x80000000u | (0x80000000u - k));
}

// shift and width of digit d of the key, high digit first (bf16 values fill
// the top 16 bits of the key: two digits; fp32: three)
__device__ __forceinline__ void sel_digit(int key_bytes, int d, int& sh, int& width) {
  if (d == 0) {
    sh = 21;
    width = 11;
  } else if (key_bytes == 2) {
    sh = 16;
    width = 5;
  } else {
    sh = d == 1 ? 10 : 0;
    width = d == 1 ? 11 : 10;
  }
}

struct SelScratch {
  unsigned long long wsum[kSelWaves];
  unsigned long long above;
  float m[kSelWaves];
  int sel, cross;
};

// The largest bin d, in descending order, of the row's histogram h (nbins
// bins) with above + sum(h[d..]) >= target (target = frac * total when
// frac > 0): every thread gets it (-1 when even the whole range falls short),
// the sum above it and the histogram's total.  Thread t holds bins
// nbins - 1 - t * per down to nbins - t * per - per.
__device__ void block_select(const unsigned long long* __restrict__ h, int nbins,
                             unsigned long long above, double target, double frac,
                             SelScratch& sc, int& sel, unsigned long long& above_out,
                             unsigned long long& total) {
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int per = nbins >= kSelThreads ? nbins / kSelThreads : 1;  // at most 8
  const int hi = nbins - 1 - t * per;
  unsigned long long v[8], mine = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = hi - j;
    const unsigned long long x = h[k > 0 ? k : 0];  // in bounds for every thread
    v[j] = j < per && k >= 0 ? x : 0ull;
    mine += v[j];
  }
  unsigned long long incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) sc.wsum[wave] = incl;
  if (t == 0) sc.cross = kSelThreads;
  __syncthreads();
  unsigned long long tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    incl += w < wave ? sc.wsum[w] : 0ull;
    tot += sc.wsum[w];
  }
  if (frac > 0.0) target = frac * (double)tot;
  const uint64_t ball = __ballot((double)(above + incl) >= target);
  if (ball && lane == __builtin_ctzll(ball)) atomicMin(&sc.cross, t);
  __syncthreads();
  const int ct = sc.cross;
  if (t == ct) {
    unsigned long long run = above + incl - mine;
    int d = hi;
    bool done = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!done && j < per && hi - j >= 0) {
        d = hi - j;
        if ((double)(run + v[j]) >= target)
          done = true;
        else
          run += v[j];
      }
    }
    sc.sel = d;
    sc.above = run;
  } else if (ct == kSelThreads && t == 0) {
    sc.sel = -1;
    sc.above = above + tot;
  }
  __syncthreads();
  sel = sc.sel;
  above_out = sc.above;
  total = tot;
  __syncthreads();  // sc may be written again
}

// The state after pass q (top-k digits first, then top-p digits) from the
// state before it and the pass's histogram.
__device__ SelState sel_advance(const SelArgs& a, int key_bytes, SelState st,
                                const unsigned long long* __restrict__ h, int q,
                                SelScratch& sc) {
  const bool mass = q >= a.nk;
  const int d = mass ? q - a.nk : q;
  int sh, width;
  sel_digit(key_bytes, d, sh, width);
  if (!(mass && st.whole)) {
    int sel;
    unsigned long long ab, total;
    block_select(h, 1 << width, st.above, mass ? st.target : (double)a.top_k,
                 mass && d == 0 ? (double)a.top_p : 0.0, sc, sel, ab, total);
    // the first top-p digit's histogram holds the whole kept mass
    if (mass && d == 0) st.target = (double)a.top_p * (double)total;
    if (sel < 0) {
      st.whole = 1;  // rounding: the range holds less than the target, keep it all
    } else {
      st.prefix |= (uint32_t)sel << sh;
      st.fixed |= (uint32_t)((1 << width) - 1) << sh;
      st.above = ab;
    }
  }
  if (!mass && d == a.nk - 1) {
    // the k-th largest key found: top-p starts over on the keys at or above it
    st.tau_k = st.prefix;
    st.prefix = st.fixed = 0u;
    st.whole = 0;
    st.above = 0ull;
    st.target = 0.0;
  }
  return st;
}

// A slice's elements as fp32 bits, one 16-byte vector per (i, thread): vector
// i of thread t starts at element lo + (i * kSelThreads + t) * VEC.  Vectors
// past the slice's last whole vector read the slice's first one (in bounds)
// and are masked by the caller; the partial vector at the row's end, if
// any, is left to sel_tail.
template <typename T, bool kVector>
struct SelSlice {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int kWords = 16 / 4;
  uint32_t w[kSelVecs][kWords];
  int lo, hi, hi_full;  // [lo, hi): the slice; [lo, hi_full): its whole vectors

  __device__ __forceinline__ void load(const T* __restrict__ src, int64_t vocab, int s) {
    constexpr int cap = kSelThreads * kSelVecs * VEC;
    lo = s * cap;
    hi = (int)(vocab - lo < cap ? vocab - lo : cap) + lo;
    hi_full = kVector ? lo + (hi - lo) / VEC * VEC : lo;
#pragma unroll
    for (int i = 0; i < kSelVecs; ++i) {
      const int k0 = lo + (i * kSelThreads + (int)threadIdx.x) * VEC;
      const int kc = k0 + VEC <= hi_full ? k0 : lo;
      if (kVector && hi_full > lo) {
        const uint4 x = *reinterpret_cast<const uint4*>(src + kc);
        w[i][0] = x.x;
        w[i][1] = x.y;
        w[i][2] = x.z;
        w[i][3] = x.w;
      }
    }
  }
  // element e of vector i as fp32 bits
  __device__ __forceinline__ uint32_t bits(int i, int e) const {
    if (sizeof(T) == 2) {
      const uint32_t x = w[i][e / 2];
      return e % 2 == 0 ? x << 16 : x & 0xFFFF0000u;
    }
    return w[i][e];
  }
  __device__ __forceinline__ bool whole(int i) const {
    return lo + (i * kSelThreads + (int)threadIdx.x) * VEC + VEC <= hi_full;
  }
};

__device__ __forceinline__ uint32_t elem_bits(bf16 x) {
  return (uint32_t)__builtin_bit_cast(unsigned short, x) << 16;
}
__device__ __forceinline__ uint32_t elem_bits(float x) { return __float_as_uint(x); }

// f(bits) for the elements of [from, hi) one lane at a time: the partial
// vector at the row's end, or a whole slice of a row read element-wise
template <typename T, typename F>
__device__ __forceinline__ void sel_tail(const T* __restrict__ src, int from, int hi, F&& f) {
  for (int k = from + (int)threadIdx.x; k < hi; k += kSelThreads) f(elem_bits(src[k]));
}

// the row maximum from its slice maxima, for every thread
__device__ __forceinline__ float sel_row_max(const SelArgs& a, int64_t row, SelScratch& sc) {
  float m = -INFINITY;
  for (int i = (int)threadIdx.x; i < a.slices; i += kSelThreads)
    m = fmaxf(m, a.slice_max[row * a.slices + i]);
  m = wave_max(m);
  if (threadIdx.x % kWave == 0) sc.m[threadIdx.x / kWave] = m;
  __syncthreads();
  m = sc.m[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) m = fmaxf(m, sc.m[w]);
  return m;
}

// first launch: the slice maxima (for top-p) and cleared histograms
template <typename T, bool kVector>
__global__ __launch_bounds__(kSelThreads) void sel_start_kernel(SelArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float s_red[kSelWaves];
  const int s = blockIdx.x, t = threadIdx.x;
  const int64_t row = blockIdx.y;
  // the row's histograms of the passes to come, cleared by its workgroups in turn
  const int words = (a.nk + a.np) * kBins;
  const int per = (words + a.slices - 1) / a.slices;
  unsigned long long* h = a.hist + row * kSelPasses * kBins;
  for (int i = s * per + t; i < min(words, s * per + per); i += kSelThreads) h[i] = 0ull;
  if (a.np == 0) return;  // uniform: counts need no maximum
  const T* src = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;
  SelSlice<T, kVector> sl;
  sl.load(src, a.vocab, s);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSelVecs; ++i) {
    const bool ok = sl.whole(i);
#pragma unroll
    for (int e = 0; e < VEC; ++e) m = fmaxf(m, ok ? __uint_as_float(sl.bits(i, e)) : -INFINITY);
  }
  sel_tail(src, sl.hi_full, sl.hi, [&](uint32_t u) { m = fmaxf(m, __uint_as_float(u)); });
  m = wave_max(m);
  if (t % kWave == 0) s_red[t / kWave] = m;
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < kSelWaves; ++w) m = fmaxf(m, s_red[w]);
    a.slice_max[row * a.slices + s] = fmaxf(m, s_red[0]);
  }
}

// pass g: the histogram of its digit over the keys still in range (counts
// for a top-k digit, masses for a top-p one)
template <typename T, bool kVector, bool kMass>
__global__ __launch_bounds__(kSelThreads) void sel_pass_kernel(SelArgs a, int g) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ unsigned long long hist[kBins];  // counts: the first kBins words as uint32
  __shared__ SelScratch sc;
  const int s = blockIdx.x, t = threadIdx.x;
  const int64_t row = blockIdx.y;
  const T* src = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;
  // the elements first: the state below does not depend on them
  SelSlice<T, kVector> sl;
  sl.load(src, a.vocab, s);
  for (int i = t; i < kBins; i += kSelThreads) hist[i] = 0ull;
  SelState st{0u, 0u, 0u, 0, 0ull, 0.0};
  if (g > 0)
    st = sel_advance(a, (int)sizeof(T), a.state[row * kSelPasses + g - 1],
                     a.hist + (row * kSelPasses + g - 1) * kBins, g - 1, sc);
  if (s == 0 && t == 0) a.state[row * kSelPasses + g] = st;
  if (kMass && st.whole) return;  // uniform over the workgroup
  // log2 of an element's fixed-point mass: l c2 + (40 - M c2)
  const float base = kMass ? 40.f - sel_row_max(a, row, sc) * a.c2 : 0.f;
  if (!kMass) __syncthreads();  // the cleared histogram (sel_row_max's barrier otherwise)
  int sh, width;
  sel_digit((int)sizeof(T), kMass ? g - a.nk : g, sh, width);
  const uint32_t mask = (1u << width) - 1u;
  uint32_t* hist32 = reinterpret_cast<uint32_t*>(hist);
  const uint32_t fixed = st.fixed, prefix = st.prefix, tau_k = st.tau_k;
  const float c2 = a.c2;
  auto add = [&](uint32_t u, auto first) {
    const uint32_t key = sel_key(u);
    if (!decltype(first)::value && (key & fixed) != prefix) return;
    const uint32_t bin = (key >> sh) & mask;
    if (kMass) {
      // 2^40 exp2((l - M) c2) as an integer: high and low 32-bit halves
      const float w = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(u), c2, base));
      if (key < tau_k || !(w >= 1.f)) return;
      const uint32_t h32 = (uint32_t)(w * 0x1p-32f);
      const uint32_t l32 = (uint32_t)fmaf((float)h32, -0x1p32f, w);
      atomicAdd(&hist[bin], ((unsigned long long)h32 << 32) | l32);
    } else {
      atomicAdd(&hist32[bin], 1u);
    }
  };
  auto run = [&](auto first) {
#pragma unroll
    for (int i = 0; i < kSelVecs; ++i) {
      const bool ok = sl.whole(i);
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (ok) add(sl.bits(i, e), first);
    }
    sel_tail(src, sl.hi_full, sl.hi, [&](uint32_t u) { add(u, first); });
  };
  if (fixed == 0u)
    run(std::true_type{});
  else
    run(std::false_type{});
  __syncthreads();
  unsigned long long* gh = a.hist + (row * kSelPasses + g) * kBins;
  for (int i = t; i <= (int)mask; i += kSelThreads) {
    const unsigned long long c = kMass ? hist[i] : hist32[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// ---- top-k of at most kCandMaxK: candidates per slice, then one workgroup per row ----
// cand_collect_kernel, over the same (slice, row) grid as the spread
// selection: the slice's elements at or above the top_k-th largest of its
// threads' maxima (top_k threads hold an element at or above it, so the
// slice's top-k, and with them the row's top-k elements of the slice, are
// among them), at most kSliceCand of them (the count says when there were
// more), and the slice maximum.  filter_threshold_kernel then takes the k-th
// largest of the row's candidates (one per thread) and top-p among the keys
// at or above it in one wave.
constexpr int kCandMaxK = 32;  // largest top_k taking this path

// The k-th largest of the keys the workgroup's NT threads hold (key valid
// where ok), by radix selection over 8-bit digits from the top, counts in an
// LDS histogram of 256 bins (hist); digits below bit `low` are not looked at
// (bf16 keys have 16 zero low bits).  Every thread gets the key.
struct KthScratch {
  uint32_t hist[256];
  int sel, need;
};

template <int NT>
__device__ uint32_t block_kth_key(uint32_t key, bool ok, int k, int low, KthScratch& sc) {
  const int t = threadIdx.x, lane = t % kWave;
  uint32_t prefix = 0u, fixed = 0u;
  int need = k;  // the rank still looked for inside the current range
  for (int sh = 24; sh >= low; sh -= 8) {
    for (int i = t; i < 256; i += NT) sc.hist[i] = 0u;
    __syncthreads();
    if (ok && (key & fixed) == prefix) atomicAdd(&sc.hist[(key >> sh) & 255u], 1u);
    __syncthreads();
    if (t < kWave) {
      // lane l holds bins 255 - 4l down to 252 - 4l; a descending inclusive scan
      uint32_t h[4], mine = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = sc.hist[255 - 4 * lane - j];
        mine += h[j];
      }
      uint32_t incl = mine;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const uint64_t b = __ballot((int)incl >= need);  // some lane crosses: need <= count
      if (lane == (b ? __builtin_ctzll(b) : kWave - 1)) {
        int run = (int)(incl - mine), d = 255 - 4 * lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run + (int)h[j] >= need) {
            d = 255 - 4 * lane - j;
            break;
          }
          run += (int)h[j];
        }
        sc.sel = d;
        sc.need = need - run;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sc.sel << sh;
    fixed |= 255u << sh;
    need = sc.need;
    __syncthreads();  // sc is written again in the next round
  }
  return prefix;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(x, off);
    x = o > x ? o : x;
  }
  return x;
}

// 2^40 exp2((l - M) c2) as an integer, from y = l c2 + 40 - M c2 (0 below 1)
__device__ __forceinline__ unsigned long long fixed_mass(float y) {
  const float w = __builtin_amdgcn_exp2f(y);
  if (!(w >= 1.f)) return 0ull;
  const uint32_t h32 = (uint32_t)(w * 0x1p-32f);
  const uint32_t l32 = (uint32_t)fmaf((float)h32, -0x1p32f, w);
  return ((unsigned long long)h32 << 32) | l32;
}

template <typename T, bool kVector>
__global__ __launch_bounds__(kSelThreads) void cand_collect_kernel(
    const T* __restrict__ logits, int64_t vocab, int64_t row_stride, int top_k, int slices,
    uint32_t* __restrict__ cand_keys, int* __restrict__ cand_count, float* __restrict__ slice_max) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int kLow = sizeof(T) == 2 ? 16 : 0;
  __shared__ uint32_t s_cand[kSliceCand];
  __shared__ uint32_t s_max[kSelWaves];
  __shared__ KthScratch ks;
  __shared__ int s_n;
  const int s = blockIdx.x, t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int64_t row = blockIdx.y;
  const T* src = reinterpret_cast<const T*>(logits) + row * row_stride;
  SelSlice<T, kVector> sl;
  sl.load(src, vocab, s);
  uint32_t mk = 0u;
#pragma unroll
  for (int i = 0; i < kSelVecs; ++i) {
    const bool ok = sl.whole(i);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const uint32_t key = sel_key(sl.bits(i, e));
      mk = ok && key > mk ? key : mk;
    }
  }
  sel_tail(src, sl.hi_full, sl.hi, [&](uint32_t u) {
    const uint32_t key = sel_key(u);
    mk = key > mk ? key : mk;
  });
  if (t == 0) s_n = 0;
  {
    const uint32_t mx = wave_max_u32(mk);
    if (lane == 0) s_max[wave] = mx;
  }
  // the bound: the top_k-th largest of the threads' largest keys (threads
  // without an element hold 0, below every key)
  const uint32_t lower = block_kth_key<kSelThreads>(mk, true, top_k, kLow, ks);
  // one LDS atomic per wave and element slot that has candidates
  auto push = [&](uint32_t key, bool take) {
    const uint64_t b = __ballot(take);
    if (b) {
      const int leader = __builtin_ctzll(b);
      int base = 0;
      if (lane == leader) base = atomicAdd(&s_n, __builtin_popcountll(b));
      base = __shfl(base, leader);
      const int i = base + __builtin_popcountll(b & ((1ull << lane) - 1ull));
      if (take && i < kSliceCand) s_cand[i] = key;
    }
  };
#pragma unroll
  for (int i = 0; i < kSelVecs; ++i) {
    const bool ok = sl.whole(i);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const uint32_t key = sel_key(sl.bits(i, e));
      push(key, ok && key >= lower);
    }
  }
  sel_tail(src, sl.hi_full, sl.hi, [&](uint32_t u) {
    const uint32_t key = sel_key(u);
    push(key, key >= lower);
  });
  __syncthreads();
  const int n = s_n;
  const int64_t q = row * slices + s;
  for (int i = t; i < min(n, kSliceCand); i += kSelThreads) cand_keys[q * kSliceCand + i] = s_cand[i];
  if (t == 0) {
    uint32_t mx = s_max[0];
#pragma unroll
    for (int w = 1; w < kSelWaves; ++w) mx = s_max[w] > mx ? s_max[w] : mx;
    cand_count[q] = n;
    slice_max[q] = mx ? sel_key_value(mx) : -INFINITY;
  }
}

// Top-p among the candidates at or above tau_k (wave 0): the kept keys are
// packed into kk with their 2^-40 fixed-point masses in kw; each lane takes
// some of them and sums the masses of the kept keys at or above its own; the
// threshold is the largest key whose sum reaches top_p of the kept mass.
__device__ uint32_t wave_top_p_key(const uint32_t* cand, int n, uint32_t tau_k, float M,
                                   float top_p, float c2, uint32_t* kk,
                                   unsigned long long* kw) {
  const int lane = threadIdx.x % kWave;
  const float base = 40.f - M * c2;
  int nk = 0;
  unsigned long long tot = 0ull;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + lane;
    const uint32_t key = i < n ? cand[i] : 0u;
    const bool kp = i < n && key >= tau_k;
    const uint64_t b = __ballot(kp);
    if (kp) {
      const int j = nk + __builtin_popcountll(b & ((1ull << lane) - 1ull));
      const unsigned long long w = fixed_mass(fmaf(sel_key_value(key), c2, base));
      kk[j] = key;
      kw[j] = w;
      tot += w;
    }
    nk += __builtin_popcountll(b);
  }
  const double target = (double)top_p * (double)wave_sum_u64(tot);
  uint32_t best = 0u;
  for (int i = lane; i < nk; i += kWave) {
    const uint32_t key = kk[i];
    unsigned long long cum = 0ull;
#pragma unroll 4
    for (int j = 0; j < nk; ++j) cum += kk[j] >= key ? kw[j] : 0ull;
    if ((double)cum >= target && key > best) best = key;
  }
  return wave_max_u32(best);
}

template <typename T, bool kVector>
__global__ __launch_bounds__(kFiltThreads) void filter_threshold_kernel(
    const T* __restrict__ logits, int64_t vocab, int64_t row_stride, int top_k, float top_p,
    float c2, float* __restrict__ tau, const uint32_t* __restrict__ cand_keys,
    const int* __restrict__ cand_count, const float* __restrict__ slice_max, int slices) {
  // One workgroup per row.  The candidates cand_collect_kernel left for the
  // row's slices go to LDS and wave 0 selects among them; when a slice had
  // more than kSliceCand (many ties) the whole search runs here over the row.
  constexpr int VEC = 16 / sizeof(T);
  __shared__ unsigned long long hist[kBins];
  __shared__ uint32_t c_key[kCand];  // candidates: the elements at or above a lower bound
  __shared__ float c_val[kCand];
  __shared__ int s_ncand;
  __shared__ float s_red[kFiltWaves];
  __shared__ int s_sel;
  __shared__ unsigned long long s_above, s_total;
  const int64_t row = blockIdx.x;
  const T* src = logits + row * row_stride;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int lo = 0, hi = (int)vocab;
  // Every value of the row this thread owns: elements k0 .. k0 + VEC - 1 for
  // k0 = (t + i * kFiltThreads) * VEC, read with 8 loads in flight per
  // thread (the row stays in L2 between passes).
  typedef T vec_t __attribute__((ext_vector_type(VEC)));
  constexpr int kBatch = 8;
  auto visit = [&](auto&& f) {
    for (int b0 = lo + t * VEC; b0 < hi; b0 += kBatch * kFiltThreads * VEC) {
      vec_t x[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int k0 = b0 + i * kFiltThreads * VEC;
        if (kVector && k0 + VEC <= hi) {
          x[i] = *reinterpret_cast<const vec_t*>(src + k0);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) x[i][e] = k0 + e < hi ? src[k0 + e] : (T)0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int k0 = b0 + i * kFiltThreads * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (k0 + e < hi) f(to_f32<T>(x[i][e]));
      }
    }
  };
  // digits of the key, high first: bf16 values fill the top 16 bits
  constexpr int kDigits = sizeof(T) == 2 ? 2 : 3;
  const int shifts[3] = {21, sizeof(T) == 2 ? 16 : 10, 0};
  const int widths[3] = {11, sizeof(T) == 2 ? 5 : 11, 10};

  auto clear = [&]() {
    for (int i = t; i < kBins; i += kFiltThreads) hist[i] = 0ull;
    __syncthreads();
  };
  // Element sources: f(key, value) for every element of the row, or of the
  // candidate list collected in LDS (below).
  auto row_src = [&](auto&& f) { visit([&](float v) { f(order_key(v), v); }); };
  auto cand_src = [&](auto&& f) {
    const int nc = s_ncand;
    for (int i = t; i < nc; i += kFiltThreads) f(c_key[i], c_val[i]);
  };

  float M = -INFINITY, m_t = -INFINITY;
  // ---- the slices' candidates: every wave reads the counts (lane = slice) ----
  {
    const int64_t r0 = row * slices;
    const int c = lane < slices ? cand_count[r0 + lane] : 0;
    const float sm = lane < slices ? slice_max[r0 + lane] : -INFINITY;
    int incl = c;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int n = __shfl(incl, kWave - 1);
    if (slices <= kWave && __ballot(c > kSliceCand) == 0 && n <= kFiltThreads) {  // uniform
      // slice q's candidates to c_key[off_q ..], off_q the counts before it
      for (int q = wave; q < slices; q += kFiltWaves) {
        const int cq = __shfl(c, q), oq = __shfl(incl - c, q);
        uint32_t k4[kSliceCand / kWave];
#pragma unroll
        for (int r = 0; r < kSliceCand / kWave; ++r)
          k4[r] = cand_keys[(r0 + q) * kSliceCand + lane + r * kWave];  // in the slice's block
#pragma unroll
        for (int r = 0; r < kSliceCand / kWave; ++r)
          if (lane + r * kWave < cq) c_key[oq + lane + r * kWave] = k4[r];
      }
      __syncthreads();
      constexpr int kLow = sizeof(T) == 2 ? 16 : 0;
      KthScratch& ks = *reinterpret_cast<KthScratch*>(hist);
      const uint32_t tk = block_kth_key<kFiltThreads>(t < n ? c_key[t] : 0u, t < n, top_k, kLow, ks);
      if (wave == 0) {
        uint32_t key = tk;
        if (top_p < 1.f) {
          const uint32_t tp = wave_top_p_key(c_key, n, tk, wave_max(sm), top_p, c2,
                                             reinterpret_cast<uint32_t*>(c_val),
                                             hist + kBins / 2);
          key = tp > tk ? tp : tk;
        }
        if (lane == 0) tau[row] = sel_key_value(key);
      }
      return;
    }
  }
  {
    // ---- the row's maximum, and each thread's own maximum ----
    visit([&](float v) { m_t = fmaxf(m_t, v); });
    const float wm = wave_max(m_t);
    if (lane == 0) s_red[wave] = wm;
    __syncthreads();
    M = s_red[0];
    for (int w = 1; w < kFiltWaves; ++w) M = fmaxf(M, s_red[w]);
  }

  // ---- top-k: the k-th largest key (ties at it are kept) ----
  // kth(src): the top_k-th largest of the keys src hands over (radix
  // selection, counts in LDS)
  auto kth = [&](auto&& src) -> uint32_t {
    uint32_t prefix = 0u, fixed = 0u;
    unsigned long long above = 0ull;
    for (int g = 0; g < kDigits; ++g) {
      const int sh = shifts[g], mask = (1 << widths[g]) - 1;
      clear();
      src([&](uint32_t key, float) {
        if ((key & fixed) == prefix) atomicAdd(&hist[(key >> sh) & mask], 1ull);
      });
      __syncthreads();
      if (wave == 0)
        select_bin(hist, mask + 1, above, (double)top_k, 0.0, &s_sel, &s_above, &s_total);
      __syncthreads();
      prefix |= (uint32_t)s_sel << sh;  // a count of >= top_k always exists
      fixed |= (uint32_t)mask << sh;
      above = s_above;
      __syncthreads();
    }
    return prefix;
  };
  uint32_t tau_k = 0u;
  bool use_cand = false;  // every key >= tau_k is in the candidate list
  if (top_k > 0 && (int64_t)top_k < vocab) {
    // A lower bound first: the top_k-th largest of the threads' maxima (top_k
    // threads hold an element at or above it, so the answer is at or above
    // it too).  The elements at or above it are few: they are collected
    // once into LDS, and the selections run on them instead of the row.
    uint32_t lower = 0u;
    if (top_k <= kFiltThreads) {
      const uint32_t mk = order_key(m_t);
      lower = kth([&](auto&& f) { f(mk, m_t); });
      if (t == 0) s_ncand = 0;
      __syncthreads();
      visit([&](float v) {
        const uint32_t key = order_key(v);
        const bool c = key >= lower;
        const uint64_t bal = __ballot(c);
        if (bal) {  // one atomic per wave and element slot
          const int leader = __builtin_ctzll(bal);
          int base = 0;
          if (lane == leader) base = atomicAdd(&s_ncand, __builtin_popcountll(bal));
          base = __shfl(base, leader);
          if (c) {
            const int i = base + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
            if (i < kCand) {
              c_key[i] = key;
              c_val[i] = v;
            }
          }
        }
      });
      __syncthreads();
      use_cand = s_ncand <= kCand;  // else (many ties) the row is used
      __syncthreads();
    }
    if (use_cand) {
      tau_k = kth(cand_src);
    } else {
      tau_k = kth([&](auto&& f) {
        row_src([&](uint32_t key, float v) {
          if (key >= lower) f(key, v);
        });
      });
    }
  }

  // ---- top-p: the last key (descending) whose strictly larger keys hold
  // less than top_p of the mass kept by top-k ----
  uint32_t tau_p = 0u;
  if (top_p < 1.f) {
    uint32_t prefix = 0u, fixed = 0u;
    unsigned long long above = 0ull;
    double target = 0.0;
    bool whole = false;  // every remaining key is kept
    auto pass = [&](auto&& src, int sh, int mask) {
      src([&](uint32_t key, float v) {
        if (key >= tau_k && (key & fixed) == prefix) {
          const unsigned long long w = (unsigned long long)(exp2f((v - M) * c2) * kFix);
          atomicAdd(&hist[(key >> sh) & mask], w);
        }
      });
    };
    for (int g = 0; g < kDigits && !whole; ++g) {
      const int sh = shifts[g], mask = (1 << widths[g]) - 1;
      clear();
      if (use_cand)
        pass(cand_src, sh, mask);
      else
        pass(row_src, sh, mask);
      __syncthreads();
      // the first digit's histogram holds the whole kept mass: target = top_p * it
      if (wave == 0)
        select_bin(hist, mask + 1, above, target, g == 0 ? (double)top_p : 0.0, &s_sel, &s_above,
                   &s_total);
      __syncthreads();
      if (g == 0) target = (double)top_p * (double)s_total;
      if (s_sel < 0) {
        whole = true;  // rounding: the range holds less than the target, keep it all
      } else {
        prefix |= (uint32_t)s_sel << sh;
        fixed |= (uint32_t)mask << sh;
        above = s_above;
      }
      __syncthreads();
    }
    tau_p = prefix;
  }
  if (t == 0) {
    const bool any = (top_k > 0 && (int64_t)top_k < vocab) || top_p < 1.f;
    tau[row] = any ? key_value(tau_k > tau_p ? tau_k : tau_p) : -INFINITY;
  }
}

// ---- kernel 1: per-chunk softmax statistics ---------------------------------------------
// Vector u of thread t covers elements begin + (u * kThreads + t) * VEC ..
// +VEC-1.  Every vector load is issued unconditionally (vectors past the
// chunk's last whole one re-read its first and are masked), so all of them
// are in flight together; the partial vector at the row's end is read
// element-wise afterwards.  With kDerive the workgroup first turns the
// spread selection's last histogram into the row's threshold (the chunk-0
// workgroup records it for the walk).
template <typename T, bool kVector, bool kDerive>
__global__ __launch_bounds__(kThreads) void softmax_stats_kernel(const T* __restrict__ logits,
                                                                 int64_t vocab, int64_t row_stride,
                                                                 int64_t chunk_len, int chunks,
                                                                 float c2, float* __restrict__ tau,
                                                                 float2* __restrict__ stats,
                                                                 SelArgs sel) {
  static_assert(kThreads == kSelThreads, "one selection per workgroup");
  constexpr int VEC = 16 / sizeof(T);
  constexpr int U = kUnroll * 8 / VEC;
  __shared__ float s_red[kWaves];
  __shared__ SelScratch sc;
  const int chunk = blockIdx.x, t = threadIdx.x;
  const int64_t row = blockIdx.y;
  const T* src = logits + row * row_stride;
  const int64_t begin = (int64_t)chunk * chunk_len;
  const int64_t end = begin + chunk_len < vocab ? begin + chunk_len : vocab;
  const int64_t end_full = kVector ? begin + (end - begin) / VEC * VEC : begin;
  const int lane = t % kWave, wave = t / kWave;

  uint4 x[U];
  if (kVector && end_full > begin) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t base = begin + ((int64_t)u * kThreads + t) * VEC;
      x[u] = *reinterpret_cast<const uint4*>(src + (base + VEC <= end_full ? base : begin));
    }
  }
  // element e of vector u as a float (-inf past the whole vectors)
  auto val = [&](int u, int e) -> float {
    const int64_t base = begin + ((int64_t)u * kThreads + t) * VEC;
    uint32_t b;
    if (sizeof(T) == 2) {
      const uint32_t w = (&x[u].x)[e / 2];
      b = e % 2 == 0 ? w << 16 : w & 0xFFFF0000u;
    } else {
      b = (&x[u].x)[e];
    }
    return base + VEC <= end_full ? __uint_as_float(b) : -INFINITY;
  };
  float lo = -INFINITY;  // kept: l >= lo
  if (kDerive) {
    const int q = sel.nk + sel.np - 1;
    const SelState st = sel_advance(sel, (int)sizeof(T), sel.state[row * kSelPasses + q],
                                    sel.hist + (row * kSelPasses + q) * kBins, q, sc);
    lo = sel_key_value(sel.np > 0 && st.prefix > st.tau_k ? st.prefix : st.tau_k);
    if (chunk == 0 && t == 0) tau[row] = lo;
  } else if (tau) {
    lo = tau[row];
  }
  // the elements read one at a time: [end_full, end), at most one per thread
  // for whole-vector rows
  const int64_t kt = end_full + t;
  float tail = -INFINITY;
  for (int64_t k = kt; k < end; k += kThreads) tail = fmaxf(tail, to_f32<T>(src[k]));
  const bool has_tail = kt < end && end - end_full <= kThreads;

  float m = tail;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < VEC; ++e) m = fmaxf(m, val(u, e));
  m = wave_max(m);
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = s_red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_red[w]);
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float v = val(u, e);
      s += v >= lo ? __builtin_amdgcn_exp2f((v - m) * c2) : 0.f;  // -inf -> 0
    }
  if (has_tail) {
    s += tail >= lo ? __builtin_amdgcn_exp2f((tail - m) * c2) : 0.f;
  } else {
    // element-wise rows (or a tail longer than a workgroup): the rest in order
    for (int64_t k = kt; k < end; k += kThreads) {
      const float v = to_f32<T>(src[k]);
      s += v >= lo ? __builtin_amdgcn_exp2f((v - m) * c2) : 0.f;
    }
  }
  if (m == -INFINITY) s = 0.f;  // no finite logit: (l - m) would be NaN
  s = wave_sum(s);
  if (lane == 0) s_red[wave] = s;
  __syncthreads();
  if (t == 0) {
    float sum = s_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += s_red[w];
    stats[row * chunks + chunk] = make_float2(m, sum);
  }
}

// ---- kernel 2: the walk ------------------------------------------------------------------
struct WalkArgs {
  const void* logits;
  int64_t vocab, row_stride, chunk_len;
  int chunks;
  float c2;
  const float2* stats;
  const float* tau;  // per row: the filter's threshold, or null (no filter)
  const int32_t* parents;
  const int32_t* draft;
  int n;
  uint64_t k0, k1, step;
  int32_t* accept_len;
  int32_t* accept_path;
  int32_t* bonus;
  int32_t* dev_err;
};

// kPer logits from..from+kPer-1 of one row as floats (-inf past `to`);
// 16-byte loads when the span is whole and aligned
template <typename T, bool kVector>
__device__ __forceinline__ void load_span(const T* row, int64_t from, int64_t to,
                                          float (&q)[kPer]) {
  constexpr int VEC = 16 / sizeof(T);
  if (kVector && from + kPer <= to) {
    typedef T vec_t __attribute__((ext_vector_type(VEC)));
    vec_t x[kPer / VEC];
#pragma unroll
    for (int u = 0; u < kPer / VEC; ++u) x[u] = *reinterpret_cast<const vec_t*>(row + from + u * VEC);
#pragma unroll
    for (int u = 0; u < kPer / VEC; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[u * VEC + e] = to_f32<T>(x[u][e]);
  } else {
    // ragged or unaligned: clamped addresses keep every load in bounds and
    // branch-free, so all of them are in flight together
    const int64_t last = to - 1;
#pragma unroll
    for (int e = 0; e < kPer; ++e) q[e] = to_f32<T>(row[from + e < to ? from + e : last]);
#pragma unroll
    for (int e = 0; e < kPer; ++e) q[e] = from + e < to ? q[e] : -INFINITY;
  }
}

template <typename T, bool kVector>
__global__ __launch_bounds__(kWalkThreads) void stochastic_walk_kernel(WalkArgs a) {
  __shared__ __attribute__((aligned(16))) int s_par[TV_MAX_NODES];
  __shared__ __attribute__((aligned(16))) int s_tok[TV_MAX_NODES];
  __shared__ int s_first[TV_MAX_NODES], s_next[TV_MAX_NODES], s_path[TV_MAX_NODES];
  __shared__ int s_rank[TV_MAX_NODES];  // node j: sibling rank, bit 30: its token repeats
  __shared__ float s_M[TV_MAX_NODES], s_Z[TV_MAX_NODES];  // row statistics of every node
  __shared__ float s_p[TV_MAX_NODES];  // node j: p_parent(token_j), 0 if invalid or repeated
  __shared__ float s_u[TV_MAX_NODES];  // node j: its acceptance uniform
  __shared__ float s_ub[TV_MAX_NODES]; // node j: the bonus uniform if the walk ends at j
  __shared__ int s_bad, s_depth, s_end, s_pick, s_last, s_chunk;
  __shared__ float s_target, s_before;
  __shared__ float s_wsum[kWalkWaves];

  const int b = blockIdx.x, t = threadIdx.x, n = a.n;
  const int lane = t % kWave, wave = t / kWave;
  const int64_t row0 = (int64_t)b * n;
  const T* logits = reinterpret_cast<const T*>(a.logits);
  if (t == 0) s_bad = 0;
  static_assert(kWalkThreads >= 4 * TV_MAX_NODES, "four thread slots per node");
  // Three jobs on three sets of waves, all started at once.  Threads t < n:
  // node t's parent and token to LDS, and the logit of its token in its
  // parent's row (with the parent's threshold) requested; threads 256 + j:
  // node j's row statistics (M, Z) from its chunk statistics; threads 512 + j:
  // node j's bonus uniform.
  float lraw = 0.f, lo_par = -INFINITY;
  int par = 0, tok = 0;
  if (t < TV_MAX_NODES) {
    if (t < n) {
      par = a.parents[row0 + t];
      tok = a.draft[row0 + t];
      s_first[t] = INT_MAX;
      const bool ok = t == 0 ? par == -1 : (par >= 0 && par < t);
      if (!ok) s_bad = 1;
      // clamped indices: the load is in bounds whatever the tree holds
      const int pc = t > 0 && par >= 0 && par < t ? par : 0;
      const int64_t tc = tok >= 0 && (int64_t)tok < a.vocab ? tok : 0;
      lraw = to_f32<T>(logits[(row0 + pc) * a.row_stride + tc]);
      if (a.tau) lo_par = a.tau[row0 + pc];
    }
    s_par[t] = t < n ? par : -2;  // slots past n match no parent
    s_tok[t] = tok;
  } else if (t < 2 * TV_MAX_NODES) {
    const int j = t - TV_MAX_NODES;
    if (j < n) {
      const float2* sr = a.stats + (row0 + j) * a.chunks;
      float2 st[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < a.chunks) st[c] = sr[c];
      float m = -INFINITY;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < a.chunks) m = fmaxf(m, st[c].x);
      for (int c = 8; c < a.chunks; ++c) m = fmaxf(m, sr[c].x);
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < a.chunks) z += st[c].y * exp2f((st[c].x - m) * a.c2);
      for (int c = 8; c < a.chunks; ++c) z += sr[c].y * exp2f((sr[c].x - m) * a.c2);
      s_M[j] = m;
      s_Z[j] = z;
    }
  } else if (t < 3 * TV_MAX_NODES) {
    const int j = t - 2 * TV_MAX_NODES;
    if (j < n) s_ub[j] = philox_uniform(a.step, (uint64_t)b, (uint64_t)j, ~0ull, a.k0, a.k1);
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  // Sibling links, rank and repeated tokens, four threads per node: thread
  // 4t + q scans the 16-slot blocks q, q + 4, ... of the tree (16-byte LDS
  // reads) for node t; the quad combines its counts and its first later
  // sibling.
  if (!bad && t < 4 * n) {
    const int nt = t >> 2, q = t & 3;
    const int pt = s_par[nt], kt = s_tok[nt];
    int nx = INT_MAX, rank = 0, rep = 0;
    if (nt > 0) {
      for (int j0 = 16 * q; j0 < n; j0 += 64) {
        int4 pp[4], tt[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          pp[q4] = *reinterpret_cast<const int4*>(&s_par[j0 + 4 * q4]);
          tt[q4] = *reinterpret_cast<const int4*>(&s_tok[j0 + 4 * q4]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = j0 + e;
          const int pj = e % 4 == 0 ? pp[e / 4].x : e % 4 == 1 ? pp[e / 4].y
                       : e % 4 == 2 ? pp[e / 4].z : pp[e / 4].w;
          const int tj = e % 4 == 0 ? tt[e / 4].x : e % 4 == 1 ? tt[e / 4].y
                       : e % 4 == 2 ? tt[e / 4].z : tt[e / 4].w;
          // arithmetic, not short-circuit logic: no branches per slot
          const int before = (pj == pt) & (j < nt);
          const int after = (pj == pt) & (j > nt);
          rank += before;
          rep |= before & (tj == kt);
          nx = min(nx, after ? j : INT_MAX);
        }
      }
    }
#pragma unroll
    for (int m = 1; m <= 2; m <<= 1) {
      rank += __shfl_xor(rank, m);
      rep |= __shfl_xor(rep, m);
      nx = min(nx, __shfl_xor(nx, m));
    }
    if (q == 0 && nt > 0) {
      atomicMin(&s_first[pt], nt);
      s_next[nt] = nx;
      s_rank[nt] = rank | (rep << 30);
    }
  }
  __syncthreads();
  // the probability of each node's token at its parent and its uniform
  if (t < n && t > 0 && !bad) {
    const int rr = s_rank[t];
    const int rank = rr & ((1 << 30) - 1);
    const bool repeated = (rr >> 30) != 0;
    const bool valid = tok >= 0 && (int64_t)tok < a.vocab && !repeated;
    s_p[t] = valid && lraw >= lo_par ? exp2f((lraw - s_M[par]) * a.c2) / s_Z[par] : 0.f;
    s_u[t] = philox_uniform(a.step, (uint64_t)b, (uint64_t)par, (uint64_t)rank, a.k0, a.k1);
  }
  __syncthreads();
  // the walk itself, from LDS
  if (t == 0) {
    int u = 0, depth = 0;
    float rest = 1.f;
    s_path[0] = 0;
    for (;;) {
      rest = 1.f;
      int next = -1;
      if (!bad)
        for (int c = s_first[u]; c != INT_MAX; c = s_next[c]) {
          if (s_u[c] * rest < s_p[c]) {
            next = c;
            break;
          }
          rest -= s_p[c];
        }
      if (next < 0) break;
      s_path[++depth] = next;
      u = next;
    }
    s_depth = depth;
    s_end = u;
    s_target = s_ub[u] * rest;
  }
  __syncthreads();

  // ---- bonus draw from the residual of the last node's row ----
  const int u = s_end;
  const int64_t row = row0 + u;
  const float M = s_M[u], Z = s_Z[u];
  const float inv_z = 1.f / Z;
  if (wave == 0) {
    // chunk masses minus the rejected children's tokens (lane = chunk), an
    // inclusive prefix in chunk order, and the first chunk whose prefix
    // passes the target
    const float target = s_target;
    float base = 0.f;
    int pick = -1, last_pos = 0;
    float before = 0.f;
    for (int c0 = 0; c0 < a.chunks && pick < 0; c0 += kWave) {
      const int c = c0 + lane;
      float w = 0.f;
      if (c < a.chunks) {
        const float2 sc = a.stats[row * a.chunks + c];
        w = sc.y * exp2f((sc.x - M) * a.c2) * inv_z;
        const int64_t lo = (int64_t)c * a.chunk_len, hi = lo + a.chunk_len;
        if (!bad)
          for (int k = s_first[u]; k != INT_MAX; k = s_next[k])
            if (s_p[k] > 0.f && s_tok[k] >= lo && s_tok[k] < hi) w -= s_p[k];
      }
      const float incl = base + wave_incl_scan(w);
      const uint64_t over = __ballot(c < a.chunks && incl > target);
      const uint64_t pos = __ballot(c < a.chunks && w > 0.f);
      if (pos) last_pos = c0 + 63 - __builtin_clzll(pos);
      if (over) {
        const int l = __builtin_ctzll(over);
        pick = c0 + l;
        before = __shfl(incl - w, l);
      }
      base = __shfl(incl, kWave - 1);
    }
    if (lane == 0) {
      if (pick < 0) {   // rounding left the target past the end: last chunk with mass,
        pick = last_pos;  // whose scan then never crosses and takes its last eligible token
        before = -INFINITY;
      }
      s_chunk = pick;
      s_before = before;
      s_pick = INT_MAX;
      s_last = -1;
    }
  }
  __syncthreads();
  const int64_t lo = (int64_t)s_chunk * a.chunk_len;
  const int64_t hi = lo + a.chunk_len < a.vocab ? lo + a.chunk_len : a.vocab;
  const int64_t my0 = lo + (int64_t)t * kPer;
  float q[kPer];
  load_span<T, kVector>(logits + row * a.row_stride, my0, hi, q);
  const float c2 = a.c2;
  const float lo_u = a.tau ? a.tau[row] : -INFINITY;
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    q[e] = my0 + e < hi && q[e] >= lo_u ? __builtin_amdgcn_exp2f((q[e] - M) * c2) * inv_z : 0.f;
  // rejected children's tokens leave the residual
  if (!bad)
    for (int k = s_first[u]; k != INT_MAX; k = s_next[k]) {
      const int64_t d = (int64_t)s_tok[k] - my0;
      if (s_p[k] > 0.f && d >= 0 && d < kPer) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) q[e] = e == d ? 0.f : q[e];
      }
    }
  float mine = 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) mine += q[e];
  // exclusive prefix of the threads' sums, in token order
  const float incl = wave_incl_scan(mine);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  float off = s_before;
#pragma unroll
  for (int w = 0; w < kWalkWaves; ++w) off += w < wave ? s_wsum[w] : 0.f;
  const float target = s_target;
  // the running sum never decreases, so the first token whose running sum
  // passes the target comes after exactly `le` tokens whose sum does not
  float run = off + incl - mine;
  int le = 0, last_e = -1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    run += q[e];
    le += run <= target ? 1 : 0;
    last_e = q[e] > 0.f ? e : last_e;
  }
  const int found = le < kPer ? (int)(my0 + le) : INT_MAX;
  const int last_ok = last_e >= 0 ? (int)(my0 + last_e) : -1;
  // both are monotone in thread order: one lane per wave reports
  const uint64_t fb = __ballot(found != INT_MAX);
  if (fb && lane == __builtin_ctzll(fb)) atomicMin(&s_pick, found);
  const uint64_t lb = __ballot(last_ok >= 0);
  if (lb && lane == 63 - __builtin_clzll(lb)) atomicMax(&s_last, last_ok);
  __syncthreads();
  if (t == 0) {
    int y = s_pick;
    if (y == INT_MAX) y = s_last;  // rounding: the last eligible token of the chunk
    if (y < 0) y = 0;              // nothing eligible at all (cannot happen for R > 0)
    a.accept_len[b] = s_depth;
    a.bonus[b] = y;
    if (bad) raise_err(a.dev_err, TV_DERR_BAD_PARENT);
  }
  int32_t* path = a.accept_path + row0;
  if (t < n) path[t] = t <= s_depth ? s_path[t] : -1;
}

}  // namespace

namespace {

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// slices per row of the spread selection: up to kSelVecs vectors per thread
int sel_slices(int64_t vocab, size_t elem) {
  const int64_t cap = (int64_t)kSelThreads * kSelVecs * (int64_t)(16 / elem);
  return (int)((vocab + cap - 1) / cap);
}

// workspace: chunk statistics, thresholds, the slices' top-k candidates,
// then the spread selection's slice maxima, histograms and states
int sel_slices_max(int64_t vocab) { return sel_slices(vocab, sizeof(float)); }

size_t sel_offset(size_t rows, int chunks, int64_t vocab) {
  return round256(rows * chunks * sizeof(float2)) + round256(rows * sizeof(float)) +
         round256(rows * sel_slices_max(vocab) *
                  (kSliceCand * sizeof(uint32_t) + sizeof(int) + sizeof(float)));
}

}  // namespace

AcceptPlan plan_stochastic(int batch, int n, int64_t vocab) {
  AcceptPlan p;
  const int64_t per_pass = (int64_t)kThreads * 8;
  int64_t chunk = per_pass * kUnroll;
  if (chunk > vocab) chunk = ((vocab + per_pass - 1) / per_pass) * per_pass;
  if (chunk < per_pass) chunk = per_pass;
  static_assert((int64_t)kThreads * 8 * kUnroll <= (int64_t)kWalkThreads * kPer, "bonus scan size");
  p.chunk_len = chunk;
  p.chunks = (int)((vocab + chunk - 1) / chunk);
  // chunk statistics, one threshold per row, then the slices' top-k candidates
  const size_t rows = (size_t)batch * n;
  p.ws_bytes = sel_offset(rows, p.chunks, vocab) +
               round256(rows * sel_slices(vocab, sizeof(float)) * sizeof(float)) +
               round256(rows * kSelPasses * kBins * sizeof(unsigned long long)) +
               rows * kSelPasses * sizeof(SelState);
  return p;
}

namespace {

template <typename T, bool kVector>
void launch_typed(const void* logits, int64_t vocab, int64_t row_stride, int batch, int n,
                  float c2, int top_k, float top_p, const AcceptPlan& plan, float2* stats,
                  float* tau, const WalkArgs& w, hipStream_t stream) {
  const unsigned rows = (unsigned)((size_t)batch * n);
  SelArgs sa{};
  bool derive = false;
  if (tau) {
    // the slices' candidate buffers follow the thresholds in the workspace
    const size_t smax = (size_t)sel_slices_max(vocab);
    char* base = reinterpret_cast<char*>(tau) + round256((size_t)rows * sizeof(float));
    uint32_t* cand_keys = reinterpret_cast<uint32_t*>(base);
    int* cand_count = reinterpret_cast<int*>(cand_keys + rows * smax * kSliceCand);
    float* slice_max = reinterpret_cast<float*>(cand_count + rows * smax);
    const int slices = sel_slices(vocab, sizeof(T));
    if (top_k > 0 && top_k <= kCandMaxK && (int64_t)top_k < vocab && slices <= kWave) {
      hipLaunchKernelGGL((cand_collect_kernel<T, kVector>), dim3(slices, rows), dim3(kSelThreads),
                         0, stream, (const T*)logits, vocab, row_stride, top_k, slices,
                         cand_keys, cand_count, slice_max);
      hipLaunchKernelGGL((filter_threshold_kernel<T, kVector>), dim3(rows), dim3(kFiltThreads), 0,
                         stream, (const T*)logits, vocab, row_stride, top_k, top_p, c2, tau,
                         cand_keys, cand_count, slice_max, slices);
    } else {
      // the spread selection
      constexpr int kDigits = sizeof(T) == 2 ? 2 : 3;
      sa.logits = logits;
      sa.vocab = vocab;
      sa.row_stride = row_stride;
      sa.slices = sel_slices(vocab, sizeof(T));
      sa.top_k = top_k;
      sa.nk = top_k > 0 && (int64_t)top_k < vocab ? kDigits : 0;
      sa.np = top_p < 1.f ? kDigits : 0;
      sa.top_p = top_p;
      sa.c2 = c2;
      char* sel = reinterpret_cast<char*>(stats) + sel_offset(rows, plan.chunks, vocab);
      sa.slice_max = reinterpret_cast<float*>(sel);
      sel += round256((size_t)rows * sel_slices(vocab, sizeof(float)) * sizeof(float));
      sa.hist = reinterpret_cast<unsigned long long*>(sel);
      sel += round256((size_t)rows * kSelPasses * kBins * sizeof(unsigned long long));
      sa.state = reinterpret_cast<SelState*>(sel);
      sa.tau = tau;
      const dim3 grid(sa.slices, rows);
      hipLaunchKernelGGL((sel_start_kernel<T, kVector>), grid, dim3(kSelThreads), 0, stream, sa);
      for (int g = 0; g < sa.nk + sa.np; ++g) {
        if (g < sa.nk)
          hipLaunchKernelGGL((sel_pass_kernel<T, kVector, false>), grid, dim3(kSelThreads), 0,
                             stream, sa, g);
        else
          hipLaunchKernelGGL((sel_pass_kernel<T, kVector, true>), grid, dim3(kSelThreads), 0,
                             stream, sa, g);
      }
      derive = true;  // the stats kernel takes tau from the last histogram
    }
  }
  if (derive)
    hipLaunchKernelGGL((softmax_stats_kernel<T, kVector, true>), dim3(plan.chunks, rows),
                       dim3(kThreads), 0, stream, (const T*)logits, vocab, row_stride,
                       plan.chunk_len, plan.chunks, c2, tau, stats, sa);
  else
    hipLaunchKernelGGL((softmax_stats_kernel<T, kVector, false>), dim3(plan.chunks, rows),
                       dim3(kThreads), 0, stream, (const T*)logits, vocab, row_stride,
                       plan.chunk_len, plan.chunks, c2, tau, stats, sa);
  hipLaunchKernelGGL((stochastic_walk_kernel<T, kVector>), dim3(batch), dim3(kWalkThreads), 0,
                     stream, w);
}

}  // namespace

hipError_t launch_stochastic(const void* logits, tv_dtype dt, int64_t vocab, int64_t row_stride,
                             const int32_t* parents, const int32_t* draft, int batch, int n,
                             float temperature, int top_k, float top_p, uint64_t seed0,
                             uint64_t seed1, uint64_t step, int32_t* accept_len,
                             int32_t* accept_path, int32_t* bonus, void* workspace,
                             const AcceptPlan& plan, int32_t* dev_err, hipStream_t stream) {
  const size_t rows = (size_t)batch * n;
  float2* stats = reinterpret_cast<float2*>(workspace);
  const bool filtered = (top_k > 0 && (int64_t)top_k < vocab) || top_p < 1.f;
  float* tau = filtered ? reinterpret_cast<float*>(
                              reinterpret_cast<char*>(workspace) +
                              ((rows * plan.chunks * sizeof(float2) + 255) / 256) * 256)
                        : nullptr;
  const float c2 = kLog2e / temperature;
  WalkArgs w{};
  w.logits = logits;
  w.vocab = vocab;
  w.row_stride = row_stride;
  w.chunk_len = plan.chunk_len;
  w.chunks = plan.chunks;
  w.c2 = c2;
  w.stats = stats;
  w.tau = tau;
  w.parents = parents;
  w.draft = draft;
  w.n = n;
  w.k0 = seed0;
  w.k1 = seed1;
  w.step = step;
  w.accept_len = accept_len;
  w.accept_path = accept_path;
  w.bonus = bonus;
  w.dev_err = dev_err;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(logits);
  if (dt == TV_BF16) {
    if ((addr % 16 == 0) && (row_stride % 8 == 0))
      launch_typed<bf16, true>(logits, vocab, row_stride, batch, n, c2, top_k, top_p, plan, stats,
                               tau, w, stream);
    else
      launch_typed<bf16, false>(logits, vocab, row_stride, batch, n, c2, top_k, top_p, plan,
                                stats, tau, w, stream);
  } else {
    if ((addr % 16 == 0) && (row_stride % 4 == 0))
      launch_typed<float, true>(logits, vocab, row_stride, batch, n, c2, top_k, top_p, plan,
                                stats, tau, w, stream);
    else
      launch_typed<float, false>(logits, vocab, row_stride, batch, n, c2, top_k, top_p, plan,
                                 stats, tau, w, stream);
  }
  return hipGetLastError();
}

}  // namespace tv
