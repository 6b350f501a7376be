// Tree-masked GQA attention, 32-row schedule (see the file comment of
// tv_attention.hip for the computation and the partial format).
//
// Built with VGPR-form MFMAs (-mllvm -amdgpu-mfma-vgpr-form): the score tiles
// the softmax reads and the output accumulators stay in the VGPR file and
// the Q^T operand is pinned to the accumulation registers, so the hot loop
// moves nothing between the two register files.
#include "tv_attn_common.h"

#include <algorithm>
#include <type_traits>

namespace tv {
namespace attn {
namespace {

// ---- wide kernel: one wave per SIMD, 64 rows per wave, 32x32x16 MFMA ----------
//
// A second schedule of the same computation for long prefixes.  Four waves
// (one per SIMD) each own RT tiles of 32 query rows, so a workgroup holds up
// to 128 RT rows of its kv head and every K/V tile read from LDS feeds 32 RT
// rows per wave: half the LDS operand bytes per MFMA of the 16-row kernel
// (tv_attention.hip).  v_mfma_f32_32x32x16_bf16 reaches the matrix-core rate from a
// single wave (two independent accumulator chains suffice), which the
// 16x16x32 shape does not, so the softmax of one tile and the QK^T products
// of the next share the wave's instruction stream instead of being split
// over two waves.  With S^T = K Q^T each lane holds one query row and 16
// tokens of a tile: tokens 8(r/4) + 4h + r%4 of register r, h = lane/32.
// The PV product O^T += V^T P^T takes its B operand straight from those
// registers -- P^T for tokens 16kt..16kt+15 is registers 8kt..8kt+7 in
// order -- when the V^T A operand lists the same tokens in the same
// k-slot order, which two transposing LDS reads per operand give.  Tiles
// stream HBM -> LDS by LDS DMA into a ring of kWRing slots, kWAhead tiles
// ahead of the one in use.
constexpr int kWWaves = 4;
constexpr int kWThreads = kWWaves * 64;
constexpr int kWRing = 8;   // LDS ring slots, a power of two
constexpr int kWAhead = 7;  // tiles requested ahead of the one in use (< kWRing)
// Tiles requested before the first step; the others follow two per step
// over the first kWAhead - kWFirst steps.  All workgroups start at once and
// a wave cannot issue past a tile request the memory system has not yet
// accepted, so requesting the whole ring first stalls the waves for several
// microseconds (about 7 at the 60000-token prefix) -- but requesting 3
// first and catching up over 4 steps measured slower still (the catch-up
// steps stalled longer), so the whole ring goes first.
constexpr int kWFirst = kWAhead;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// s_waitcnt vmcnt(n) for a run-time n in [0, 6] * DPW (the immediate must be
// a constant: one case per value).
template <int DPW>
__device__ __forceinline__ void vm_wait_tiles(int tiles) {
  switch (tiles) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<1 * DPW>(); break;
    case 2: vm_wait<2 * DPW>(); break;
    case 3: vm_wait<3 * DPW>(); break;
    case 4: vm_wait<4 * DPW>(); break;
    case 5: vm_wait<5 * DPW>(); break;
    default: vm_wait<6 * DPW>(); break;
  }
}


template <int D, int RT, bool PARTIAL>
__global__ __launch_bounds__(kWThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_wide_kernel(AttnArgs a) {
  constexpr int ROWB = D * 2;           // bytes per K/V row
  constexpr int KC = D / 16;            // k-chunks of QK^T = LDS column blocks per tensor
  constexpr int DT = D / 32;            // 32-wide D tiles of O^T
  constexpr int TILE_B = kTile * ROWB;  // bytes of one K (or V) tile
  constexpr int SLOT_B = 2 * TILE_B;    // K tile then V tile
  constexpr int NDMA = 2 * KC;          // 1 KB DMA instructions per tile
  constexpr int DPW = NDMA / kWWaves;   // per wave
  constexpr int WROWS = 32 * RT;        // query rows per wave
  constexpr int GROWS = kWWaves * WROWS;
  static_assert(DPW >= 1 && DPW * kWWaves == NDMA, "DMA split across waves");
  static_assert(kWAhead >= 3 && kWAhead < kWRing, "prefetch distance within the ring");
  static_assert(kWFirst >= 3 && kWFirst <= kWAhead && (kWAhead - kWFirst) % 2 == 0,
                "the first steps need tiles 0-2; the catch-up takes an even number of steps");

  __shared__ __attribute__((aligned(1024))) char ring[kWRing * SLOT_B];
  __shared__ uint32_t smask[TV_MAX_NODES * (TV_MAX_NODES / 32)];
  __shared__ int sblk[kBlkCache];
  __shared__ int s_par[TV_MAX_NODES];
  __shared__ int s_first, s_bad, s_redo;

  if ((int)blockIdx.x >= a.nsplit_wg) {
    merge_role<D, kWWaves>(a, (int)blockIdx.x - a.nsplit_wg);
    return;
  }

  // ---- split role -----------------------------------------------------------
  auto split_role = [&]() {
    // Workgroup -> (split, unit): units vary fastest and (sequence, kv head)
    // fastest within a unit, so with a multiple of 8 of them every split and
    // row group of a (sequence, kv head) runs on the same XCD (workgroups are
    // dealt to the 8 XCDs round robin) and shares its L2 for Q, the tree and
    // the K/V chunks its row groups both read.
    const int bgs = a.batch * a.hkv;
    const int units = bgs * a.row_groups;
    const int unit = blockIdx.x % units;
    const int s = blockIdx.x / units;
    const int rg = unit / bgs;
    const int g = (unit % bgs) % a.hkv;
    const int b = (unit % bgs) / a.hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;   // query row within a 32-row tile
    const int half = lane >> 5;  // which 16 tokens of a tile the lane's accumulators hold

    const int wg_row0 = rg * GROWS;
    const int row0 = wg_row0 + wave * WROWS;
    const bool active = row0 < a.rows;
    const bool active_all = wg_row0 + (kWWaves - 1) * WROWS < a.rows;  // uniform over the workgroup
    const int node0 = wg_row0 / a.grp;

    const int begin = s * a.chunk;
    const char* kc = reinterpret_cast<const char*>(a.k_cache + b * a.seq_stride + (int64_t)g * a.cap * D);
    const char* vc = reinterpret_cast<const char*>(a.v_cache + b * a.seq_stride + (int64_t)g * a.cap * D);
    const char* kt = reinterpret_cast<const char*>(a.k_tree + ((int64_t)b * a.n * a.hkv + g) * D);
    const char* vt = reinterpret_cast<const char*>(a.v_tree + ((int64_t)b * a.n * a.hkv + g) * D);
    const int64_t tree_rowb = (int64_t)a.hkv * ROWB;

    // ---- DMA: instruction k of this wave fills 1 KB column block cb (16
    // columns) of the K or V tile.  The block holds the columns' two 16-byte
    // halves apart: half h of token t at 512 h + 16 (t ^ 4h ^ 8(cb&1)).  The
    // 16-byte K reads of a wave (token l%32, half l/32) then cover each
    // 512-byte half once, and the transposing V reads of the four 16-lane
    // groups (4 tokens x 16 columns each, two groups per block of a pair)
    // fall on disjoint banks: conflict-free both.  DMA lane i writes 16-byte
    // slot i, so it carries half i/32 of token (i%32) ^ 4(i/32) ^ 8(cb&1);
    // a wave's instructions alternate the block parity (DPW is even).
    const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ring;
    const int dhalf = lane >> 5;
    const int dtok_e = (lane & 31) ^ (4 * dhalf);  // even column blocks
    const int dtok_o = dtok_e ^ 8;                   // odd column blocks
    static_assert(DPW % 2 == 0, "block parity of instruction k is k & 1");
    bool dvt[DPW];
    uint32_t ddst[DPW], dcol[DPW];
  #pragma unroll
    for (int k = 0; k < DPW; ++k) {
      const int inst = wave * DPW + k;
      const int cb = inst % KC;
      dvt[k] = inst >= KC;
      ddst[k] = (dvt[k] ? TILE_B : 0) + cb * 1024;
      dcol[k] = 32u * cb + 16u * dhalf;
    }
    // A wave's DPW instructions all fill one tensor (DPW divides KC): whole
    // full-mode tiles use one scalar base per wave and one lane offset, the
    // instructions 32 bytes apart in the row and 1 KB apart in LDS.
    const char* fbase = (wave * DPW >= KC ? vc : kc) + (int64_t)begin * ROWB;
    const uint32_t fvoff_e = dtok_e * ROWB + dcol[0];
    const uint32_t fvoff_o = dtok_o * ROWB + dcol[0];
    const uint32_t fdst0 = __builtin_amdgcn_readfirstlane(ring_base + ddst[0]);
    static_assert(KC % DPW == 0, "a wave's DMA instructions stay within one tensor");

    // ---- Q^T fragments (B operand of S^T = K Q^T): lane (half, col) of row
    // tile rt holds row row0 + 32 rt + col, columns 16 kc + 8 half .. +7.
    bf16x8 qf[RT][KC];
  #pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int m = row0 + 32 * rt + col;
      // a row past the last (m >= rows) reads row 0 of the group: finite
      // values whose results are never stored
      const bool real = m < a.rows;
      const int i = real ? m / a.grp : 0;
      const int h = g * a.grp + (real ? m - i * a.grp : 0);
      const bf16* qrow = a.q + (((int64_t)b * a.n + i) * a.hq + h) * D + 8 * half;
  #pragma unroll
      for (int kc2 = 0; kc2 < KC; ++kc2)
        // straight into accumulation registers, outside the compiler's wait
        // tracking: the tile requests below are inline assembly it does not
        // count, so its own wait for these loads would drain them too.  The
        // waits before the first use are explicit (pin_q).
        asm volatile("global_load_dwordx4 %0, %1, off" : "=a"(qf[rt][kc2]) : "v"(qrow + 16 * kc2) : "memory");
    }
    constexpr int kMaskPer = TV_MAX_NODES * (TV_MAX_NODES / 32) / kWThreads;
    const int node1 = min(a.n, (wg_row0 + GROWS + a.grp - 1) / a.grp);
    const int mcnt = (node1 - node0) * a.words;
    uint32_t mw[kMaskPer];
    int par_t = 0;
    if (a.mask) {
      const uint32_t* src = a.mask + ((int64_t)b * a.n + node0) * a.words;
  #pragma unroll
      for (int u = 0; u < kMaskPer; ++u) {
        const int k = tid + u * kWThreads;
        mw[u] = k < mcnt ? src[k] : 0u;
      }
    } else if (tid < a.n) {
      par_t = a.parents[(int64_t)b * a.n + tid];
    }
    constexpr int kBlkPer = kBlkCache / kWThreads;
    int pre_blk[kBlkPer];
    if (PARTIAL) {
      const int pbi0 = begin / a.block_size;
      const int pcount = min((begin + a.chunk - 1) / a.block_size - pbi0 + 1, a.max_blocks - pbi0);
      const int32_t* blist = a.block_idx + (int64_t)b * a.max_blocks;
  #pragma unroll
      for (int u = 0; u < kBlkPer; ++u) {
        const int k = tid + u * kWThreads;
        pre_blk[u] = k < pcount ? blist[pbi0 + k] : -1;
      }
    }

    __builtin_amdgcn_sched_barrier(0);  // the loads above stay ahead of the tile requests
    // ---- first tiles before the prefix length is known (full mode): whole
    // tiles below the declared maximum prefix, or the tree of a tree-only
    // workgroup.  Their rows do not depend on the prefix length.  They are
    // requested after the loads above, and the wait below is for those loads
    // only when all kWFirst tiles went out in straight-line code (the usual
    // case): the first step then waits for its own tiles, not the whole ring.
    // Q^T stays in the accumulation registers (MFMA reads its A/B operands
    // from either file; the VGPRs hold the score tiles); pin_q, after the
    // explicit wait of each branch, orders every use after that wait.
    const bool tree_own = a.tree_sep && s == a.splits;
    int spec = 0;
    int spec_landed = 0;  // first tiles known to have landed
    auto pin_q = [&]() {
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt)
  #pragma unroll
        for (int kc2 = 0; kc2 < KC; ++kc2) asm volatile("" : "+a"(qf[rt][kc2]));
    };
    const int lim = min(begin + a.chunk, a.max_prefix);
    if (!PARTIAL && !tree_own && begin < lim && (lim - begin) / kTile >= kWFirst) {
      spec = kWFirst;
  #pragma unroll
      for (int t = 0; t < kWFirst; ++t)
  #pragma unroll
        for (int k = 0; k < DPW; ++k)
          dma16s(fdst0 + t * SLOT_B + 1024 * k, fbase + (int64_t)t * (kTile * ROWB),
                 ((k & 1) ? fvoff_o : fvoff_e) + 32 * k);
      vm_wait<kWFirst * DPW>();  // the loads above, not the tiles
      pin_q();
    } else {
      if (!PARTIAL) {
        if (tree_own) {
          spec = min(kWFirst, (a.n + kTile - 1) / kTile);
          for (int t = 0; t < spec; ++t) {
            const int64_t off_e = (int64_t)min(t * kTile + dtok_e, a.n - 1) * tree_rowb;
            const int64_t off_o = (int64_t)min(t * kTile + dtok_o, a.n - 1) * tree_rowb;
  #pragma unroll
            for (int k = 0; k < DPW; ++k)
              dma16(__builtin_amdgcn_readfirstlane(ring_base + t * SLOT_B + ddst[k]),
                    (dvt[k] ? vt : kt) + ((k & 1) ? off_o : off_e) + dcol[k]);
          }
        } else {
          spec = begin < lim ? min(kWFirst, (lim - begin) / kTile) : 0;
          for (int t = 0; t < spec; ++t) {
  #pragma unroll
            for (int k = 0; k < DPW; ++k)
              dma16s(fdst0 + t * SLOT_B + 1024 * k, fbase + (int64_t)t * (kTile * ROWB),
                     ((k & 1) ? fvoff_o : fvoff_e) + 32 * k);
          }
        }
      }
      vm_wait<0>();  // the loads above and the first tiles
      pin_q();
      spec_landed = spec;
    }
    int err = 0;
    const int p_len = clamped_prefix(a, b, &err);
    const int slots = prefix_slots(a, b, p_len, &err);
    if (err && s == 0 && unit == 0 && tid == 0) raise_err(a.dev_err, err);
    err = 0;
    const int ns = (slots + a.chunk - 1) / a.chunk;
    const bool has_tree = a.tree_sep ? s == a.splits : s == max(ns - 1, 0);
    const int end = min(begin + a.chunk, slots);
    int np = begin < end ? (end - begin + kTile - 1) / kTile : 0;
    const int nt = has_tree ? (a.n + kTile - 1) / kTile : 0;
    const int64_t prow0 = (((int64_t)b * a.nparts + s) * a.hkv + g) * a.rows;
    auto write_empty = [&]() {
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int m = row0 + 32 * rt + col;
        if (active && m < a.rows && half == 0) store_part_ml(a, a.part_ml + prow0 + m, make_float2(-INFINITY, 0.f));
      }
    };
    if (np == 0 && nt == 0) {
      write_empty();
      vm_wait<0>();  // no first-tile request outlives the workgroup's LDS
      return;
    }

    // ---- per-split tables in LDS (tree mask rows, partial-mode block ids) ----
    int bi0 = 0;
    int fb_row = begin;
    if (has_tree && a.mask) {
  #pragma unroll
      for (int u = 0; u < kMaskPer; ++u) {
        const int k = tid + u * kWThreads;
        if (k < mcnt) smask[k] = mw[u];
      }
    } else if (has_tree) {
      // the mask from the parent array (SpecBlock App. A.2: ancestors and
      // self), the rule and fallback of tv_build_tree_mask
      if (tid == 0) s_bad = 0;
      if (tid < a.n) s_par[tid] = par_t;
      __syncthreads();
      if (tid < a.n && !(tid == 0 ? par_t == -1 : (par_t >= 0 && par_t < tid))) s_bad = 1;
      __syncthreads();
      const bool bad = s_bad != 0;
      const bool writer = g == 0 && (a.mask_out || a.depth_out);
      if (tid >= node0 && tid < node1) {
        uint32_t* row = &smask[(tid - node0) * a.words];
        for (int w = 0; w < a.words; ++w) row[w] = 0u;
        row[tid >> 5] |= 1u << (tid & 31);
        int depth = 0;
        if (!bad)
          for (int j = s_par[tid]; j >= 0; j = s_par[j]) {
            row[j >> 5] |= 1u << (j & 31);
            ++depth;
          }
        if (writer) {
          if (a.mask_out)
            for (int w = 0; w < a.words; ++w) a.mask_out[((int64_t)b * a.n + tid) * a.words + w] = row[w];
          if (a.depth_out) a.depth_out[(int64_t)b * a.n + tid] = depth;
        }
      }
      if (bad && g == 0 && rg == 0 && tid == 0) raise_err(a.dev_err, TV_DERR_BAD_PARENT);
    }
    if (PARTIAL && np > 0) {
      bi0 = begin / a.block_size;
      const int bi1 = (end - 1) / a.block_size;
      if (tid == 0) s_first = INT32_MAX;
      __syncthreads();
  #pragma unroll
      for (int u = 0; u < kBlkPer; ++u) {
        const int k = tid + u * kWThreads;
        if (k < bi1 - bi0 + 1) {
          const int blk = pre_blk[u];
          sblk[k] = blk;
          if (blk >= 0 && (int64_t)blk * a.block_size < p_len) atomicMin(&s_first, k);
          else err |= TV_DERR_BAD_BLOCK;
        }
      }
      __syncthreads();
      const int first = s_first;
      if (first == INT32_MAX) {
        if (!has_tree) {
          if (err) raise_err(a.dev_err, err);
          write_empty();
          vm_wait<0>();  // no first-tile request outlives the workgroup's LDS
          return;
        }
        np = 0;
      } else {
        fb_row = sblk[first] * a.block_size;
      }
    }
    const int ntiles = np + nt;
    const int nfull = PARTIAL ? 0 : (end - begin) / kTile;
    // requested tiles that are this split's own first tiles
    const int skip = tree_own ? spec : max(0, min(spec, nfull));
    // first tiles that are not this split's own are requested again into
    // the same slots: the speculative requests must have landed before.
    // Of the first tiles, those below skip count as landed only when waited
    // for; the ones requested again have not.
    if (skip < spec && spec_landed < spec) vm_wait<0>();
    spec_landed = spec_landed > 0 || skip < spec ? skip : 0;
    auto slot_row = [&](int u, bool& valid) -> int {
      if (u >= end) {
        valid = false;
        return fb_row;
      }
      if (!PARTIAL) {
        valid = true;
        return u;
      }
      const int bi = a.block_shift >= 0 ? (u >> a.block_shift) : (u / a.block_size);
      const int blk = sblk[bi - bi0];
      const int row = blk * a.block_size + (u - bi * a.block_size);
      valid = blk >= 0 && (int64_t)blk * a.block_size < p_len && row < p_len;
      return valid ? row : fb_row;
    };
    // whole tile it of full mode into ring slot `slot`
    auto dma_whole = [&](int slot, int it) {
  #pragma unroll
      for (int k = 0; k < DPW; ++k)
        dma16s(fdst0 + slot * SLOT_B + 1024 * k, fbase + (int64_t)it * (kTile * ROWB),
               ((k & 1) ? fvoff_o : fvoff_e) + 32 * k);
    };
    auto dma_tile = [&](int slot, int it) {
      if (it < nfull) {
        dma_whole(slot, it);
        return;
      }
      const char* kb;
      const char* vb;
      int64_t off_e, off_o;
      if (it < np) {
        bool valid;
        off_e = (int64_t)slot_row(begin + it * kTile + dtok_e, valid) * ROWB;
        off_o = (int64_t)slot_row(begin + it * kTile + dtok_o, valid) * ROWB;
        kb = kc;
        vb = vc;
      } else {
        off_e = (int64_t)min((it - np) * kTile + dtok_e, a.n - 1) * tree_rowb;
        off_o = (int64_t)min((it - np) * kTile + dtok_o, a.n - 1) * tree_rowb;
        kb = kt;
        vb = vt;
      }
  #pragma unroll
      for (int k = 0; k < DPW; ++k)
        dma16(__builtin_amdgcn_readfirstlane(ring_base + slot * SLOT_B + ddst[k]),
              (dvt[k] ? vb : kb) + ((k & 1) ? off_o : off_e) + dcol[k]);
    };
    auto tile_bits = [&](int it) -> uint32_t {
      int cnt;
      if (it >= np) {
        cnt = a.n - (it - np) * kTile;
      } else if (!PARTIAL) {
        cnt = end - (begin + it * kTile);
      } else {
        bool valid = false;
        if (lane < kTile) slot_row(begin + it * kTile + lane, valid);
        return (uint32_t)__ballot(valid);
      }
      return cnt >= kTile ? 0xFFFFFFFFu : (cnt <= 0 ? 0u : ((1u << cnt) - 1u));
    };

    // ---- LDS operand addressing ------------------------------------------------
    // K fragment kc (A operand, token col, columns 16kc + 8half..+7): column
    // block kc, each half a contiguous 512 bytes over its 32 lanes.
    const uint32_t koff_e = 512u * half + 16u * (col ^ (4 * half));
    const uint32_t koff_o = 512u * half + 16u * (col ^ (4 * half) ^ 8);
    // V^T fragment (dt, kt): in 16-lane group q the transposing read returns
    // column 16(q&1) + j of tokens T0..T0+3 to lane j when lane j addresses
    // token T0 + j/4, columns 4(j&3)..+3 (half (j&3)/2, bytes 8(j&1)) of
    // column block 2dt + (q&1).  T0 = 16kt + 4(q>>1) for k-slots 0-3, and 8
    // tokens later for k-slots 4-7: the tokens of registers 8kt..8kt+7 of
    // the S^T accumulator of lane half q>>1.  The token XORs flip bits 2
    // and 3 of a token below 8, so the 16kt step stays a plain offset (256
    // kt) while the 8-token step (bit 3) is +128 bytes in even blocks and
    // -128 in odd ones: voff_hi.
    const int q16 = lane >> 4, j16 = lane & 15;
    const int vh = (j16 & 3) >> 1;
    const uint32_t voff = TILE_B + 1024u * (q16 & 1) + 512u * vh +
                          16u * ((4 * (q16 >> 1) + (j16 >> 2)) ^ (4 * vh) ^ (8 * (q16 & 1))) +
                          8u * (j16 & 1);
    const uint32_t voff_hi = voff + ((q16 & 1) ? -128u : 128u);
    typedef __attribute__((address_space(3))) char lds_char;
    auto lds_at = [&](uint32_t addr) { return (lds_char*)(uintptr_t)addr; };
    auto kfrag = [&](uint32_t sa, int kc2) -> bf16x8 {
      return *(__attribute__((address_space(3))) const bf16x8*)lds_at(sa + ((kc2 & 1) ? koff_o : koff_e) + 1024 * kc2);
    };
    auto vfrag = [&](uint32_t sa, int dt, int ktk) -> bf16x8 {
      const uint32_t ad = sa + voff + 2048 * dt + 256 * ktk;
      const uint32_t ad2 = sa + voff_hi + 2048 * dt + 256 * ktk;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds_at(ad));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds_at(ad2));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // ---- per-tile math ---------------------------------------------------------
    f32x16 o[DT][RT];
    float lsum[RT];  // this lane's share of the row sum (its 16 tokens of each tile)
    float mref[RT];  // reference max per row (log2 units), -inf until set

    auto mask_tile = [&](int it, f32x16 (&sc)[RT]) {
      const uint32_t vbits = tile_bits(it);
      const bool tt = it >= np;
      if (!tt && vbits == 0xFFFFFFFFu) return;
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        uint32_t allow = vbits;
        if (tt) {
          const int m = row0 + 32 * rt + col;
          allow &= m < a.rows ? smask[(m / a.grp - node0) * a.words + (it - np)] : 0u;
        }
        allow >>= 4 * half;
  #pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((allow >> (8 * (r >> 2) + (r & 3))) & 1u)) sc[rt][r] = -INFINITY;
      }
    };
    auto track_max = [&](f32x16 (&sc)[RT]) {
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float mx = sc[rt][0];
  #pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[rt][r]);
        mx = xmax_half(mx) * a.c;
        mref[rt] = mref[rt] == -INFINITY ? mx : mref[rt];
      }
    };
    // p = 2^(s c - mref) of row tile rt, as the two bf16 B operands of PV; the
    // row sum adds the fp32 weights before rounding
    auto softmax = [&](const f32x16& sc, int rt, bf16x8 (&pb)[2]) {
      const float mu = mref[rt] == -INFINITY ? 0.f : mref[rt];
      float p[16];
  #pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], a.c, -mu));
  #pragma unroll
      for (int ktk = 0; ktk < 2; ++ktk)
  #pragma unroll
        for (int e = 0; e < 8; ++e) pb[ktk][e] = (bf16)p[8 * ktk + e];
      float t[8];
  #pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = p[2 * e] + p[2 * e + 1];
      lsum[rt] += ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    };

  #define TV_SCHED_FENCE __builtin_amdgcn_sched_barrier(0)
    // Operand reads of a tile (K, or V^T): the loop reads the next tile's
    // operands while the current tile's MFMAs run.
    auto read_k = [&](int it, bf16x8 (&kf)[KC]) {
      const uint32_t kbase = ring_base + (it & (kWRing - 1)) * SLOT_B;
      const uint32_t kaddr_e = koff_e + kbase, kaddr_o = koff_o + kbase;
  #pragma unroll
      for (int kc2 = 0; kc2 < KC; ++kc2) {
        kf[kc2] = *(__attribute__((address_space(3))) const bf16x8*)lds_at(((kc2 & 1) ? kaddr_o : kaddr_e) + 1024 * kc2);
      }
    };
    auto read_v = [&](int it, bf16x8 (&vf)[DT][2]) {
      const uint32_t vbase = ring_base + (it & (kWRing - 1)) * SLOT_B;
      const uint32_t vaddr = voff + vbase, vaddr2 = voff_hi + vbase;
  #pragma unroll
      for (int dt = 0; dt < DT; ++dt)
  #pragma unroll
        for (int ktk = 0; ktk < 2; ++ktk) {
          const uint32_t ad = vaddr + 2048 * dt + 256 * ktk;
          const uint32_t ad2 = vaddr2 + 2048 * dt + 256 * ktk;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds_at(ad));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds_at(ad2));
          vf[dt][ktk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    auto qk = [&](const bf16x8 (&kf)[KC], f32x16 (&sc)[RT]) {
  #pragma unroll
      for (int kc2 = 0; kc2 < KC; ++kc2)
  #pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc2], qf[rt][kc2], kc2 == 0 ? f32x16{} : sc[rt], 0, 0, 0);
    };
    // tiles that need a mask: the prefix tail (full mode), every partial-mode
    // tile (listed blocks may be invalid or past the prefix), the tree tiles
    auto needs_mask = [&](int it) { return PARTIAL || it >= nfull; };

    // run(skip_tiles, landed_tiles, track): tiles below skip_tiles were
    // requested already, those below landed_tiles have landed
    auto run = [&](int skip_tiles, int landed_tiles, bool track) {
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        lsum[rt] = 0.f;
  #pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][rt] = f32x16{};
      }
      // tiles skip_tiles .. kWFirst-1 (those that exist) into their slots
      for (int t = skip_tiles; t < min(kWFirst, ntiles); ++t) dma_tile(t & (kWRing - 1), t);
      int issued = min(kWFirst, ntiles) - 1;  // last requested tile
      // wait until tile x has landed (tiles below landed_tiles landed
      // before); in the steady state kWAhead - 3 later tiles are in flight
      auto wait_tile = [&](int x) {
        if (x < landed_tiles) return;
        const int c = issued - x;
        if (c >= kWAhead - 3) vm_wait<(kWAhead - 3) * DPW>();
        else vm_wait_tiles<DPW>(c);
      };
      wait_tile(min(1, ntiles - 1));
      lds_barrier();
      f32x16 sA[RT], sB[RT];
      // P of the current and of the previous tile: the PV product of a tile
      // runs one step after its softmax, so that both MFMA groups of a step
      // have softmax work to overlap
      bf16x8 pA[RT][2], pB[RT][2];
      // The K and V^T operands of the next products.  Each fragment is read
      // again for a later tile right after the last MFMA that uses it, so one
      // set of registers carries the pipeline.  vf holds V of the tile whose
      // PV product comes next; before the first step that is a product with
      // zero weights.
      bf16x8 kf[KC];
      bf16x8 vf[DT][2];
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) pB[rt][0] = pB[rt][1] = bf16x8{};
  #pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt][0] = vf[dt][1] = bf16x8{};
      if (active) {
        read_k(0, kf);
        qk(kf, sA);
        read_k(1, kf);   // past the last tile this reads a stale slot; never used
        mask_tile(0, sA);
        if (track) track_max(sA);
      }
      // Step t (tile t+2 has landed for every wave; every wave is past step
      // t-1): request tile t + kWAhead into the slot of tile
      // t + kWAhead - kWRing < t, which is no longer read;
      //   group 1: QK^T of tile t+1 (K in kf) with the softmax of S(t) for the
      //            first row tile, refilling kf with K of tile t+2;
      //   group 2: PV of tile t-1 (V in vf, P in pprev) with the softmax of the
      //            other row tile, refilling vf with V of tile t.
      // FAST: a steady-state step (whole unmasked tiles, the tile kWAhead
      // ahead is whole too): no branch.
      auto step = [&](auto fast_tag, int t, f32x16 (&cur)[RT], f32x16 (&nxt)[RT], bf16x8 (&pcur)[RT][2],
                      bf16x8 (&pprev)[RT][2]) {
        constexpr bool FAST = decltype(fast_tag)::value;
        if (FAST) {
          vm_wait<(kWAhead - 3) * DPW>();
        } else if (t + 2 < ntiles) {
          wait_tile(t + 2);
        }
        lds_barrier();
        if (FAST) {
          dma_whole((t + kWAhead) & (kWRing - 1), t + kWAhead);
        } else {
          // up to tile t + kWAhead, at most two per step (the first steps
          // catch up with the tiles not requested before the first step);
          // tile x goes to the slot of tile x - kWRing <= t - 1, free now
          const int want = min(t + kWAhead, ntiles - 1);
          if (issued < want) {
            ++issued;
            dma_tile(issued & (kWRing - 1), issued);
          }
          if (issued < want) {
            ++issued;
            dma_tile(issued & (kWRing - 1), issued);
          }
        }
        if (!FAST && !active) return;
        const uint32_t kbase = ring_base + ((t + 2) & (kWRing - 1)) * SLOT_B;
        const uint32_t kaddr_e = koff_e + kbase, kaddr_o = koff_o + kbase;
        const uint32_t vbase = ring_base + (t & (kWRing - 1)) * SLOT_B;
        const uint32_t vaddr = voff + vbase, vaddr2 = voff_hi + vbase;
        TV_SCHED_FENCE;
        softmax(cur[0], 0, pcur[0]);
  #pragma unroll
        for (int kc2 = 0; kc2 < KC; ++kc2) {
  #pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            nxt[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc2], qf[rt][kc2], kc2 == 0 ? f32x16{} : nxt[rt], 0, 0, 0);
          kf[kc2] = *(__attribute__((address_space(3))) const bf16x8*)lds_at(((kc2 & 1) ? kaddr_o : kaddr_e) + 1024 * kc2);
        }
  #pragma unroll
        for (int i = 0; i < KC * RT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);  // VALU incl. transcendental
          if (i % RT == RT - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        TV_SCHED_FENCE;
  #pragma unroll
        for (int rt = 1; rt < RT; ++rt) softmax(cur[rt], rt, pcur[rt]);
  #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
  #pragma unroll
          for (int ktk = 0; ktk < 2; ++ktk) {
  #pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              o[dt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][ktk], pprev[rt][ktk], o[dt][rt], 0, 0, 0);
            const uint32_t ad = vaddr + 2048 * dt + 256 * ktk;
            const uint32_t ad2 = vaddr2 + 2048 * dt + 256 * ktk;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds_at(ad));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds_at(ad2));
            vf[dt][ktk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
  #pragma unroll
        for (int i = 0; i < DT * 2 * RT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (RT > 1) __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);  // VALU incl. transcendental
          __builtin_amdgcn_sched_group_barrier(0x100, 2 / RT, 0);  // DS read
        }
        TV_SCHED_FENCE;
        if (!FAST && t + 1 < ntiles && needs_mask(t + 1)) mask_tile(t + 1, nxt);
      };
      // Steps go in pairs, which keeps the roles of the two score and P
      // buffers.  The first kWAhead - kWFirst steps catch up with the tile
      // requests (general steps); then steady steps t < nfast: every wave is
      // active, tiles t+1 and t+2 exist, tile t+1 needs no mask and tile
      // t + kWAhead is a whole tile, requested with no branch.
      constexpr int kRamp = kWAhead - kWFirst;
      int nfast = active_all ? min(nfull - kWAhead, min(ntiles - 2, nfull - 1)) : 0;
      nfast = nfast > kRamp ? (nfast & ~1) : 0;
      int t = 0;
      bool last_in_b = true;  // which P buffer holds the last tile's weights
      auto general_pairs = [&](int t_end) {
        for (; t < t_end; t += 2) {
          step(std::false_type{}, t, sA, sB, pA, pB);
          last_in_b = false;
          if (t + 1 < ntiles) {
            step(std::false_type{}, t + 1, sB, sA, pB, pA);
            last_in_b = true;
          }
        }
      };
      if (nfast > 0) {
        general_pairs(kRamp);  // issued == kRamp - 1 + kWAhead afterwards
        for (; t < nfast; t += 2) {
          step(std::true_type{}, t, sA, sB, pA, pB);
          step(std::true_type{}, t + 1, sB, sA, pB, pA);
        }
        issued = nfast - 1 + kWAhead;
        last_in_b = true;
      }
      general_pairs(ntiles);
      // PV of the last tile (V read in the last step)
      if (active) {
        vm_wait<0>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
  #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
  #pragma unroll
          for (int ktk = 0; ktk < 2; ++ktk)
  #pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              o[dt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  vf[dt][ktk], last_in_b ? pB[rt][ktk] : pA[rt][ktk], o[dt][rt], 0, 0, 0);
      }
      vm_wait<0>();
      lds_barrier();
    };
  #undef TV_SCHED_FENCE

  #pragma unroll
    for (int rt = 0; rt < RT; ++rt) mref[rt] = -INFINITY;
    run(skip, spec_landed, true);

    // ---- overflow check; exact two-pass recompute when needed ------------------
    if (tid == 0) s_redo = 0;
    __syncthreads();
    if (active) {
      bool bad = false;
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float l = xsum_half(lsum[rt]);
        float acc = 0.f;
  #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
  #pragma unroll
          for (int r = 0; r < 16; ++r) acc += o[dt][rt][r];
        const bool fin = __builtin_isfinite(acc);
        const bool real = row0 + 32 * rt + col < a.rows;
        bad |= real && (mref[rt] == -INFINITY ? l > 0.f : !(l <= kSumMax && fin));
      }
      if (__ballot(bad) && lane == 0) s_redo = 1;
    }
    __syncthreads();
    if (s_redo) {
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) mref[rt] = -INFINITY;
      for (int it = 0; it < ntiles; ++it) {
        dma_tile(0, it);
        vm_wait<0>();
        lds_barrier();
        if (active) {
          bf16x8 kf[KC];
  #pragma unroll
          for (int kc2 = 0; kc2 < KC; ++kc2) kf[kc2] = kfrag(ring_base, kc2);
          f32x16 sc[RT];
  #pragma unroll
          for (int kc2 = 0; kc2 < KC; ++kc2)
  #pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              sc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc2], qf[rt][kc2], kc2 == 0 ? f32x16{} : sc[rt], 0, 0, 0);
          mask_tile(it, sc);
  #pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            float mx = sc[rt][0];
  #pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[rt][r]);
            mref[rt] = fmaxf(mref[rt], xmax_half(mx) * a.c);
          }
        }
        lds_barrier();
      }
      run(0, 0, false);
    }
    if (err) raise_err(a.dev_err, err);

    // ---- partial write: output / own row sum as bf16, (reference max, sum) --
    // Staged per wave in the idle ring as [row][D] with 16-byte chunk c of row
    // r at position c ^ (r mod CH), then written as whole rows.
    if (!active) return;
    {
      constexpr int CH = ROWB / 16;      // 16-byte chunks per row
      constexpr int RPI = 1024 / ROWB;   // rows per 1 KB wave store
      static_assert(kWWaves * WROWS * ROWB <= kWRing * SLOT_B, "staging fits the ring");
      const uint32_t stage = ring_base + wave * (WROWS * ROWB);
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float l = xsum_half(lsum[rt]);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int r = 32 * rt + col;
  #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x4 v;
  #pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[dt][rt][4 * q + e] * inv);
            const int c = 4 * dt + q;
            *(__attribute__((address_space(3))) bf16x4*)lds_at(stage + r * ROWB + 16 * (c ^ (r & (CH - 1))) + 8 * half) = v;
          }
        if (half == 0 && row0 + r < a.rows) store_part_ml(a, a.part_ml + prow0 + row0 + r, make_float2(mref[rt], l));
      }
  #pragma unroll
      for (int j = 0; j < WROWS / RPI; ++j) {
        const int r = j * RPI + lane / CH;
        const int p = lane % CH;
        const bf16x8 v = *(__attribute__((address_space(3))) const bf16x8*)lds_at(stage + r * ROWB + 16 * p);
        if (row0 + r < a.rows) store_part_o(a, a.part_o + (prow0 + row0 + r) * D + 8 * (p ^ (r & (CH - 1))), v);
      }
    }

  };
  split_role();
  if (a.sync) split_done(a, (int)(blockIdx.x % (a.batch * a.hkv * a.row_groups)) % (a.batch * a.hkv));
}

template <int D, int RT>
void launch_wide_t(const AttnArgs& args, unsigned grid, hipStream_t stream) {
  if (args.max_blocks)
    hipLaunchKernelGGL((attn_wide_kernel<D, RT, true>), dim3(grid), dim3(kWThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((attn_wide_kernel<D, RT, false>), dim3(grid), dim3(kWThreads), 0, stream, args);
}

}  // namespace

hipError_t launch_wide(const AttnArgs& a, int head_dim, int rt, unsigned grid, hipStream_t stream) {
  if (head_dim == 128) {
    if (rt == 1) launch_wide_t<128, 1>(a, grid, stream);
    else launch_wide_t<128, 2>(a, grid, stream);
  } else {
    if (rt == 1) launch_wide_t<64, 1>(a, grid, stream);
    else launch_wide_t<64, 2>(a, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace attn
}  // namespace tv
