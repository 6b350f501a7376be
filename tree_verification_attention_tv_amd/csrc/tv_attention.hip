// Tree-masked GQA attention for the verify forward of a draft tree.
//
// Sources: SpecBlock App. A.2 (a node sees the verified prefix, its on-path
// ancestors and itself); SpecPV Sec. 3.2 (a selected subset of KV blocks is
// attended as one continuous segment); "Dynamic Speculative Decoding",
// Roofline analysis (decode attention is bandwidth-bound; a tree of N
// proposed tokens multiplies the arithmetic intensity by N).
//
// Design (gfx950):
//  * One workgroup (8 waves) per (sequence, kv head, row group, split).  It
//    holds up to 256 query rows of its kv head -- the n_nodes x group rows
//    -- so each K/V tile is read from HBM once and reused by all rows (rows
//    FLOP/byte).  Each wave owns RB (1 or 2) blocks of 16 rows.  At least
//    two waves per SIMD are needed to keep the matrix core busy: a single
//    wave issues dependent-free MFMAs at well under peak.  Two-block plans
//    run one workgroup per CU (two waves per SIMD, the ping-pong schedule
//    below); one-block plans may run two per CU (four waves per SIMD, the
//    flat schedule, 128 VGPRs).
//  * The prefix (full rows, or the listed blocks) is cut into `splits`
//    contiguous ranges, one workgroup each, with `splits` chosen so that the
//    grid fits the CUs in one round.  The workgroup of the last non-empty
//    range also runs the tree block's tiles, masked with the packed ancestor
//    bits, after its prefix tiles.  Each split writes, per row, its output
//    divided by its own row sum (bf16) and the (reference max, sum) pair
//    (fp32); a combine kernel merges them in a fixed order.
//  * 32-token K/V tiles go from HBM straight to LDS with LDS DMA
//    (global_load_lds_dwordx4) into a 4-slot ring, two tiles in flight, with
//    no staging registers.  The tile layout in LDS (column blocks, below)
//    keeps the K and V operand reads free of bank conflicts and makes every
//    operand address one per-lane base plus an immediate.
//  * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16.  The
//    S^T accumulator gives every lane one query row and four tokens, so row
//    statistics need two cross-lane steps (the row sum only once, at the
//    end: each lane accumulates its share in fp32 before p is rounded).
//    P^T is packed to bf16 straight from those registers as the B operand
//    of the PV product, and the V^T A operand comes from ds_read_b64_tr_b16
//    (two per operand).
//  * Software pipeline: each step first issues all LDS operand reads (K of
//    tile i+1, V of tile i), then the softmax of tile i, then the QK chains
//    of tile i+1 interleaved with the independent PV products of tile i.
//  * Softmax in fp32, log2 domain (scale * log2 e folded into one FMA
//    before v_exp_f32).  Each row's reference max is fixed at the first tile
//    in which the row sees a key, so the hot loop never rescales the output
//    accumulators: later scores above the reference only make p > 1, which
//    fp32 accumulates exactly enough (p is also exact in bf16's 8-bit
//    exponent).  If a row's sum leaves [1, 2^100] or an output is not
//    finite, the split is recomputed with the exact row max from a QK-only
//    pre-pass (p <= 1 then).  Masked scores are -inf.
#include "tv_attn_common.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace tv {
namespace {

using namespace attn;

constexpr int kThreads = 256;      // combine kernel
constexpr int kWaves = 8;          // split kernel: 8 waves (two or four per SIMD with OCC)
constexpr int kSplitThreads = kWaves * 64;

// OCC: waves per SIMD.  2: one workgroup per CU, the ping-pong schedule
// below.  4: two workgroups per CU (128 VGPRs), a flat schedule with one
// barrier per tile whose operand-read latency the other waves hide.
template <int D, int RB, bool PARTIAL, int OCC>
__global__ __launch_bounds__(kSplitThreads, OCC) void attn_split_kernel(AttnArgs a) {
  constexpr int ROWB = D * 2;               // bytes per row
  constexpr int DC = D / 32;                // k-steps of the QK^T product
  constexpr int DB = D / 16;                // 16-wide output blocks of PV
  constexpr int TILE_B = kTile * ROWB;      // bytes of one K (or V) tile
  constexpr int SLOT_B = 2 * TILE_B;        // K tile then V tile
  constexpr int IPT = D / 16;               // DMA instructions (1 KB column blocks) per tensor per tile
  constexpr int DPT = 2 * IPT / kWaves;     // DMA instructions per wave per tile
  static_assert(DPT == 1 || DPT == 2, "DMA split across waves");

  __shared__ __attribute__((aligned(1024))) char ring[kRing * SLOT_B];
  __shared__ uint32_t smask[TV_MAX_NODES * (TV_MAX_NODES / 32)];  // tree rows of this WG
  __shared__ int sblk[kBlkCache];                                 // partial: block ids
  __shared__ int s_par[TV_MAX_NODES];                             // parents (in-kernel mask)
  __shared__ int s_first, s_bad;

  if ((int)blockIdx.x >= a.nsplit_wg) {
    merge_role<D, kWaves>(a, (int)blockIdx.x - a.nsplit_wg);
    return;
  }
  // Workgroup -> (split, unit), units varying fastest and (sequence, kv
  // head) fastest within a unit: with a multiple of 8 of them every split and
  // every row group of a (sequence, kv head) lands on the same XCD
  // (workgroups are dealt to the XCDs in turn), so the row groups reading one
  // K/V chunk share its L2 lines.
  const int bgs = a.batch * a.hkv;
  const int units = bgs * a.row_groups;
  const int unit = (int)blockIdx.x % units;
  const int s = (int)blockIdx.x / units;
  const int bg = unit % bgs;
  const int b = bg / a.hkv;
  const int g = bg % a.hkv;
  const int rg = unit / bgs;
  {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15;   // MFMA column (query row within a block)
  const int grp4 = lane >> 4;  // lane group 0..3

  const int wg_row0 = rg * (16 * kWaves * RB);
  const int row0 = wg_row0 + wave * (16 * RB);
  const bool active = row0 < a.rows;
  const int node0 = wg_row0 / a.grp;

  // ---- sources --------------------------------------------------------------
  const int begin = s * a.chunk;  // first prefix slot of this split
  const char* kc = reinterpret_cast<const char*>(a.k_cache + b * a.seq_stride + (int64_t)g * a.cap * D);
  const char* vc = reinterpret_cast<const char*>(a.v_cache + b * a.seq_stride + (int64_t)g * a.cap * D);
  const char* kt = reinterpret_cast<const char*>(a.k_tree + ((int64_t)b * a.n * a.hkv + g) * D);
  const char* vt = reinterpret_cast<const char*>(a.v_tree + ((int64_t)b * a.n * a.hkv + g) * D);
  const int64_t tree_rowb = (int64_t)a.hkv * ROWB;  // bytes between tree nodes

  // ---- tile layout in LDS and its DMA ------------------------------------
  // A K (or V) tile is stored as D/16 column blocks of 1 KB; block cb holds
  // columns 16cb..16cb+15 of the 32 tokens, 32 bytes per token.  The
  // 16-byte K reads of a wave then cover two contiguous 512-byte runs and
  // the transposing V reads 128 contiguous bytes per 16 lanes, both at the
  // full LDS rate on gfx950 (measured: 16-byte reads at ~250 B/clk per CU,
  // transposing 8-byte reads at ~125), and every operand read is one
  // per-lane base plus an immediate.  DMA instruction cb of a tensor fills
  // block cb: lane i writes 16-byte slot i, i.e. token i/2, half i&1.
  const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ring;
  const int dtok = lane >> 1;                               // token of this lane's DMA slot
  const int dhalf = lane & 1;                               // 16-byte half it carries
  int dt[DPT];        // tensor of the instruction (0 = K, 1 = V)
  uint32_t ddst[DPT]; // slot-relative LDS byte offset of the instruction
  uint32_t dcol[DPT]; // byte offset of the lane's 16 bytes within the source row
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int inst = wave * DPT + k;  // 0 .. 2*IPT-1
    const int cb = inst % IPT;
    dt[k] = inst / IPT;
    ddst[k] = dt[k] * TILE_B + cb * 1024;
    dcol[k] = 16u * (2 * cb + dhalf);
  }
  // Whole prefix tiles of full mode read 32 consecutive rows: a scalar base
  // per tile plus a fixed per-lane offset.
  uint32_t fvoff[DPT];      // per-lane offset within the tile's rows
  const char* fbase[DPT];   // source of tile 0 (wave-uniform)
  uint32_t fdst[DPT];       // LDS address in slot 0 (wave-uniform)
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    fvoff[k] = dtok * ROWB + dcol[k];
    fbase[k] = (dt[k] ? vc : kc) + (int64_t)begin * ROWB;
    fdst[k] = __builtin_amdgcn_readfirstlane(ring_base + ddst[k]);
  }

  // ---- first tiles, requested before the prefix length is known -----------
  // Their rows do not depend on it: whole prefix tiles below the declared
  // maximum prefix (full mode), or the tree tiles of a workgroup that holds
  // only the tree.  They share the memory round trip of the loads below;
  // once the prefix length is known, the run keeps those that are its own
  // first tiles (all of them unless the prefix is shorter than the maximum)
  // and requests the others again.
  const bool tree_own = a.tree_sep && s == a.splits;
  int spec = 0;
  if (!PARTIAL) {
    if (tree_own) {
      spec = min(kRing, (a.n + kTile - 1) / kTile);
#pragma unroll
      for (int t = 0; t < kRing; ++t)
        if (t < spec) {
          const int64_t off = (int64_t)min(t * kTile + dtok, a.n - 1) * tree_rowb;
#pragma unroll
          for (int k = 0; k < DPT; ++k)
            dma16(__builtin_amdgcn_readfirstlane(ring_base + t * SLOT_B + ddst[k]),
                  (dt[k] ? vt : kt) + off + dcol[k]);
        }
    } else {
      const int lim = min(begin + a.chunk, a.max_prefix);
      spec = begin < lim ? min(kRing, (lim - begin) / kTile) : 0;
#pragma unroll
      for (int t = 0; t < kRing; ++t)
        if (t < spec) {
#pragma unroll
          for (int k = 0; k < DPT; ++k)
            dma16s(fdst[k] + t * SLOT_B, fbase[k] + (int64_t)t * (kTile * ROWB), fvoff[k]);
        }
    }
  }

  // ---- loads that do not depend on the prefix length ------------------------
  // Issued first so that they share one memory round trip with prefix_len:
  // the Q^T fragments (B operand of S^T = K Q^T) and this workgroup's mask
  // words (kept in registers until it is known whether the tree is ours).
  bf16x8 qf[RB][DC];
#pragma unroll
  for (int mb = 0; mb < RB; ++mb) {
    const int m = row0 + 16 * mb + col;
    // a row past the last (m >= rows) reads row 0 of the group: finite
    // values whose results are never stored
    const bool real = m < a.rows;
    const int i = real ? m / a.grp : 0;
    const int h = g * a.grp + (real ? m - i * a.grp : 0);
    const bf16* qrow = a.q + (((int64_t)b * a.n + i) * a.hq + h) * D + 8 * grp4;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[mb][dc] = *reinterpret_cast<const bf16x8*>(qrow + 32 * dc);
  }
  constexpr int kMaskPer = TV_MAX_NODES * (TV_MAX_NODES / 32) / kSplitThreads;  // words per thread
  const int node1 = min(a.n, (wg_row0 + 16 * kWaves * RB + a.grp - 1) / a.grp);
  const int mcnt = (node1 - node0) * a.words;
  uint32_t mw[kMaskPer];
  int par_t = 0;
  if (a.mask) {
    const uint32_t* src = a.mask + ((int64_t)b * a.n + node0) * a.words;
#pragma unroll
    for (int u = 0; u < kMaskPer; ++u) {
      const int k = tid + u * kSplitThreads;
      mw[u] = k < mcnt ? src[k] : 0u;
    }
  } else if (tid < a.n) {
    par_t = a.parents[(int64_t)b * a.n + tid];
  }
  // partial mode: the block ids this split can touch (the blocks of slots
  // begin .. begin + chunk - 1, within the list), in the same round trip;
  // which of them count is decided once the list length and the prefix
  // length are known
  constexpr int kBlkPer = kBlkCache / kSplitThreads;
  int pre_blk[kBlkPer];
  if (PARTIAL) {
    const int pbi0 = begin / a.block_size;
    const int pcount = min((begin + a.chunk - 1) / a.block_size - pbi0 + 1, a.max_blocks - pbi0);
    const int32_t* blist = a.block_idx + (int64_t)b * a.max_blocks;
#pragma unroll
    for (int u = 0; u < kBlkPer; ++u) {
      const int k = tid + u * kSplitThreads;
      pre_blk[u] = k < pcount ? blist[pbi0 + k] : -1;
    }
  }

  int err = 0;
  const int p_len = clamped_prefix(a, b, &err);
  const int slots = prefix_slots(a, b, p_len, &err);
  // Wait for all of the above (and the first tiles) here, on every path: the
  // compiler's own wait would otherwise be placed inside the loop (vmcnt(0),
  // draining the tile DMA each step).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding: vmcnt(0)
  if (err && s == 0 && g == 0 && rg == 0 && tid == 0) raise_err(a.dev_err, err);
  err = 0;
  // Prefix range of this split.  The tree block runs either in a workgroup of
  // its own (split index `splits`, whose prefix range is empty) or, when the
  // grid must stay within one workgroup per CU, after the prefix tiles of the
  // last non-empty split (split 0 when the prefix is empty).
  const int ns = (slots + a.chunk - 1) / a.chunk;
  const bool has_tree = a.tree_sep ? s == a.splits : s == max(ns - 1, 0);
  const int end = min(begin + a.chunk, slots);
  int np = begin < end ? (end - begin + kTile - 1) / kTile : 0;  // prefix tiles
  const int nt = has_tree ? (a.n + kTile - 1) / kTile : 0;       // tree tiles
  // partial rows of this (sequence, split, kv head) are consecutive, in row
  // order m = node * grp + head within the group
  const int64_t prow0 = (((int64_t)b * a.nparts + s) * a.hkv + g) * a.rows;
  if (np == 0 && nt == 0) {
    // nothing to attend (uniform over the workgroup): an empty partial, so
    // that the combine reads every split without the prefix length
    for (int mb = 0; mb < RB; ++mb) {
      const int m = row0 + 16 * mb + col;
      if (active && m < a.rows && grp4 == 0) store_part_ml(a, a.part_ml + prow0 + m, make_float2(-INFINITY, 0.f));
    }
    goto done;
  }

  // ---- per-split tables staged in LDS --------------------------------------
  int bi0 = 0;         // partial: first block index of the split
  int fb_row = begin;  // a valid prefix row of this split (stands in for empty slots)
  if (has_tree && a.mask) {
#pragma unroll
    for (int u = 0; u < kMaskPer; ++u) {
      const int k = tid + u * kSplitThreads;
      if (k < mcnt) smask[k] = mw[u];
    }
  } else if (has_tree) {
    // The mask from the parent array (SpecBlock App. A.2: a node sees its
    // ancestors and itself), the rule tv_build_tree_mask applies: a malformed
    // array gives self-only rows and depth 0.  Thread t owns node t's row.
    if (tid == 0) s_bad = 0;
    if (tid < a.n) s_par[tid] = par_t;
    __syncthreads();
    if (tid < a.n && !(tid == 0 ? par_t == -1 : (par_t >= 0 && par_t < tid))) s_bad = 1;
    __syncthreads();
    const bool bad = s_bad != 0;
    // KV head 0 writes the a1 outputs: each row group its own nodes
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
          for (int w = 0; w < a.words; ++w)
            a.mask_out[((int64_t)b * a.n + tid) * a.words + w] = row[w];
        if (a.depth_out) a.depth_out[(int64_t)b * a.n + tid] = depth;
      }
    }
    if (bad && g == 0 && rg == 0 && tid == 0) raise_err(a.dev_err, TV_DERR_BAD_PARENT);
  }
  if (PARTIAL && np > 0) {
    bi0 = begin / a.block_size;
    const int bi1 = (end - 1) / a.block_size;
    // the plan keeps a split within kBlkCache blocks, all of them loaded above
    if (tid == 0) s_first = INT32_MAX;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kBlkPer; ++u) {
      const int k = tid + u * kSplitThreads;
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
      // no valid slot in the split's prefix range
      if (!has_tree) {
        // an empty partial
        if (err) raise_err(a.dev_err, err);
        for (int mb = 0; mb < RB; ++mb) {
          const int m = row0 + 16 * mb + col;
          if (active && m < a.rows && grp4 == 0) store_part_ml(a, a.part_ml + prow0 + m, make_float2(-INFINITY, 0.f));
        }
        goto done;
      }
      np = 0;
    } else {
      fb_row = sblk[first] * a.block_size;
    }
  }
  const int ntiles = np + nt;
  // whole prefix tiles (full mode): 32 consecutive rows each
  const int nfull = PARTIAL ? 0 : (end - begin) / kTile;
  // requested tiles that are this split's own first tiles
  const int skip = tree_own ? spec : max(0, min(spec, nfull));
  // cache row of prefix slot u, fb_row when the slot is empty
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

  // Tile it of the split: prefix tiles 0..np-1, then tree tiles.  Lanes past
  // the tree's last node re-read that node.
  auto dma_tile = [&](int slot, int it) {
    if (it < nfull) {
#pragma unroll
      for (int k = 0; k < DPT; ++k)
        dma16s(fdst[k] + slot * SLOT_B, fbase[k] + (int64_t)it * (kTile * ROWB), fvoff[k]);
      return;
    }
    const char* kb;
    const char* vb;
    int64_t off;
    if (it < np) {
      bool valid;
      off = (int64_t)slot_row(begin + it * kTile + dtok, valid) * ROWB;
      kb = kc;
      vb = vc;
    } else {
      off = (int64_t)min((it - np) * kTile + dtok, a.n - 1) * tree_rowb;
      kb = kt;
      vb = vt;
    }
#pragma unroll
    for (int k = 0; k < DPT; ++k)
      dma16(__builtin_amdgcn_readfirstlane(ring_base + slot * SLOT_B + ddst[k]),
            (dt[k] ? vb : kb) + off + dcol[k]);
  };
  // validity bits of the 32 slots of tile it (wave-uniform)
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

  // ---- LDS operand addressing ----------------------------------------------
  // K fragment (tb, dc): token 16tb + col, columns 32dc + 8grp4 .. +7, i.e.
  // block 2dc + grp4/2, half grp4&1 -> kbase + 2048 dc + 512 tb.
  const uint32_t kbase = 1024u * (grp4 >> 1) + 32u * col + 16u * (grp4 & 1);
  // V^T fragment (db, hf): ds_read_b64_tr_b16 gives, in each 16-lane group,
  // lane i element i%4 of the 8-byte pieces addressed by lanes 4k + i/4
  // (k = 0..3).  Lane 4kk + qq addresses token 16hf + 4grp4 + kk, columns
  // 16db + 4qq .. +3, so lane i receives column 16db + i of tokens
  // 16hf + 4grp4 + 0..3: k-slot j of lane group q is token 4q+j (j<4) or
  // 16+4q+(j-4), the tokens the lane holds in the S^T accumulators.
  // Address: vbase + 1024 db + 512 hf.
  const uint32_t vbase = TILE_B + 32u * (4 * grp4 + (col >> 2)) + 16u * ((col & 3) >> 1) + 8u * (col & 1);

  typedef __attribute__((address_space(3))) char lds_char;
  auto lds_at = [&](uint32_t addr) { return (lds_char*)(uintptr_t)addr; };
  auto kfrag = [&](uint32_t slot_addr, int tb, int dc) -> bf16x8 {
    return *(__attribute__((address_space(3))) const bf16x8*)lds_at(slot_addr + kbase + 2048 * dc + 512 * tb);
  };
  auto vfrag = [&](uint32_t slot_addr, int db) -> bf16x8 {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)lds_at(slot_addr + vbase + 1024 * db));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)lds_at(slot_addr + vbase + 1024 * db + 512));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- per-tile math --------------------------------------------------------
  // S^T for one tile: sacc[tb][mb][r] = score of token tb*16 + 4*grp4 + r,
  // row row0 + 16*mb + col.  The first k-step starts from a zero accumulator.
  auto qk_mfma = [&](const bf16x8 (&kf)[DC][2], f32x4 (&sacc)[2][RB], int dc) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int mb = 0; mb < RB; ++mb)
        sacc[tb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            kf[dc][tb], qf[mb][dc], dc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[tb][mb], 0, 0, 0);
  };
  auto qk_tile = [&](int slot, f32x4 (&sacc)[2][RB]) {
    const uint32_t sa = ring_base + slot * SLOT_B;
    bf16x8 kf[DC][2];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) kf[dc][tb] = kfrag(sa, tb, dc);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qk_mfma(kf, sacc, dc);
  };

  // -inf for tokens outside the tile's valid set (and, in the tree block,
  // outside the row's ancestor set)
  auto mask_tile = [&](int it, f32x4 (&sacc)[2][RB]) {
    const uint32_t vbits = tile_bits(it);
    const bool tt = it >= np;  // a tree tile
    if (!tt && vbits == 0xFFFFFFFFu) return;
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) {
      uint32_t allow = vbits;
      if (tt) {
        const int m = row0 + 16 * mb + col;
        allow &= m < a.rows ? smask[(m / a.grp - node0) * a.words + (it - np)] : 0u;
      }
      allow >>= 4 * grp4;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (!((allow >> (16 * tb + r)) & 1u)) sacc[tb][mb][r] = -INFINITY;
    }
  };

  f32x4 o[RB][DB];
  float lpart[RB];    // this lane's share of the row sum of p (fp32, before rounding)
  float mref[RB];     // reference max per row (log2 units), -inf until set

  // p = 2^(s*c - mref) of one tile for row block mb, packed as the PV B
  // operand.  With TRACK (first tile) the reference is taken from this tile
  // where unset.
  auto softmax_block = [&](f32x4 (&sacc)[2][RB], int mb, auto track_tag) -> bf16x8 {
    if (decltype(track_tag)::value) {
      float mx = fmaxf(fmaxf(fmaxf(sacc[0][mb][0], sacc[0][mb][1]), fmaxf(sacc[0][mb][2], sacc[0][mb][3])),
                       fmaxf(fmaxf(sacc[1][mb][0], sacc[1][mb][1]), fmaxf(sacc[1][mb][2], sacc[1][mb][3])));
      mx = xmax16_32(mx) * a.c;
      mref[mb] = mref[mb] == -INFINITY ? mx : mref[mb];
    }
    const float muse = (mref[mb] == -INFINITY) ? 0.f : mref[mb];
    float pv[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        pv[tb * 4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tb][mb][r], a.c, -muse));
    lpart[mb] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (bf16)pv[e];
    return pb;
  };

  auto pv_mfma = [&](const bf16x8 (&vf)[DB], const bf16x8 (&pb)[RB], int db) {
#pragma unroll
    for (int mb = 0; mb < RB; ++mb)
      o[mb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pb[mb], o[mb][db], 0, 0, 0);
  };

  // ---- pipeline -------------------------------------------------------------
  // Tile t lives in ring slot t % 4.  Tiles 0-2 are requested before the
  // loop (or earlier, see above); step s waits for tile s+1 (the older of
  // its two outstanding tiles, or the last one), passes the workgroup
  // barrier (after which the slot of tile s-1 is free) and asks for tile
  // s+3.  No tile past the last is requested: a short split ends without a
  // memory round trip for data it never uses.  The math of a tile is split
  // in two halves:
  //   R(s): read the operands of M(s) from LDS (K of tile s+1, V of tile s),
  //         mask and softmax the scores S(s);
  //   M(s): QK of tile s+1 -> S(s+1), then PV of tile s.
  // Waves 0-3 (one per SIMD) run R(s) then M(s) in step s; waves 4-7 run
  // M(s-1) then R(s).  On every SIMD one wave is then on the matrix core
  // while the other uses LDS and the VALU.  All LDS reads of tile s finish
  // before the barrier of step s+1, so the slot reuse above is safe.
  const bool lead = wave < kWaves / 2;

  auto run = [&](int skip) {
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) {
      lpart[mb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[mb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // The first `skip` tiles were requested before the prefix length was
    // known and have landed.  Otherwise wait for tile 0, the oldest of the
    // min(3, ntiles) requests.
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (t >= skip && t < ntiles) dma_tile(t, t);
    if (skip == 0) {
      if (ntiles >= 3) vm_wait<2 * DPT>();
      else if (ntiles == 2) vm_wait<DPT>();
      else vm_wait<0>();
    }
    lds_barrier();

    f32x4 sA[2][RB], sB[2][RB];
    bf16x8 kf[DC][2], vf[DB], pb[RB];
    if (active) qk_tile(0, sA);

    // operand reads of M(s): K of tile s+1, V of tile s
    auto read_k = [&](int s) {
      const uint32_t ka = ring_base + ((s + 1) % kRing) * SLOT_B;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) kf[dc][tb] = kfrag(ka, tb, dc);
    };
    auto read_v = [&](int s) {
      const uint32_t va = ring_base + (s % kRing) * SLOT_B;
#pragma unroll
      for (int db = 0; db < DB; ++db) vf[db] = vfrag(va, db);
    };
    auto qk = [&](f32x4 (&nxt)[2][RB]) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qk_mfma(kf, nxt, dc);
    };
    auto pv = [&]() {
#pragma unroll
      for (int db = 0; db < DB; ++db) pv_mfma(vf, pb, db);
    };
#define TV_SCHED_FENCE __builtin_amdgcn_sched_barrier(0)
    // b1: tile s+1 has landed for every wave; the slot of tile s-1 is free
    auto sync = [&](int s) {
      // requests are in tile order, so tile s+1 has landed once at most the
      // requests of tile s+2 (if there is one) are outstanding
      if (s + 2 < ntiles) vm_wait<DPT>();
      else vm_wait<0>();
      lds_barrier();
      if (s + 3 < ntiles && s + 3 >= skip) dma_tile((s + 3) % kRing, s + 3);
    };
    // b2: mid-step barrier that only keeps the two groups half a step apart
    // (no data hand-off: outstanding LDS reads may cross it).  With one row
    // block per wave the groups are left to drift instead: measured on
    // MI355X, dropping it takes 4 % off the 16 x 32-node batch and 2 % off
    // the 8B layer (one block each) but adds 12 % at the 60000-token prefix
    // (two blocks).
    auto half_sync = [&]() {
      if (RB == 1) return;
      TV_SCHED_FENCE;
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      TV_SCHED_FENCE;
    };
    // R(s): the operand reads of M(s) and the mask of S(s): LDS work and
    // little VALU.  The wave runs it at raised priority, so that its reads
    // issue ahead of the other wave's softmax on the same SIMD (measured on
    // MI355X: 5 % off the 60000-token prefix, neutral at one row block).
    auto R = [&](int s, f32x4 (&cur)[2][RB]) {
      __builtin_amdgcn_s_setprio(1);
      read_k(s);
      read_v(s);
      TV_SCHED_FENCE;
      mask_tile(s, cur);
      TV_SCHED_FENCE;
      __builtin_amdgcn_s_setprio(0);
    };
    // M(s): the softmax of S(s) interleaved with the QK products of tile s+1
    // (one MFMA, then up to six VALU instructions that issue while it runs;
    // six measured ~1.5 % faster than four at the 60000-token prefix), then
    // the PV products of tile s.  The QK of the tile after the last one reads
    // whatever its slot holds; its result is never used.
    auto M = [&](auto track_tag, f32x4 (&cur)[2][RB], f32x4 (&nxt)[2][RB]) {
      TV_SCHED_FENCE;
#pragma unroll
      for (int mb = 0; mb < RB; ++mb) pb[mb] = softmax_block(cur, mb, track_tag);
      qk(nxt);
#pragma unroll
      for (int i = 0; i < 2 * RB * DC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);  // VALU incl. transcendental
      }
      TV_SCHED_FENCE;
      pv();
      TV_SCHED_FENCE;
    };
    // Each group runs its own loop (separate register allocation); both pass
    // the same barriers (ntiles + 1 of b1, and as many of b2 with two row
    // blocks).  S(s) of even s lives in sA, odd in sB.
    if (lead) {
      // b1 R(s) b2 M(s)
      auto step = [&](auto track_tag, int s, f32x4 (&cur)[2][RB], f32x4 (&nxt)[2][RB]) {
        sync(s);
        const bool work = active && s < ntiles;
        if (work) R(s, cur);
        half_sync();
        if (work) M(track_tag, cur, nxt);
      };
      step(std::true_type{}, 0, sA, sB);
      for (int s = 1; s <= ntiles; s += 2) {
        step(std::false_type{}, s, sB, sA);
        if (s + 1 <= ntiles) step(std::false_type{}, s + 1, sA, sB);
      }
    } else {
      // b1 M(s-1) b2 R(s): M(s-1) consumes S(s-1) in prev and writes S(s)
      // into cur, which R(s) masks
      auto step = [&](auto track_tag, int s, f32x4 (&prev)[2][RB], f32x4 (&cur)[2][RB]) {
        sync(s);
        if (active) M(track_tag, prev, cur);
        half_sync();
        if (active && s < ntiles) R(s, cur);
      };
      sync(0);
      half_sync();
      if (active) R(0, sA);
      step(std::true_type{}, 1, sA, sB);  // ntiles >= 1
      for (int s = 2; s <= ntiles; s += 2) {
        step(std::false_type{}, s, sB, sA);
        if (s + 1 <= ntiles) step(std::false_type{}, s + 1, sA, sB);
      }
    }
#undef TV_SCHED_FENCE
    lds_barrier();
  };

  // Flat schedule (OCC = 4): per tile, one barrier, then each wave reads
  // its K operands, runs QK, the softmax, reads its V operands and runs
  // PV.  Tile t lives in slot t % 4; tiles s+1 and s+2 are in flight while
  // tile s is used, and tile s+3 is requested once every wave has passed
  // the barrier of step s (all reads of tile s-1, in slot (s+3) % 4, done).
  auto run_flat = [&](int skip) {
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) {
      lpart[mb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[mb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (t >= skip && t < ntiles) dma_tile(t, t);
    for (int s = 0; s < ntiles; ++s) {
      // requests are in tile order: tile s has landed once at most those
      // of tiles s+1 and s+2 are outstanding
      if (s + 2 < ntiles) vm_wait<2 * DPT>();
      else if (s + 1 < ntiles) vm_wait<DPT>();
      else vm_wait<0>();
      lds_barrier();
      if (s + 3 < ntiles && s + 3 >= skip) dma_tile((s + 3) % kRing, s + 3);
      if (!active) continue;
      f32x4 sc[2][RB];
      qk_tile(s % kRing, sc);
      mask_tile(s, sc);
      bf16x8 pbl[RB];
      if (s == 0) {
#pragma unroll
        for (int mb = 0; mb < RB; ++mb) pbl[mb] = softmax_block(sc, mb, std::true_type{});
      } else {
#pragma unroll
        for (int mb = 0; mb < RB; ++mb) pbl[mb] = softmax_block(sc, mb, std::false_type{});
      }
      const uint32_t va = ring_base + (s % kRing) * SLOT_B;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 v = vfrag(va, db);
#pragma unroll
        for (int mb = 0; mb < RB; ++mb)
          o[mb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pbl[mb], o[mb][db], 0, 0, 0);
      }
    }
    lds_barrier();
  };

#pragma unroll
  for (int mb = 0; mb < RB; ++mb) mref[mb] = -INFINITY;
  if constexpr (OCC == 4) run_flat(skip);
  else run(skip);

  // ---- overflow check; exact two-pass recompute when needed --------------
  __shared__ int s_redo;
  if (tid == 0) s_redo = 0;
  __syncthreads();
  if (active) {
    bool bad = false;
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) {
      const float l = xsum16_32(lpart[mb]);
      // One finiteness test of the sum of the lane's outputs: it is not
      // finite if any output is (or if the sum overflows, which only asks
      // for the exact recompute).  A compare per element would put 16 DB
      // VALU-to-scalar dependencies in series here.
      float acc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = o[mb][0][e];
#pragma unroll
        for (int db = 1; db < DB; ++db) acc[e] += o[mb][db][e];
      }
      const bool fin = __builtin_isfinite((acc[0] + acc[1]) + (acc[2] + acc[3]));
      const bool real = row0 + 16 * mb + col < a.rows;
      // a row whose first tile was fully masked used 0 as its reference:
      // recompute it with the exact max as well
      bad |= real && (mref[mb] == -INFINITY ? l > 0.f : !(l <= kSumMax && fin));
    }
    if (__ballot(bad) && lane == 0) s_redo = 1;
  }
  __syncthreads();
  if (s_redo) {
    // QK-only pre-pass for the exact row max (single-buffered, rare path)
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) mref[mb] = -INFINITY;
    for (int it = 0; it < ntiles; ++it) {
      dma_tile(0, it);
      vm_wait<0>();
      lds_barrier();
      if (active) {
        f32x4 sc[2][RB];
        qk_tile(0, sc);
        mask_tile(it, sc);
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
      lds_barrier();
    }
    if constexpr (OCC == 4) run_flat(0);
    else run(0);
  }
  if (err) raise_err(a.dev_err, err);

  // ---- partial write -------------------------------------------------------
  // Each row's output is divided by its own sum and stored as bf16, its
  // (reference max, sum) pair in fp32.  A wave stages its 16 RB rows in its
  // own part of the (now idle) ring and writes them back as contiguous 1 KB
  // runs.  Staging address of row r, 32-byte chunk ch: r * 2D + 32 (ch ^ z(r))
  // with z(r) = (r / RPB) mod DB, so that the 16 rows written by one
  // instruction, and the rows read back by one, cover all 64 banks.
  if (!active) goto done;
  {
    constexpr int RPB = 128 / D;  // rows per 256-byte row of banks
    constexpr int RPI = 512 / D;  // rows per 1 KB store
    constexpr int QPR = D / 8;    // 16-byte pieces per row
    static_assert(kWaves * 32 * RB * D <= kRing * SLOT_B, "staging fits the ring");
    const uint32_t stage = ring_base + wave * (32 * RB * D);
#pragma unroll
    for (int mb = 0; mb < RB; ++mb) {
      const float l = xsum16_32(lpart[mb]);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int r = 16 * mb + col;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[mb][db][e] * inv);
        *(__attribute__((address_space(3))) bf16x4*)lds_at(
            stage + r * (2 * D) + 32 * (db ^ ((r / RPB) & (DB - 1))) + 8 * grp4) = v;
      }
      if (grp4 == 0 && row0 + r < a.rows) store_part_ml(a, a.part_ml + prow0 + row0 + r, make_float2(mref[mb], l));
    }
#pragma unroll
    for (int j = 0; j < 16 * RB / RPI; ++j) {
      const int r = j * RPI + lane / QPR;
      const int q = lane % QPR;
      const bf16x8 v = *(__attribute__((address_space(3))) const bf16x8*)lds_at(
          stage + r * (2 * D) + 32 * ((q >> 1) ^ ((r / RPB) & (DB - 1))) + 16 * (q & 1));
      if (row0 + r < a.rows) store_part_o(a, a.part_o + (prow0 + row0 + r) * D + 8 * q, v);
    }
  }
  }
done:
  // (every path of the split work ends here: the signal below counts the
  // workgroup's partials, empty ones included)
  if (a.sync) split_done(a, bg);
}


// The merge of the split partials (combine_rows in tv_attn_common.h), NR
// rows per wave (rows (b * n + i) * hq + h), its lanes splitting each row's
// partials; launched with NR = 1 for rows with more than 8 partials.
template <int D, int NR>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnArgs a) {
  const int64_t rows_total = (int64_t)a.batch * a.n * a.hq;
  const int64_t r0 = ((int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64) * NR;
  if (r0 >= rows_total) return;
  int64_t ids[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) ids[r] = r0 + r < rows_total ? r0 + r : -1;
  combine_rows<D, NR, false>(a, ids, threadIdx.x & 63);
}

// The merge for rows with at most KMAX partials: lane r * C + c of a wave
// (C = D / 8) owns the 8 output elements of chunk c of row r, so a wave
// covers 64 / C rows.  Each lane loads that chunk of every partial of its
// row at once (indices clamped to the last partial, so every load is in
// bounds and none waits on a branch), then merges them in partial order:
// m = max_s m_s, w_s = 2^(m_s - m) l_s, o = sum_s w_s o_s / sum_s w_s,
// lse = (m + log2 sum_s w_s) ln 2.  No value crosses lanes.  An empty
// partial (m = -inf) weighs 0 and its output is not used.
template <int D, int KMAX>
__global__ __launch_bounds__(kThreads) void attn_combine_lane_kernel(AttnArgs a) {
  constexpr int C = D / 8;
  constexpr int RPW = kWave / C;  // rows per wave
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane / C, c = lane % C;
  const int64_t rows_total = (int64_t)a.batch * a.n * a.hq;
  const int64_t row = ((int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave) * RPW + r;
  if (row >= rows_total) return;  // per lane: nothing below crosses lanes
  // row = (b * n + i) * hq + h; partial rows of (b, split, g) are consecutive
  // in m = i * grp + h % grp (32-bit: the descriptor check keeps B·N·Hq < 2^31)
  const uint32_t id = (uint32_t)row;
  const uint32_t bi = id / (uint32_t)a.hq;
  const int h = (int)(id - bi * (uint32_t)a.hq);
  const uint32_t bq = bi / (uint32_t)a.n;
  const int i = (int)(bi - bq * (uint32_t)a.n);
  const int g = h / a.grp;
  const int64_t p0 = ((int64_t)bq * a.nparts * a.hkv + g) * a.rows + i * a.grp + h % a.grp;
  const int64_t stride = (int64_t)a.hkv * a.rows;  // partial rows between splits
  const int cnt = a.nparts;
  float2 ml[KMAX];
  bf16x8 ov[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int64_t pi = p0 + (int64_t)(k < cnt ? k : cnt - 1) * stride;
    ml[k] = load_ml<false>(a.part_ml + pi);
    ov[k] = load_o<false>(a.part_o + pi * D + 8 * c);
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (k < cnt) m = fmaxf(m, ml[k].x);
  bf16x8 res = bf16x8{};
  float lse_v = -INFINITY;
  if (m != -INFINITY) {
    float l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (k < cnt && ml[k].x != -INFINITY) {
        const float w = __builtin_amdgcn_exp2f(ml[k].x - m) * ml[k].y;
        l += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w, (float)ov[k][e], acc[e]);
      }
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] = (bf16)(acc[e] * inv);
    lse_v = (m + log2f(l)) * 0.69314718055994530942f;
  }
  *reinterpret_cast<bf16x8*>(a.out + row * D + 8 * c) = res;
  if (c == 0 && a.lse) a.lse[row] = lse_v;
}

template <int D, int RB, int OCC>
void launch_split(const AttnArgs& args, dim3 grid, hipStream_t stream) {
  if (args.max_blocks)
    hipLaunchKernelGGL((attn_split_kernel<D, RB, true, OCC>), grid, dim3(kSplitThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, RB, false, OCC>), grid, dim3(kSplitThreads), 0, stream, args);
}

template <int D>
void launch_split_rb(int rb, int wg_per_cu, const AttnArgs& args, dim3 grid, hipStream_t stream) {
  if (rb == 1 && wg_per_cu == 2)
    launch_split<D, 1, 4>(args, grid, stream);
  else if (rb == 1)
    launch_split<D, 1, 2>(args, grid, stream);
  else
    launch_split<D, 2, 2>(args, grid, stream);
}

}  // namespace

namespace {

// Plan with at most `max_rb` 16-row blocks per wave; *crit receives the
// tiles of the longest workgroup.
AttnPlan plan_rows(const tv_attn_desc& d, int cu_count, int max_rb, int* crit) {
  AttnPlan p{};
  const int grp = d.n_q_heads / d.n_kv_heads;
  p.rows = d.n_nodes * grp;
  // a workgroup covers 16 * kWaves * RB rows, RB in {1, 2}
  p.row_groups = (p.rows + 16 * kWaves * max_rb - 1) / (16 * kWaves * max_rb);
  const int per_group = (p.rows + p.row_groups - 1) / p.row_groups;
  p.row_blocks = per_group <= 16 * kWaves ? 1 : 2;
  p.prefix_slots = d.max_blocks ? d.max_blocks * d.block_size : d.max_prefix_len;
  const int units = d.batch * d.n_kv_heads * p.row_groups;
  const int tree_tiles = (d.n_nodes + kTile - 1) / kTile;
  auto chunk_for = [&](int splits) {
    int c = p.prefix_slots > 0 ? (p.prefix_slots + splits - 1) / splits : kTile;
    c = ((c + kTile - 1) / kTile) * kTile;
    if (d.max_blocks) {
      // the block ids a split touches must fit its LDS table
      const int64_t lim =
          std::max<int64_t>(kTile, ((kBlkCache - 2) * (int64_t)d.block_size / kTile) * kTile);
      if (c > lim) c = (int)lim;
    }
    return c;
  };
  // tiles on the longest workgroup: with the tree folded into the last
  // non-empty split, or with the tree in a workgroup of its own
  auto critical = [&](int splits, bool sep) {
    const int c = chunk_for(splits);
    const int full = (c + kTile - 1) / kTile;
    if (sep) return std::max(full, tree_tiles);
    const int ns = p.prefix_slots > 0 ? (p.prefix_slots + c - 1) / c : 1;
    const int last = p.prefix_slots - (ns - 1) * c;
    return std::max(full, (std::max(last, 0) + kTile - 1) / kTile + tree_tiles);
  };
  int splits;
  bool sep;
  if (d.num_splits > 0) {
    splits = d.num_splits;
    sep = (int64_t)units * (splits + 1) <= cu_count;
  } else if (d.tree_placement != TV_TREE_AUTO) {
    splits = std::max(std::min(std::max(cu_count / units, 1),
                               std::max((p.prefix_slots + kMinChunk - 1) / kMinChunk, 1)), 1);
    sep = d.tree_placement == TV_TREE_OWN_WORKGROUP;
  } else {
    // one workgroup per CU (two waves per SIMD): a grid of at most cu_count
    // workgroups runs in a single round
    const int smax = std::max(cu_count / units, 1);
    const int cap = std::max((p.prefix_slots + kMinChunk - 1) / kMinChunk, 1);
    const int s_fold = std::min(smax, cap);
    const int s_sep = std::min(smax - 1, cap);
    sep = s_sep >= 1 && critical(s_sep, true) <= critical(s_fold, false);
    splits = sep ? s_sep : s_fold;
  }
  p.chunk = chunk_for(splits);
  p.splits = p.prefix_slots > 0 ? (p.prefix_slots + p.chunk - 1) / p.chunk : 1;
  if (d.tree_placement != TV_TREE_AUTO) sep = d.tree_placement == TV_TREE_OWN_WORKGROUP;
  else if ((int64_t)units * (p.splits + 1) > std::max(cu_count, units * 2)) sep = false;
  p.tree_sep = sep ? 1 : 0;
  *crit = critical(splits, sep);
  const size_t parts = (size_t)d.batch * (p.splits + p.tree_sep) * d.n_nodes * d.n_q_heads;
  p.ws_o_bytes = ((parts * d.head_dim * sizeof(uint16_t) + 255) / 256) * 256;  // bf16
  p.ws_ml_bytes = ((parts * sizeof(float2) + 255) / 256) * 256;
  p.ws_sync_bytes = TV_ATTN_WS_COUNTER_BYTES;
  return p;
}

}  // namespace

// Rows per wave: two 16-row blocks halve the LDS operand bytes per MFMA and
// the workgroups that read each K/V tile, one block halves a tile's matrix
// work per wave.  With one block a 32-token tile takes a workgroup about
// 0.65 as long (measured on MI355X: 15.2 vs 17.4 us for the 1000-token
// prefix of an 8B layer, where each workgroup has 4 tiles either way; at a
// 60000-token prefix, where the grid is already full, the doubled
// workgroups lose).  The plan with the shorter longest workgroup wins.
// The 16-row schedule merges in a second launch: measured on MI355X with
// the 1000-token prefix of an 8B layer, its merge workgroups (dispatched
// beside the splits, spinning from the start) ended the launch 21.5 us
// after its start, against 11.4 + 4.7 us for the split and merge launches.
// Merge workgroups of the in-launch merge: `waves` waves of rpw rows each
// (rows go two to a wave's memory round trip, so rpw is even), about
// `slots` workgroups over the whole chip.
void set_merge_shape(const tv_attn_desc& d, int waves, int slots, AttnPlan* p) {
  const int64_t all_rows = (int64_t)d.batch * d.n_kv_heads * p->rows;
  const int64_t per = (all_rows + (int64_t)waves * slots - 1) / ((int64_t)waves * slots);
  p->rpw = (int)std::max<int64_t>(2, (per + 1) / 2 * 2);
  p->ncw_unit = (p->rows + waves * p->rpw - 1) / (waves * p->rpw);
}

AttnPlan plan_attention(const tv_attn_desc& d, int cu_count) {
  int crit2 = 0, crit1 = 0;
  if (d.kernel == TV_ATTN_KERNEL_WIDE) {
    // 32-row MFMA tiles, one or two per wave: 128 or 256 rows per workgroup
    // (one workgroup per CU)
    AttnPlan p = plan_rows(d, cu_count, 2, &crit2);
    p.kind = TV_ATTN_KERNEL_WIDE;
    set_merge_shape(d, 4, cu_count, &p);
    p.merge_in_launch = true;
    return p;
  }
  // 16-row MFMA tiles, one workgroup per CU (two waves per SIMD)
  AttnPlan p2 = plan_rows(d, cu_count, 2, &crit2);
  p2.kind = TV_ATTN_KERNEL_SPLIT16;
  set_merge_shape(d, kWaves, 2 * cu_count, &p2);
  // One block per wave on the flat schedule, up to two workgroups per CU
  // (four waves per SIMD).  Measured on MI355X against the plans above
  // (attention call, same box): alone on its CU the flat schedule is 3-4 %
  // faster than the ping-pong at one block per wave (8-node tree 8.0 ->
  // 7.7 us, 8B layer 13.7 -> 13.2 us).  Two workgroups on a CU take about
  // twice a lone one's time per tile (16 x 32-node batch: 13 tiles in
  // 33.2 us against 25 in 31.6), i.e. ~1.15 of a two-block tile (60000-token
  // prefix: 88.7 against 82.5 us at the same tile count), which still wins
  // where it shortens the longest workgroup enough (83-node tree over 4096
  // tokens: 7 tiles against 9, 21.4 against 22.6 us).
  AttnPlan p1 = plan_rows(d, 2 * cu_count, 1, &crit1);
  p1.kind = TV_ATTN_KERNEL_SPLIT16;
  p1.wg_per_cu = 2;
  set_merge_shape(d, kWaves, 2 * cu_count, &p1);
  const bool shared = (int64_t)(p1.splits + p1.tree_sep) * d.batch * d.n_kv_heads * p1.row_groups > cu_count;
  if (p2.row_blocks == 1) return (shared ? 2 * crit1 < crit2 : crit1 <= crit2) ? p1 : p2;
  return (shared ? 23 * crit1 < 20 * crit2 : 13 * crit1 < 20 * crit2) ? p1 : p2;
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
  a.parents = p.parents;
  a.mask_out = p.mask_out;
  a.depth_out = p.depth_out;
  a.block_idx = p.block_idx;
  a.n_blocks = p.n_blocks;
  // workspace: [merge counters][partial outputs][partial (max, sum)]
  char* const ws = reinterpret_cast<char*>(workspace);
  a.part_o = reinterpret_cast<bf16*>(ws + plan.ws_sync_bytes);
  a.part_ml = reinterpret_cast<float2*>(ws + plan.ws_sync_bytes + plan.ws_o_bytes);
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
  a.tree_sep = plan.tree_sep;
  a.nparts = plan.splits + plan.tree_sep;
  a.row_groups = plan.row_groups;
  a.rows = plan.rows;
  const float scale = d.softmax_scale > 0.f ? d.softmax_scale : 1.f / sqrtf((float)d.head_dim);
  a.c = scale * 1.44269504088896340736f;

  // split workgroups, then (when the counters hold every unit) the merge
  // workgroups of the same launch; else a second launch merges
  a.nsplit_wg = (plan.splits + plan.tree_sep) * d.batch * d.n_kv_heads * plan.row_groups;
  const int64_t units_bg = (int64_t)d.batch * d.n_kv_heads;
  const bool merge_in_launch =
      plan.merge_in_launch && 2 * units_bg * (int64_t)sizeof(int) <= (int64_t)plan.ws_sync_bytes;
  a.sync = merge_in_launch ? reinterpret_cast<int*>(ws) : nullptr;
  a.ncw_unit = plan.ncw_unit;
  a.rpw = plan.rpw;
  const unsigned grid = (unsigned)(a.nsplit_wg + (merge_in_launch ? units_bg * plan.ncw_unit : 0));
  if (plan.kind == TV_ATTN_KERNEL_WIDE) {
    hipError_t e = launch_wide(a, d.head_dim, plan.row_blocks, grid, stream);
    if (e != hipSuccess || merge_in_launch) return e;
  } else {
    if (d.head_dim == 128)
      launch_split_rb<128>(plan.row_blocks, plan.wg_per_cu, a, dim3(grid), stream);
    else
      launch_split_rb<64>(plan.row_blocks, plan.wg_per_cu, a, dim3(grid), stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || merge_in_launch) return e;
  }

  const int64_t rows_total = (int64_t)d.batch * d.n_nodes * d.n_q_heads;
  if (a.nparts <= 8) {
    // Few partials per row: one lane per output chunk, all of its row's
    // partials loaded at once, so the whole grid is one round of waves
    // (measured on MI355X, per attention call: 11.7 -> 8.0 us for the
    // 8-node tree over 256 tokens, 42.2 -> 35.1 us for 16 ragged
    // sequences; with the 9 partials of the 8B layer the 16-partial form
    // was slower, 14.0 -> 16.5 us, so more partials take the wave-per-row
    // merge below).
    const int64_t per_wg = (int64_t)(kThreads / 64) * (64 / (d.head_dim / 8));
    const dim3 lgrid((unsigned)((rows_total + per_wg - 1) / per_wg));
    const bool k4 = a.nparts <= 4;
    if (d.head_dim == 128) {
      if (k4) hipLaunchKernelGGL((attn_combine_lane_kernel<128, 4>), lgrid, dim3(kThreads), 0, stream, a);
      else hipLaunchKernelGGL((attn_combine_lane_kernel<128, 8>), lgrid, dim3(kThreads), 0, stream, a);
    } else {
      if (k4) hipLaunchKernelGGL((attn_combine_lane_kernel<64, 4>), lgrid, dim3(kThreads), 0, stream, a);
      else hipLaunchKernelGGL((attn_combine_lane_kernel<64, 8>), lgrid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
  }
  // one wave per row, its lanes splitting the partials
  const int64_t per_wg = kThreads / 64;
  const dim3 cgrid((unsigned)((rows_total + per_wg - 1) / per_wg));
  if (d.head_dim == 128)
    hipLaunchKernelGGL((attn_combine_kernel<128, 1>), cgrid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<64, 1>), cgrid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tv
