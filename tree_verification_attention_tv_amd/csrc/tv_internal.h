// Internal declarations shared by the libtreeverify HIP sources (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treeverify.h"

namespace tv {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// launch wrappers implemented in the kernel sources; each returns the HIP
// launch status.  Arguments have been validated by the API layer.
// ---------------------------------------------------------------------------

hipError_t launch_build_mask(const int32_t* parents, int batch, int n, uint32_t* mask,
                             int32_t* depth, int32_t* dev_err, hipStream_t stream);

struct AttnPlan {
  int rows;          // query rows per (sequence, kv head) = n_nodes * group
  int row_blocks;    // 16-row MFMA blocks per wave (1..4)
  int row_groups;    // workgroups sharing one (sequence, kv head, split) in rows
  int splits;        // prefix splits
  int tree_sep;      // 1: the tree block has a workgroup of its own (split index `splits`);
                     // 0: it runs in the last non-empty prefix split
  int chunk;         // prefix slots per split (multiple of the 32-token tile)
  int wg_per_cu;     // 16-row schedule: 2 = one-block waves, four per SIMD; else one workgroup per CU
  int prefix_slots;  // upper bound of prefix slots per sequence
  int kind;          // TV_ATTN_KERNEL_SPLIT16 or TV_ATTN_KERNEL_WIDE
  size_t ws_o_bytes, ws_ml_bytes;
  size_t ws_sync_bytes;  // counters of the in-launch merge, first in the workspace (zero between calls)
  int ncw_unit;          // 32-row kernel: merge workgroups per (sequence, kv head)
  int rpw;               // rows merged per wave
  bool merge_in_launch;  // merge workgroups in the split launch (else a second launch)
  size_t ws_bytes() const { return ws_o_bytes + ws_ml_bytes + ws_sync_bytes; }
};

AttnPlan plan_attention(const tv_attn_desc& d, int cu_count);
// Argument checks of tv_tree_attention other than the workspace size, then
// the plan for the current device; *empty: batch 0, nothing to launch.
tv_status prepare_attention(const tv_attn_desc* desc, const tv_attn_ptrs* ptrs,
                            const void* workspace, AttnPlan* plan, bool* empty);

hipError_t launch_attention(const tv_attn_desc& d, const AttnPlan& plan, const tv_attn_ptrs& p,
                            void* workspace, int32_t* dev_err, hipStream_t stream);

struct AcceptPlan {
  int chunks;        // vocabulary chunks per row
  int64_t chunk_len; // elements per chunk
  size_t ws_bytes;
};

AcceptPlan plan_accept(int batch, int n, int64_t vocab);

// commit of the accepted rows folded into the acceptance's walk kernel
struct CommitTarget {
  const void* k_tree;
  const void* v_tree;
  const int32_t* prefix_len;
  int32_t* new_prefix_len;
  void* k_cache;
  void* v_cache;
  int64_t seq_stride;  // elements
  int cap, hkv, d;
  int layers;                 // >= 1; layer l's tensors at the strides below (elements)
  int64_t tree_layer_stride, cache_layer_stride;
};

hipError_t launch_accept(const void* logits, tv_dtype dt, int64_t vocab, int64_t row_stride,
                         const int32_t* parents, const int32_t* draft, int batch, int n,
                         int32_t* target_argmax, int32_t* accept_len, int32_t* accept_path,
                         int32_t* bonus, void* workspace, const AcceptPlan& plan,
                         int32_t* dev_err, hipStream_t stream,
                         const CommitTarget* commit = nullptr);

hipError_t launch_commit(const void* k_tree, const void* v_tree, const int32_t* path,
                         const int32_t* accept_len, const int32_t* prefix_len,
                         int32_t* new_prefix_len, void* k_cache, void* v_cache,
                         int64_t seq_stride, int cap, int batch, int n, int hkv, int d,
                         int layers, int64_t tree_layer_stride, int64_t cache_layer_stride,
                         int32_t* dev_err, hipStream_t stream);

AcceptPlan plan_stochastic(int batch, int n, int64_t vocab);

hipError_t launch_stochastic(const void* logits, tv_dtype dt, int64_t vocab, int64_t row_stride,
                             const int32_t* parents, const int32_t* draft, int batch, int n,
                             float temperature, int top_k, float top_p, uint64_t seed0,
                             uint64_t seed1, uint64_t step, int32_t* accept_len,
                             int32_t* accept_path, int32_t* bonus, void* workspace,
                             const AcceptPlan& plan, int32_t* dev_err, hipStream_t stream);

struct SelectPlan {
  int nb_cap;        // summary records per (sequence, kv head): ceil(capacity / block_size)
  int nb_max;        // blocks that can hold prefix tokens: ceil(min(max_prefix, cap) / bs)
  int chunk;         // blocks per scoring workgroup (multiple of 16)
  int chunks;        // scoring workgroups per (sequence, kv head)
  int part_stride;   // floats per (sequence, kv head) row of partial scores (multiple of 4)
  int kpt;           // blocks per selection thread (4, 16 or 32); 0: too many blocks
  size_t ws_part_bytes;
};

SelectPlan plan_select(const tv_select_desc& d, int cu_count);

hipError_t launch_summaries(const void* k_cache, int64_t seq_stride, int cap, int batch, int hkv,
                            int d, int bs, const int32_t* prefix_len, const int32_t* first_token,
                            int max_tokens, void* summaries, int32_t* dev_err, hipStream_t stream);

hipError_t launch_select(const tv_select_desc& d, const SelectPlan& plan, const void* q,
                         const void* summaries, const int32_t* prefix_len, int32_t* block_idx,
                         int32_t* n_blocks, float* scores, void* workspace, int32_t* dev_err,
                         hipStream_t stream);

}  // namespace tv
