// C ABI of libtreeverify: host-side validation, launch planning and error
// mapping.  No allocation, no host synchronisation, no per-call state.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>

#include "tv_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

int cu_count_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tv_status launch_status(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_LAUNCH; }

// Layer arguments of the commit calls.  With several layers the strides are
// positive whole 16-byte vectors, and new_prefix_len may not overlap
// prefix_len: a later layer's workgroup still reads prefix_len after layer
// 0 has written the new lengths.
tv_status check_layers(int32_t n_layers, int64_t tree_layer_stride, int64_t cache_layer_stride,
                       const int32_t* prefix_len, const int32_t* new_prefix_len, int32_t batch) {
  if (n_layers < 1 || n_layers > TV_MAX_LAYERS) return TV_ERR_SHAPE;
  if (n_layers == 1) return TV_OK;
  if (tree_layer_stride <= 0 || cache_layer_stride <= 0 || tree_layer_stride % 8 ||
      cache_layer_stride % 8)
    return TV_ERR_SHAPE;
  const uintptr_t a = reinterpret_cast<uintptr_t>(prefix_len);
  const uintptr_t b = reinterpret_cast<uintptr_t>(new_prefix_len);
  const uintptr_t len = (uintptr_t)batch * sizeof(int32_t);
  if (a < b + len && b < a + len) return TV_ERR_UNSUPPORTED;
  return TV_OK;
}

tv_status check_attn_desc(const tv_attn_desc* d) {
  if (!d) return TV_ERR_NULL;
  if (d->batch < 0 || d->n_nodes < 1 || d->n_nodes > TV_MAX_NODES) return TV_ERR_SHAPE;
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads != 0)
    return TV_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return TV_ERR_UNSUPPORTED;
  if ((int64_t)d->n_nodes * (d->n_q_heads / d->n_kv_heads) > 1024) return TV_ERR_UNSUPPORTED;
  if ((int64_t)d->batch * d->n_nodes * d->n_q_heads > INT_MAX) return TV_ERR_UNSUPPORTED;
  if (d->cache_capacity < 0) return TV_ERR_SHAPE;
  if (d->max_blocks < 0 || d->num_splits < 0 || d->num_splits > 4096) return TV_ERR_SHAPE;
  if (d->tree_placement < TV_TREE_AUTO || d->tree_placement > TV_TREE_IN_LAST_SPLIT ||
      d->kernel < TV_ATTN_KERNEL_AUTO || d->kernel > TV_ATTN_KERNEL_WIDE)
    return TV_ERR_SHAPE;
  if (d->max_blocks > 0) {
    if (d->block_size < 1) return TV_ERR_SHAPE;
    if ((int64_t)d->max_blocks * d->block_size > INT_MAX / 2) return TV_ERR_SHAPE;
  } else {
    if (d->max_prefix_len < 0 || d->max_prefix_len > d->cache_capacity) return TV_ERR_SHAPE;
  }
  const int64_t min_stride = (int64_t)d->n_kv_heads * d->cache_capacity * d->head_dim;
  if (d->cache_seq_stride != 0 && (d->cache_seq_stride < min_stride || d->cache_seq_stride % 8))
    return TV_ERR_SHAPE;
  if (!(d->softmax_scale >= 0.f) || std::isinf(d->softmax_scale)) return TV_ERR_SHAPE;
  return TV_OK;
}

tv_status check_select_desc(const tv_select_desc* d) {
  if (!d) return TV_ERR_NULL;
  if (d->batch < 0 || d->batch > 65535 || d->n_nodes < 1 || d->n_nodes > TV_MAX_NODES)
    return TV_ERR_SHAPE;
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_kv_heads > 65535 ||
      d->n_q_heads % d->n_kv_heads != 0)
    return TV_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return TV_ERR_UNSUPPORTED;
  if (d->cache_capacity < 0 || d->max_prefix_len < 0 || d->max_prefix_len > d->cache_capacity)
    return TV_ERR_SHAPE;
  if (d->block_size < 1 || d->n_sink_blocks < 0 || d->n_window_blocks < 0 || d->top_k < 0)
    return TV_ERR_SHAPE;
  if (d->reduction != TV_REDUCE_MEAN && d->reduction != TV_REDUCE_MAX &&
      d->reduction != TV_REDUCE_LAST)
    return TV_ERR_SHAPE;
  if (d->reduction == TV_REDUCE_MAX && d->n_q_heads / d->n_kv_heads > TV_MAX_SELECT_GROUP)
    return TV_ERR_UNSUPPORTED;
  if (d->max_blocks < 0 ||
      (int64_t)d->max_blocks < (int64_t)d->n_sink_blocks + d->n_window_blocks + d->top_k)
    return TV_ERR_SHAPE;
  if (d->reserved != 0) return TV_ERR_SHAPE;
  return TV_OK;
}

}  // namespace

namespace tv {

tv_status prepare_attention(const tv_attn_desc* desc, const tv_attn_ptrs* ptrs,
                            const void* workspace, AttnPlan* plan, bool* empty) {
  const tv_status st = check_attn_desc(desc);
  if (st != TV_OK) return st;
  if (!ptrs) return TV_ERR_NULL;
  const tv_attn_ptrs& p = *ptrs;
  if (!p.q || !p.k_tree || !p.v_tree || !p.k_cache || !p.v_cache || !p.prefix_len || !p.out ||
      !workspace)
    return TV_ERR_NULL;
  if (!p.mask && !p.parents) return TV_ERR_NULL;
  if (p.mask && p.parents) return TV_ERR_SHAPE;
  if (desc->max_blocks > 0 && (!p.block_idx || !p.n_blocks)) return TV_ERR_NULL;
  if (!aligned(p.q, 16) || !aligned(p.k_tree, 16) || !aligned(p.v_tree, 16) ||
      !aligned(p.k_cache, 16) || !aligned(p.v_cache, 16) || !aligned(p.out, 16))
    return TV_ERR_UNSUPPORTED;
  *empty = desc->batch == 0;
  if (*empty) return TV_OK;
  const int cus = cu_count_for_current_device();
  if (cus <= 0) return TV_ERR_DEVICE;
  *plan = plan_attention(*desc, cus);
  return TV_OK;
}

}  // namespace tv

extern "C" {

tv_status tv_build_tree_mask(const int32_t* parents, int32_t batch, int32_t n_nodes,
                             uint32_t* mask, int32_t* depth, int32_t* dev_err,
                             hipStream_t stream) {
  if (!parents || !mask) return TV_ERR_NULL;
  if (batch < 0 || n_nodes < 1 || n_nodes > TV_MAX_NODES) return TV_ERR_SHAPE;
  if (batch == 0) return TV_OK;
  return launch_status(tv::launch_build_mask(parents, batch, n_nodes, mask, depth, dev_err, stream));
}

int32_t tv_tree_attention_num_splits(const tv_attn_desc* desc) {
  if (check_attn_desc(desc) != TV_OK) return -1;
  const int cus = cu_count_for_current_device();
  if (cus <= 0) return -1;
  return tv::plan_attention(*desc, cus).splits;
}


size_t tv_tree_attention_workspace_size(const tv_attn_desc* desc) {
  if (check_attn_desc(desc) != TV_OK) return 0;
  const int cus = cu_count_for_current_device();
  if (cus <= 0) return 0;
  const tv::AttnPlan p = tv::plan_attention(*desc, cus);
  return p.ws_bytes();
}

tv_status tv_tree_attention(const tv_attn_desc* desc, const tv_attn_ptrs* ptrs, void* workspace,
                            size_t workspace_bytes, int32_t* dev_err, hipStream_t stream) {
  tv::AttnPlan plan{};
  bool empty = false;
  const tv_status st = tv::prepare_attention(desc, ptrs, workspace, &plan, &empty);
  if (st != TV_OK || empty) return st;
  if (!aligned(workspace, 16) || workspace_bytes < plan.ws_bytes())
    return TV_ERR_WORKSPACE;
  return launch_status(tv::launch_attention(*desc, plan, *ptrs, workspace, dev_err, stream));
}

size_t tv_greedy_accept_workspace_size(int32_t batch, int32_t n_nodes, int64_t vocab) {
  if (batch < 0 || n_nodes < 1 || n_nodes > TV_MAX_NODES || vocab < 1 || vocab >= INT_MAX)
    return 0;
  return tv::plan_accept(batch, n_nodes, vocab).ws_bytes;
}

tv_status tv_greedy_accept(const void* logits, tv_dtype dtype, int64_t vocab, int64_t row_stride,
                           const int32_t* parents, const int32_t* draft_tokens, int32_t batch,
                           int32_t n_nodes, int32_t* target_argmax, int32_t* accept_len,
                           int32_t* accept_path, int32_t* bonus_token, void* workspace,
                           size_t workspace_bytes, int32_t* dev_err, hipStream_t stream) {
  if (!logits || !parents || !draft_tokens || !target_argmax || !accept_len || !accept_path ||
      !bonus_token || !workspace)
    return TV_ERR_NULL;
  if (dtype != TV_BF16 && dtype != TV_F32) return TV_ERR_UNSUPPORTED;
  if (batch < 0 || n_nodes < 1 || n_nodes > TV_MAX_NODES) return TV_ERR_SHAPE;
  if (vocab < 1 || vocab >= INT_MAX || row_stride < vocab) return TV_ERR_SHAPE;
  if (batch == 0) return TV_OK;
  const tv::AcceptPlan plan = tv::plan_accept(batch, n_nodes, vocab);
  if (!aligned(workspace, 16) || workspace_bytes < plan.ws_bytes) return TV_ERR_WORKSPACE;
  return launch_status(tv::launch_accept(logits, dtype, vocab, row_stride, parents, draft_tokens,
                                         batch, n_nodes, target_argmax, accept_len, accept_path,
                                         bonus_token, workspace, plan, dev_err, stream));
}

tv_status tv_greedy_accept_commit(const void* logits, tv_dtype dtype, int64_t vocab,
                                  int64_t row_stride, const int32_t* parents,
                                  const int32_t* draft_tokens, int32_t batch, int32_t n_nodes,
                                  int32_t* target_argmax, int32_t* accept_len,
                                  int32_t* accept_path, int32_t* bonus_token, void* workspace,
                                  size_t workspace_bytes, const void* k_tree, const void* v_tree,
                                  const int32_t* prefix_len, int32_t* new_prefix_len,
                                  void* k_cache, void* v_cache, int64_t cache_seq_stride,
                                  int32_t cache_capacity, int32_t n_kv_heads, int32_t head_dim,
                                  int32_t* dev_err, hipStream_t stream) {
  return tv_greedy_accept_commit_layers(
      logits, dtype, vocab, row_stride, parents, draft_tokens, batch, n_nodes, target_argmax,
      accept_len, accept_path, bonus_token, workspace, workspace_bytes, k_tree, v_tree, prefix_len,
      new_prefix_len, k_cache, v_cache, cache_seq_stride, cache_capacity, n_kv_heads, head_dim, 1,
      0, 0, dev_err, stream);
}

tv_status tv_greedy_accept_commit_layers(
    const void* logits, tv_dtype dtype, int64_t vocab, int64_t row_stride, const int32_t* parents,
    const int32_t* draft_tokens, int32_t batch, int32_t n_nodes, int32_t* target_argmax,
    int32_t* accept_len, int32_t* accept_path, int32_t* bonus_token, void* workspace,
    size_t workspace_bytes, const void* k_tree, const void* v_tree, const int32_t* prefix_len,
    int32_t* new_prefix_len, void* k_cache, void* v_cache, int64_t cache_seq_stride,
    int32_t cache_capacity, int32_t n_kv_heads, int32_t head_dim, int32_t n_layers,
    int64_t tree_layer_stride, int64_t cache_layer_stride, int32_t* dev_err, hipStream_t stream) {
  if (!logits || !parents || !draft_tokens || !target_argmax || !accept_len || !accept_path ||
      !bonus_token || !workspace || !k_tree || !v_tree || !prefix_len || !new_prefix_len ||
      !k_cache || !v_cache)
    return TV_ERR_NULL;
  if (dtype != TV_BF16 && dtype != TV_F32) return TV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return TV_ERR_UNSUPPORTED;
  if (batch < 0 || n_nodes < 1 || n_nodes > TV_MAX_NODES || n_kv_heads < 1 || cache_capacity < 0)
    return TV_ERR_SHAPE;
  if (vocab < 1 || vocab >= INT_MAX || row_stride < vocab) return TV_ERR_SHAPE;
  const int64_t min_stride = (int64_t)n_kv_heads * cache_capacity * head_dim;
  if (cache_seq_stride == 0) cache_seq_stride = min_stride;
  if (cache_seq_stride < min_stride || cache_seq_stride % 8) return TV_ERR_SHAPE;
  if (!aligned(k_tree, 16) || !aligned(v_tree, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16))
    return TV_ERR_UNSUPPORTED;
  const tv_status ls = check_layers(n_layers, tree_layer_stride, cache_layer_stride, prefix_len,
                                    new_prefix_len, batch);
  if (ls != TV_OK) return ls;
  if (batch == 0) return TV_OK;
  const tv::AcceptPlan plan = tv::plan_accept(batch, n_nodes, vocab);
  if (!aligned(workspace, 16) || workspace_bytes < plan.ws_bytes) return TV_ERR_WORKSPACE;
  const tv::CommitTarget ct{k_tree,           v_tree,         prefix_len, new_prefix_len,
                            k_cache,          v_cache,        cache_seq_stride,
                            cache_capacity,   n_kv_heads,     head_dim,
                            n_layers,         tree_layer_stride, cache_layer_stride};
  return launch_status(tv::launch_accept(logits, dtype, vocab, row_stride, parents, draft_tokens,
                                         batch, n_nodes, target_argmax, accept_len, accept_path,
                                         bonus_token, workspace, plan, dev_err, stream, &ct));
}

size_t tv_stochastic_accept_workspace_size(int32_t batch, int32_t n_nodes, int64_t vocab) {
  if (batch < 0 || n_nodes < 1 || n_nodes > TV_MAX_NODES || vocab < 1 || vocab >= INT_MAX)
    return 0;
  return tv::plan_stochastic(batch, n_nodes, vocab).ws_bytes;
}

tv_status tv_stochastic_accept(const void* logits, tv_dtype dtype, int64_t vocab,
                               int64_t row_stride, const int32_t* parents,
                               const int32_t* draft_tokens, int32_t batch, int32_t n_nodes,
                               float temperature, uint64_t seed0, uint64_t seed1, uint64_t step,
                               int32_t* accept_len, int32_t* accept_path, int32_t* bonus_token,
                               void* workspace, size_t workspace_bytes, int32_t* dev_err,
                               hipStream_t stream) {
  return tv_stochastic_accept_filtered(logits, dtype, vocab, row_stride, parents, draft_tokens,
                                       batch, n_nodes, temperature, 0, 1.f, seed0, seed1, step,
                                       accept_len, accept_path, bonus_token, workspace,
                                       workspace_bytes, dev_err, stream);
}

tv_status tv_stochastic_accept_filtered(const void* logits, tv_dtype dtype, int64_t vocab,
                                        int64_t row_stride, const int32_t* parents,
                                        const int32_t* draft_tokens, int32_t batch,
                                        int32_t n_nodes, float temperature, int32_t top_k,
                                        float top_p, uint64_t seed0, uint64_t seed1,
                                        uint64_t step, int32_t* accept_len, int32_t* accept_path,
                                        int32_t* bonus_token, void* workspace,
                                        size_t workspace_bytes, int32_t* dev_err,
                                        hipStream_t stream) {
  if (!logits || !parents || !draft_tokens || !accept_len || !accept_path || !bonus_token ||
      !workspace)
    return TV_ERR_NULL;
  if (dtype != TV_BF16 && dtype != TV_F32) return TV_ERR_UNSUPPORTED;
  if (batch < 0 || n_nodes < 1 || n_nodes > TV_MAX_NODES) return TV_ERR_SHAPE;
  if (vocab < 1 || vocab >= INT_MAX || row_stride < vocab) return TV_ERR_SHAPE;
  if (!(temperature > 0.f) || std::isinf(temperature)) return TV_ERR_SHAPE;
  if (top_k < 0 || !(top_p > 0.f && top_p <= 1.f)) return TV_ERR_SHAPE;
  if (batch == 0) return TV_OK;
  const tv::AcceptPlan plan = tv::plan_stochastic(batch, n_nodes, vocab);
  if (!aligned(workspace, 16) || workspace_bytes < plan.ws_bytes) return TV_ERR_WORKSPACE;
  return launch_status(tv::launch_stochastic(logits, dtype, vocab, row_stride, parents,
                                             draft_tokens, batch, n_nodes, temperature, top_k,
                                             top_p, seed0, seed1, step, accept_len, accept_path,
                                             bonus_token, workspace, plan, dev_err, stream));
}

tv_status tv_commit_kv(const void* k_tree, const void* v_tree, const int32_t* accept_path,
                       const int32_t* accept_len, const int32_t* prefix_len,
                       int32_t* new_prefix_len, void* k_cache, void* v_cache,
                       int64_t cache_seq_stride, int32_t cache_capacity, int32_t batch,
                       int32_t n_nodes, int32_t n_kv_heads, int32_t head_dim, int32_t* dev_err,
                       hipStream_t stream) {
  return tv_commit_kv_layers(k_tree, v_tree, accept_path, accept_len, prefix_len, new_prefix_len,
                             k_cache, v_cache, cache_seq_stride, cache_capacity, batch, n_nodes,
                             n_kv_heads, head_dim, 1, 0, 0, dev_err, stream);
}

tv_status tv_commit_kv_layers(const void* k_tree, const void* v_tree, const int32_t* accept_path,
                              const int32_t* accept_len, const int32_t* prefix_len,
                              int32_t* new_prefix_len, void* k_cache, void* v_cache,
                              int64_t cache_seq_stride, int32_t cache_capacity, int32_t batch,
                              int32_t n_nodes, int32_t n_kv_heads, int32_t head_dim,
                              int32_t n_layers, int64_t tree_layer_stride,
                              int64_t cache_layer_stride, int32_t* dev_err, hipStream_t stream) {
  if (!k_tree || !v_tree || !accept_path || !accept_len || !prefix_len || !new_prefix_len ||
      !k_cache || !v_cache)
    return TV_ERR_NULL;
  if (head_dim != 64 && head_dim != 128) return TV_ERR_UNSUPPORTED;
  if (batch < 0 || n_nodes < 1 || n_nodes > TV_MAX_NODES || n_kv_heads < 1 || cache_capacity < 0)
    return TV_ERR_SHAPE;
  const int64_t min_stride = (int64_t)n_kv_heads * cache_capacity * head_dim;
  if (cache_seq_stride == 0) cache_seq_stride = min_stride;
  if (cache_seq_stride < min_stride || cache_seq_stride % 8) return TV_ERR_SHAPE;
  if (!aligned(k_tree, 16) || !aligned(v_tree, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16))
    return TV_ERR_UNSUPPORTED;
  const tv_status ls = check_layers(n_layers, tree_layer_stride, cache_layer_stride, prefix_len,
                                    new_prefix_len, batch);
  if (ls != TV_OK) return ls;
  if (batch == 0) return TV_OK;
  return launch_status(tv::launch_commit(k_tree, v_tree, accept_path, accept_len, prefix_len,
                                         new_prefix_len, k_cache, v_cache, cache_seq_stride,
                                         cache_capacity, batch, n_nodes, n_kv_heads, head_dim,
                                         n_layers, tree_layer_stride, cache_layer_stride,
                                         dev_err, stream));
}

tv_status tv_block_summaries(const void* k_cache, int64_t cache_seq_stride,
                             int32_t cache_capacity, int32_t batch, int32_t n_kv_heads,
                             int32_t head_dim, int32_t block_size, const int32_t* prefix_len,
                             const int32_t* first_token, int32_t max_tokens, void* summaries,
                             int32_t* dev_err, hipStream_t stream) {
  if (!k_cache || !prefix_len || !summaries) return TV_ERR_NULL;
  if (head_dim != 64 && head_dim != 128) return TV_ERR_UNSUPPORTED;
  if (batch < 0 || batch > 65535 || n_kv_heads < 1 || n_kv_heads > 65535 || cache_capacity < 0 ||
      block_size < 1 || max_tokens < 0)
    return TV_ERR_SHAPE;
  const int64_t min_stride = (int64_t)n_kv_heads * cache_capacity * head_dim;
  if (cache_seq_stride == 0) cache_seq_stride = min_stride;
  if (cache_seq_stride < min_stride || cache_seq_stride % 8) return TV_ERR_SHAPE;
  if (!aligned(k_cache, 16) || !aligned(summaries, 16)) return TV_ERR_UNSUPPORTED;
  if (batch == 0 || cache_capacity == 0) return TV_OK;
  return launch_status(tv::launch_summaries(k_cache, cache_seq_stride, cache_capacity, batch,
                                            n_kv_heads, head_dim, block_size, prefix_len,
                                            first_token, max_tokens, summaries, dev_err, stream));
}

size_t tv_select_blocks_workspace_size(const tv_select_desc* desc) {
  if (check_select_desc(desc) != TV_OK) return 0;
  const int cus = cu_count_for_current_device();
  if (cus <= 0) return 0;
  const tv::SelectPlan p = tv::plan_select(*desc, cus);
  return p.kpt ? p.ws_part_bytes : 0;
}

tv_status tv_select_blocks(const tv_select_desc* desc, const void* q, const void* summaries,
                           const int32_t* prefix_len, int32_t* block_idx, int32_t* n_blocks,
                           float* scores, void* workspace, size_t workspace_bytes,
                           int32_t* dev_err, hipStream_t stream) {
  const tv_status st = check_select_desc(desc);
  if (st != TV_OK) return st;
  if (!q || !summaries || !prefix_len || !block_idx || !n_blocks || !workspace)
    return TV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(summaries, 16) || !aligned(scores, 4) || !aligned(block_idx, 4) ||
      !aligned(n_blocks, 4))
    return TV_ERR_UNSUPPORTED;
  if (desc->batch == 0) return TV_OK;
  const int cus = cu_count_for_current_device();
  if (cus <= 0) return TV_ERR_DEVICE;
  const tv::SelectPlan plan = tv::plan_select(*desc, cus);
  if (!plan.kpt) return TV_ERR_UNSUPPORTED;
  if (!aligned(workspace, 256) || workspace_bytes < plan.ws_part_bytes) return TV_ERR_WORKSPACE;
  return launch_status(tv::launch_select(*desc, plan, q, summaries, prefix_len, block_idx,
                                         n_blocks, scores, workspace, dev_err, stream));
}

const char* tv_status_string(tv_status status) {
  switch (status) {
    case TV_OK: return "TV_OK";
    case TV_ERR_NULL: return "TV_ERR_NULL: a required pointer is NULL";
    case TV_ERR_SHAPE: return "TV_ERR_SHAPE: a size is out of range or inconsistent";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED: head_dim, dtype or alignment not supported";
    case TV_ERR_WORKSPACE: return "TV_ERR_WORKSPACE: workspace too small or misaligned";
    case TV_ERR_LAUNCH: return "TV_ERR_LAUNCH: the HIP runtime refused a launch";
    case TV_ERR_DEVICE: return "TV_ERR_DEVICE: no usable HIP device";
  }
  return "unknown tv_status";
}

int32_t tv_version(void) { return 100; }

}  // extern "C"
