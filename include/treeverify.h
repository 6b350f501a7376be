/*
 * libtreeverify -- target-side verification of a speculative draft tree on
 * AMD Instinct MI355X (gfx950).
 *
 * The target model checks a whole draft tree in one forward pass ("SpecBlock:
 * Block-Iterative Speculative Decoding with Dynamic Tree Drafting", Abstract
 * and App. A.5).  This library implements the data-parallel part of that
 * pass for one attention layer plus the acceptance step:
 *
 *   tv_build_tree_mask   parent array -> packed ancestor-or-self bitmask
 *   tv_tree_attention    tree-masked GQA attention over the verified-prefix KV
 *                        (full, or a listed subset of KV blocks) and the tree
 *   tv_greedy_accept     per-node vocabulary argmax, longest accepted path,
 *                        accepted length and bonus token
 *   tv_stochastic_accept the same at temperature > 0 (speculative sampling
 *                        along the tree, counter-based random numbers);
 *                        tv_stochastic_accept_filtered adds top-k / top-p
 *   tv_commit_kv         copy the accepted nodes' K/V rows into the cache;
 *                        tv_greedy_accept_commit does acceptance and commit
 *                        in one call, the *_layers forms commit every layer's
 *                        cache in one launch
 *   tv_block_summaries   per-block element-wise max/min keys (SpecPV retrieval)
 *   tv_select_blocks     score blocks against the tree's queries and pick the
 *                        sink + top-k + window list for partial attention
 *   tv_specpv_*          host policy of the partial-verification buffer and
 *                        the tree of a rectifying full verification
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tree: n_nodes nodes per sequence, node 0 is the root (the last committed
 *   token, whose K/V is not yet in the cache), nodes are topologically
 *   ordered: parents[0] == -1 and 0 <= parents[i] < i.  1 <= n_nodes <= 256.
 * - Every pointer argument is a device pointer unless stated otherwise.  The
 *   caller owns every buffer; the library allocates nothing, keeps no state
 *   between calls (apart from cached device properties) and never
 *   synchronises the host.  All work is enqueued on `stream` in order.
 * - Host-checkable problems (null pointers, unsupported sizes, misaligned
 *   buffers, a workspace that is too small) return a non-zero tv_status and
 *   enqueue nothing.
 * - Problems that live in device memory (a malformed parent array, a block id
 *   outside the prefix, a prefix length outside the cache, a commit that would
 *   overflow the cache) cannot be seen by the host: the kernels take the
 *   defined fallback documented with each call and OR the matching TV_DERR_*
 *   bit into *dev_err when dev_err is not NULL.  The caller clears *dev_err.
 * - bf16 tensors hold IEEE bfloat16 values; int32/uint32 are little endian.
 *   Tensor layouts are C-contiguous in the order given.  Every bf16 tensor
 *   and the cache base pointers must be 16-byte aligned.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TV_OK = 0,
  TV_ERR_NULL = 1,         /* a required pointer is NULL */
  TV_ERR_SHAPE = 2,        /* a size is out of range or inconsistent */
  TV_ERR_UNSUPPORTED = 3,  /* head_dim, dtype or alignment not supported */
  TV_ERR_WORKSPACE = 4,    /* workspace too small or misaligned */
  TV_ERR_LAUNCH = 5,       /* the HIP runtime refused a launch */
  TV_ERR_DEVICE = 6        /* no usable HIP device */
} tv_status;

typedef enum { TV_BF16 = 0, TV_F32 = 1 } tv_dtype;

/* device-side data-error bits, OR-ed into *dev_err */
#define TV_DERR_BAD_PARENT 1  /* parents[0] != -1 or parents[i] not in [0, i) */
#define TV_DERR_BAD_BLOCK 2   /* a listed block id < 0, starting at/after prefix_len,
                                 or n_blocks outside [0, max_blocks] */
#define TV_DERR_CAPACITY 4    /* prefix_len + accept_len + 1 > cache_capacity */
#define TV_DERR_BAD_PREFIX 8  /* prefix_len < 0, > cache_capacity or > max_prefix_len */
#define TV_DERR_BAD_PATH 16   /* accept_len or an accept_path entry out of range */
#define TV_DERR_SYNC 32       /* an in-launch merge waited past its bound for the
                                 partials of its split workgroups (outputs undefined) */

#define TV_MAX_NODES 256
#define TV_MAX_LAYERS 4096  /* layers of one multi-layer commit */

/*
 * tv_build_tree_mask -- ancestor-or-self visibility of every tree node.
 *
 * Source: SpecBlock App. A.2 "Attention Mask for SpecBlock": a position sees
 * its on-path ancestors and itself, never positions on other branches (the
 * verified prefix is visible to all and is handled by tv_tree_attention).
 *
 * parents  int32  [batch][n_nodes]
 * mask     uint32 [batch][n_nodes][W], W = ceil(n_nodes / 32): bit (j % 32) of
 *          word (j / 32) of row i is set iff node j is node i or an ancestor
 *          of i.  Bits for j >= n_nodes are zero.
 * depth    int32  [batch][n_nodes] or NULL: number of edges from the root.
 * Fallback: a sequence with any malformed parent entry gets self-only rows
 * and depth 0 everywhere, and TV_DERR_BAD_PARENT is raised.
 */
tv_status tv_build_tree_mask(const int32_t* parents, int32_t batch, int32_t n_nodes,
                             uint32_t* mask, int32_t* depth, int32_t* dev_err,
                             hipStream_t stream);

/*
 * tv_tree_attention -- one layer's attention for all tree nodes.
 *
 * Sources: SpecBlock App. A.2 (visibility: the verified prefix, the node's
 * ancestors and itself); SpecPV Sec. 3.2 "Partial Verification" (a selected
 * subset of KV blocks is attended as one continuous segment).
 *
 * For sequence b, node i and query head h (kv head g = h / (Hq / Hkv)) the
 * visible keys are
 *   full mode (max_blocks == 0): cache rows 0 .. prefix_len[b]-1;
 *   partial mode: for t < n_blocks[b], block blk = block_idx[b][t] covers rows
 *     blk*block_size .. min((blk+1)*block_size, prefix_len[b]) - 1, in list
 *     order (a block listed twice counts twice);
 * followed by the tree nodes j whose bit is set in mask[b][i].
 * out = softmax(scale * q k^T) v over those keys, accumulated in fp32 and
 * rounded to bf16 (nearest even); lse = natural-log sum of exp(scale q.k).
 *
 * Layouts:
 *   q        bf16 [batch][n_nodes][n_q_heads][head_dim]
 *   k_tree   bf16 [batch][n_nodes][n_kv_heads][head_dim]    (v_tree the same)
 *   k_cache  bf16, sequence b at k_cache + b * cache_seq_stride elements, then
 *            [n_kv_heads][cache_capacity][head_dim]          (v_cache the same)
 *   prefix_len int32 [batch]; mask as produced by tv_build_tree_mask (or the
 *            parent array, see tv_attn_ptrs)
 *   block_idx int32 [batch][max_blocks], n_blocks int32 [batch] (partial mode)
 *   out      bf16 [batch][n_nodes][n_q_heads][head_dim]
 *   lse      fp32 [batch][n_nodes][n_q_heads] or NULL
 * Supported: head_dim 64 or 128, n_q_heads % n_kv_heads == 0,
 *   n_nodes * (n_q_heads / n_kv_heads) <= 1024, batch * n_nodes * n_q_heads
 *   below 2^31 (query rows are indexed in 32 bits).
 * Fallbacks: a block that is invalid is skipped (TV_DERR_BAD_BLOCK); a
 *   prefix_len outside [0, min(cache_capacity, max_prefix_len)] is clamped to
 *   that range (TV_DERR_BAD_PREFIX); a row that sees no key at all (possible
 *   only with a hand-made mask) gets out = 0 and lse = -inf.
 * Workspace: at least tv_tree_attention_workspace_size(desc) bytes, 256-byte
 *   aligned.  Its first TV_ATTN_WS_COUNTER_BYTES bytes are counters by which
 *   the merge of the split partials waits for them inside the same launch:
 *   they must be zero before the first call on the workspace (a hipMemset
 *   once, at allocation), and every call leaves them zero, so later calls of
 *   any descriptor may reuse the workspace.  Everything after them is
 *   scratch, undefined on entry and exit.  Calls that share a workspace must
 *   not overlap in time, and the workspace must not serve other calls in
 *   between.  A call that raised TV_DERR_SYNC (a merge that waited past its
 *   bound) may leave the counters non-zero: zero them again.
 */
typedef struct {
  int32_t batch, n_nodes, n_q_heads, n_kv_heads, head_dim;
  int32_t cache_capacity;   /* rows per (sequence, kv head) in the cache */
  int32_t max_prefix_len;   /* host-side upper bound of prefix_len[] (grid sizing) */
  int32_t block_size;       /* partial mode: tokens per KV block (>= 1) */
  int32_t max_blocks;       /* partial mode: columns of block_idx; 0 = full mode */
  float softmax_scale;      /* <= 0 means 1 / sqrt(head_dim) */
  int32_t num_splits;       /* prefix splits per (sequence, kv head); 0 = automatic.  A hint:
                               partial mode raises it so that one split spans at most
                               1022 blocks; tv_tree_attention_num_splits gives the count */
  int64_t cache_seq_stride; /* elements between sequences; 0 = n_kv_heads*capacity*head_dim */
  int32_t tree_placement;   /* where the tree block runs: TV_TREE_AUTO (chosen by the
                               planner), TV_TREE_OWN_WORKGROUP, or TV_TREE_IN_LAST_SPLIT
                               (after the prefix tiles of the last non-empty split).
                               Results are the same; only the schedule differs. */
  int32_t kernel;           /* which schedule runs the call: TV_ATTN_KERNEL_AUTO (chosen by
                               the planner), TV_ATTN_KERNEL_SPLIT16 (eight waves of 16-32
                               rows on 16x16x32 MFMAs) or TV_ATTN_KERNEL_WIDE (four waves of
                               32-64 rows on 32x32x16 MFMAs).  Results agree within the
                               stated tolerance; only the schedule differs. */
} tv_attn_desc;

enum { TV_TREE_AUTO = 0, TV_TREE_OWN_WORKGROUP = 1, TV_TREE_IN_LAST_SPLIT = 2 };
enum { TV_ATTN_KERNEL_AUTO = 0, TV_ATTN_KERNEL_SPLIT16 = 1, TV_ATTN_KERNEL_WIDE = 2 };
/* counters at the start of every attention workspace (zero between calls);
   batch * n_kv_heads above TV_ATTN_WS_COUNTER_BYTES / 8 merges in a second launch */
#define TV_ATTN_WS_COUNTER_BYTES 32768

typedef struct {
  const void* q;
  const void* k_tree;
  const void* v_tree;
  const void* k_cache;
  const void* v_cache;
  const int32_t* prefix_len;
  const uint32_t* mask;     /* as produced by tv_build_tree_mask; or NULL with parents */
  const int32_t* block_idx; /* NULL in full mode */
  const int32_t* n_blocks;  /* NULL in full mode */
  void* out;
  float* lse;               /* may be NULL */
  /* Instead of `mask`: the parent array int32 [batch][n_nodes].  The
     workgroups that attend to the tree then build their mask rows
     themselves, by the rule and fallback of tv_build_tree_mask, and write
     that call's outputs to mask_out / depth_out when these are not NULL
     (both ignored when `mask` is given).  Exactly one of mask / parents. */
  const int32_t* parents;
  uint32_t* mask_out;
  int32_t* depth_out;
} tv_attn_ptrs;

size_t tv_tree_attention_workspace_size(const tv_attn_desc* desc);
/* number of prefix splits the call will use for this descriptor (>= 1) */
int32_t tv_tree_attention_num_splits(const tv_attn_desc* desc);
tv_status tv_tree_attention(const tv_attn_desc* desc, const tv_attn_ptrs* ptrs, void* workspace,
                            size_t workspace_bytes, int32_t* dev_err, hipStream_t stream);

/*
 * tv_tree_attention_noalloc -- tv_tree_attention without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops or harnesses that forbid allocation).
 *
 * The workspace is a library-owned device array of
 * TV_ATTN_NOALLOC_SCRATCH_BYTES on each device, held until the process
 * ends; the call allocates nothing.  Same descriptor, pointers, results and
 * errors as tv_tree_attention, plus TV_ERR_WORKSPACE when the descriptor
 * needs more than TV_ATTN_NOALLOC_SCRATCH_BYTES
 * (tv_tree_attention_workspace_size tells), and TV_ERR_DEVICE when the
 * array's address cannot be found on the current device.  Every call on a
 * device shares that device's array: calls that overlap in time on one
 * device (other streams, other threads) race and must not be issued.  Each
 * call first clears the array's merge counters with a small kernel on
 * `stream`.
 */
#define TV_ATTN_NOALLOC_SCRATCH_BYTES 33554432
tv_status tv_tree_attention_noalloc(const tv_attn_desc* desc, const tv_attn_ptrs* ptrs,
                                    int32_t* dev_err, hipStream_t stream);

/*
 * tv_greedy_accept -- temperature-0 acceptance of a verified tree.
 *
 * Sources: SpecBlock Sec. 4 (greedy decoding at T = 0), App. A.5 (the longest
 * accepted prefix is committed), App. E (the target adds one bonus token);
 * papernotes on SpecBlock, key design 3 (the valid-prefix recurrence, whose
 * tree form is the acceptance rule below).
 *
 * logits        [batch][n_nodes] rows of `vocab` values (bf16 or fp32), row
 *               r = b*n_nodes + i starting at element r*row_stride
 *               (row_stride >= vocab)
 * parents       int32 [batch][n_nodes]
 * draft_tokens  int32 [batch][n_nodes] (entry 0 of each sequence is ignored;
 *               ids outside [0, vocab) never match)
 * target_argmax int32 [batch][n_nodes]: lowest index of the largest logit
 *               (values compare as reals: -0 == +0)
 * accept_len    int32 [batch]: depth of the path's last node (drafts accepted)
 * accept_path   int32 [batch][n_nodes]: node ids root first, -1 padded
 * bonus_token   int32 [batch]: target_argmax of the path's last node
 * Rule: node i >= 1 is accepted iff its parent is accepted and
 *   draft_tokens[i] == target_argmax[parent]; the root is accepted; the path
 *   ends at the deepest accepted node, the lowest index among equal depths.
 * Fallback: a malformed parent array gives accept_len 0, path [0, -1, ...],
 *   bonus = target_argmax of the root, and TV_DERR_BAD_PARENT.
 * NaN logits are outside the contract (result unspecified).
 * Workspace: tv_greedy_accept_workspace_size(...) bytes, 256-byte aligned.
 */
size_t tv_greedy_accept_workspace_size(int32_t batch, int32_t n_nodes, int64_t vocab);
tv_status tv_greedy_accept(const void* logits, tv_dtype dtype, int64_t vocab, int64_t row_stride,
                           const int32_t* parents, const int32_t* draft_tokens, int32_t batch,
                           int32_t n_nodes, int32_t* target_argmax, int32_t* accept_len,
                           int32_t* accept_path, int32_t* bonus_token, void* workspace,
                           size_t workspace_bytes, int32_t* dev_err, hipStream_t stream);

/*
 * tv_greedy_accept_commit -- tv_greedy_accept followed by tv_commit_kv of
 * its path, in one call: the workgroup that walks a sequence's tree also
 * copies the accepted rows into the cache (SpecBlock App. A.5: the longest
 * accepted prefix is committed before the next iteration).
 *
 * Outputs, cache contents, new_prefix_len, device error bits and fallbacks
 * are exactly those of the two calls made in a row with the same arguments
 * (tv_greedy_accept's workspace size applies).  new_prefix_len may alias
 * prefix_len.
 */
tv_status tv_greedy_accept_commit(const void* logits, tv_dtype dtype, int64_t vocab,
                                  int64_t row_stride, const int32_t* parents,
                                  const int32_t* draft_tokens, int32_t batch, int32_t n_nodes,
                                  int32_t* target_argmax, int32_t* accept_len,
                                  int32_t* accept_path, int32_t* bonus_token, void* workspace,
                                  size_t workspace_bytes, const void* k_tree, const void* v_tree,
                                  const int32_t* prefix_len, int32_t* new_prefix_len,
                                  void* k_cache, void* v_cache, int64_t cache_seq_stride,
                                  int32_t cache_capacity, int32_t n_kv_heads, int32_t head_dim,
                                  int32_t* dev_err, hipStream_t stream);

/*
 * tv_greedy_accept_commit_layers -- tv_greedy_accept followed by
 * tv_commit_kv_layers of its path, in one call (the multi-layer form of
 * tv_greedy_accept_commit; same sources as those two calls).  Layer
 * arguments and their errors as tv_commit_kv_layers; outputs, caches,
 * new_prefix_len and device error bits exactly those of the two calls in a
 * row.  One walk-and-copy workgroup per (sequence, layer).
 */
tv_status tv_greedy_accept_commit_layers(
    const void* logits, tv_dtype dtype, int64_t vocab, int64_t row_stride, const int32_t* parents,
    const int32_t* draft_tokens, int32_t batch, int32_t n_nodes, int32_t* target_argmax,
    int32_t* accept_len, int32_t* accept_path, int32_t* bonus_token, void* workspace,
    size_t workspace_bytes, const void* k_tree, const void* v_tree, const int32_t* prefix_len,
    int32_t* new_prefix_len, void* k_cache, void* v_cache, int64_t cache_seq_stride,
    int32_t cache_capacity, int32_t n_kv_heads, int32_t head_dim, int32_t n_layers,
    int64_t tree_layer_stride, int64_t cache_layer_stride, int32_t* dev_err, hipStream_t stream);

/*
 * tv_stochastic_accept -- acceptance at temperature T > 0 (sampling).
 *
 * Sources: SpecPV Sec. 2 "Related Work" (speculative sampling is equivalent
 * to sampling from the target; tree-structured candidates as in SpecInfer);
 * SpecPV App. D / App. E and SpecBlock Sec. 4 (sampling at T = 0.6, 0.7,
 * 1.0).  Random numbers: Philox-4x64-10 (Salmon et al., SC 2011).
 *
 * p_u = softmax(logits_u / T) over the whole vocabulary (fp32).  Drafts are
 * point masses.  Starting at the root, at accepted node u the children are
 * tried in ascending node index: child c (token x) is accepted iff
 *   U(step, b, u, k) * R < p_u(x)      (k = c's rank among u's children)
 * where R is the mass of u's distribution not yet rejected (starts at 1;
 * R -= p_u(x) on rejection); a token outside [0, vocab) or already rejected
 * at u has probability 0.  The first accepted child becomes the next node.
 * When no child is accepted the walk ends at u and the bonus token is the
 * smallest y (vocabulary order) whose cumulative residual probability
 * (p_u without the rejected tokens) exceeds U(step, b, u, 2^64-1) * R.
 * U(c0, c1, c2, c3) = (first word of Philox-4x64-10 with counter
 * (c0, c1, c2, c3) and key (seed0, seed1)) >> 40, times 2^-24.
 * The emitted tokens (accepted drafts, then the bonus) are distributed as
 * sampling from the target one token at a time.
 *
 * Layouts and outputs as tv_greedy_accept (no target_argmax).  temperature
 * must be finite and > 0 (TV_ERR_SHAPE).  Fallbacks: a malformed parent
 * array gives the root-only walk (bonus drawn from p_root) and
 * TV_DERR_BAD_PARENT.  NaN/inf logits are outside the contract.
 * Workspace: tv_stochastic_accept_workspace_size(...) bytes, 16-byte aligned.
 */
size_t tv_stochastic_accept_workspace_size(int32_t batch, int32_t n_nodes, int64_t vocab);
tv_status tv_stochastic_accept(const void* logits, tv_dtype dtype, int64_t vocab,
                               int64_t row_stride, const int32_t* parents,
                               const int32_t* draft_tokens, int32_t batch, int32_t n_nodes,
                               float temperature, uint64_t seed0, uint64_t seed1, uint64_t step,
                               int32_t* accept_len, int32_t* accept_path, int32_t* bonus_token,
                               void* workspace, size_t workspace_bytes, int32_t* dev_err,
                               hipStream_t stream);

/*
 * tv_stochastic_accept_filtered -- tv_stochastic_accept with every node's
 * distribution filtered by top-k and top-p first.
 *
 * Source: SpecPV App. D "Generation Settings" (Qwen3 thinking mode samples at
 * temperature 0.6 with top-p 0.95 and top-k 20) and App. E (temperatures 0.7
 * and 1.0 with top-k off and top-p 0.9).
 *
 * Filters, in this order, on p_u = softmax(l_u / T):
 *   top-k (top_k > 0): token x is kept iff fewer than top_k tokens have a
 *     strictly larger logit (ties with the top_k-th largest are all kept);
 *   top-p (top_p < 1): of the tokens top-k kept, with their probabilities
 *     renormalised, x is kept iff the tokens with a strictly larger logit
 *     hold less than top_p of that mass (the most likely token always stays);
 * and the kept probabilities are renormalised.  Every kept set is "logit >=
 * tau_u" for one threshold per row, which a radix selection finds (the
 * top-p masses are fp32 exponentials summed in 2^-40 fixed point, so a
 * token whose larger tokens hold within about 1e-6 of top_p may fall either
 * way).  The walk, the bonus draw,
 * the uniforms, outputs and fallbacks are then exactly those of
 * tv_stochastic_accept with p_u replaced by the filtered distribution;
 * top_k = 0 and top_p = 1 give tv_stochastic_accept itself.
 * Errors: top_k < 0 or top_p outside (0, 1] (TV_ERR_SHAPE).  Workspace:
 * tv_stochastic_accept_workspace_size(...) bytes, as for tv_stochastic_accept.
 */
tv_status tv_stochastic_accept_filtered(const void* logits, tv_dtype dtype, int64_t vocab,
                                        int64_t row_stride, const int32_t* parents,
                                        const int32_t* draft_tokens, int32_t batch,
                                        int32_t n_nodes, float temperature, int32_t top_k,
                                        float top_p, uint64_t seed0, uint64_t seed1,
                                        uint64_t step, int32_t* accept_len, int32_t* accept_path,
                                        int32_t* bonus_token, void* workspace,
                                        size_t workspace_bytes, int32_t* dev_err,
                                        hipStream_t stream);

/*
 * tv_commit_kv -- append the accepted path's K/V to the cache.
 *
 * Source: SpecBlock App. A.5 (commit the longest accepted prefix before the
 * next iteration) and App. A.2 (the prefix holds previously committed
 * positions).
 *
 * For r = 0 .. accept_len[b] and every kv head h:
 *   k_cache[b][h][prefix_len[b] + r] = k_tree[b][accept_path[b][r]][h]  (same for v)
 * then new_prefix_len[b] = prefix_len[b] + accept_len[b] + 1.  Rows are copied
 * bit for bit; no other cache row is touched.  new_prefix_len may alias
 * prefix_len.  Layouts as for tv_tree_attention.
 * Fallback: if the commit would overflow cache_capacity (TV_DERR_CAPACITY),
 *   prefix_len is out of range (TV_DERR_BAD_PREFIX), or accept_len / a path
 *   entry is out of range (TV_DERR_BAD_PATH), nothing is written for that
 *   sequence and new_prefix_len[b] = prefix_len[b].
 */
tv_status tv_commit_kv(const void* k_tree, const void* v_tree, const int32_t* accept_path,
                       const int32_t* accept_len, const int32_t* prefix_len,
                       int32_t* new_prefix_len, void* k_cache, void* v_cache,
                       int64_t cache_seq_stride, int32_t cache_capacity, int32_t batch,
                       int32_t n_nodes, int32_t n_kv_heads, int32_t head_dim, int32_t* dev_err,
                       hipStream_t stream);

/*
 * tv_commit_kv_layers -- tv_commit_kv for the n_layers attention layers of a
 * model in one launch.
 *
 * Sources: SpecBlock App. A.5 (the accepted prefix is committed before the
 * next iteration: every layer's cache receives the same accepted nodes) and
 * "Dynamic Speculative Decoding", the section on fusing target decode and
 * draft extension into one CUDA graph (per-step launch overhead matters at
 * batch 1).
 *
 * Layer l (0 <= l < n_layers) has its tree K/V at k_tree + l *
 * tree_layer_stride (v_tree likewise) and its cache at k_cache + l *
 * cache_layer_stride (v_cache likewise), strides in bf16 elements, each
 * laid out as for tv_commit_kv; the layers' caches must not overlap.  The
 * result is that of tv_commit_kv called once per layer with the same path,
 * lengths and prefix lengths: every layer receives the same rows at the
 * same positions, and new_prefix_len is written once.  One workgroup per
 * (sequence, layer).
 * Errors: n_layers outside [1, TV_MAX_LAYERS] (TV_ERR_SHAPE); with
 *   n_layers > 1, a stride that is not a positive multiple of 8 elements
 *   (TV_ERR_SHAPE) or new_prefix_len overlapping prefix_len
 *   (TV_ERR_UNSUPPORTED: layer 0 may write the new lengths before another
 *   layer has read the old ones).  Device fallbacks as tv_commit_kv, for
 *   all layers alike.
 */
tv_status tv_commit_kv_layers(const void* k_tree, const void* v_tree, const int32_t* accept_path,
                              const int32_t* accept_len, const int32_t* prefix_len,
                              int32_t* new_prefix_len, void* k_cache, void* v_cache,
                              int64_t cache_seq_stride, int32_t cache_capacity, int32_t batch,
                              int32_t n_nodes, int32_t n_kv_heads, int32_t head_dim,
                              int32_t n_layers, int64_t tree_layer_stride,
                              int64_t cache_layer_stride, int32_t* dev_err, hipStream_t stream);

/*
 * tv_block_summaries -- element-wise max and min key of every KV block.
 *
 * Source: SpecPV Sec. 3.2 "Partial Verification": the key states of each
 * block are summarised by their element-wise maximum and minimum, and the
 * summaries are cached so that retrieval does not re-read the keys.
 *
 * Block j of sequence b covers cache rows j*block_size ..
 * min((j+1)*block_size, prefix_len[b]) - 1.  For every kv head h and every
 * block j with first_token[b] <= (j+1)*block_size - 1 and j*block_size <
 * prefix_len[b] (that is, every block that holds a row in
 * [first_token[b], prefix_len[b])):
 *   summaries[b][h][j][0][d] = max over the block's rows of k_cache[..][d]
 *   summaries[b][h][j][1][d] = min over the block's rows of k_cache[..][d]
 * as bf16 values (a maximum or minimum of zero may carry either sign).  No
 * other record is touched, so after tv_commit_kv a call with first_token =
 * the old prefix length and prefix_len = the new one updates the cache.
 *
 * k_cache     bf16, sequence b at k_cache + b * cache_seq_stride elements
 *             (0 = n_kv_heads*capacity*head_dim), then [n_kv_heads][capacity][head_dim]
 * prefix_len  int32 [batch]; first_token int32 [batch] or NULL (= 0)
 * summaries   bf16 [batch][n_kv_heads][ceil(capacity / block_size)][2][head_dim]
 * max_tokens  host-side estimate of max_b (prefix_len[b] - first_token[b]);
 *             it only sizes the grid (every block is processed whatever it is).
 * Supported: head_dim 64 or 128, block_size >= 1.
 * Fallback: a sequence with prefix_len outside [0, capacity] or first_token
 *   outside [0, prefix_len] is skipped (TV_DERR_BAD_PREFIX).
 */
tv_status tv_block_summaries(const void* k_cache, int64_t cache_seq_stride,
                             int32_t cache_capacity, int32_t batch, int32_t n_kv_heads,
                             int32_t head_dim, int32_t block_size, const int32_t* prefix_len,
                             const int32_t* first_token, int32_t max_tokens, void* summaries,
                             int32_t* dev_err, hipStream_t stream);

/*
 * tv_select_blocks -- the KV blocks a partial verification attends to.
 *
 * Sources: SpecPV Sec. 3.2 (blocks are scored against the query states of
 * all candidate tokens, the per-query scores folded by a reduction such as
 * max, mean or last; the partial cache keeps sink blocks, retrieved blocks
 * and a local window), App. C (mean works best), App. D (16-token blocks,
 * 32 sink tokens, a 128-token window).
 *
 * For sequence b let nv = ceil(P / block_size), P = prefix_len[b].  For block
 * j < nv, query head h (kv head g = h / (Hq/Hkv)) and node i:
 *   ub(i, h, j) = sum_d max(q[b][i][h][d] * hi[d], q[b][i][h][d] * lo[d])
 * with hi, lo = summaries[b][g][j][0], [1] (the largest q.k over the box
 * between them, so an upper bound of q.k for each key of the block).  Then
 *   TV_REDUCE_MEAN: score[j] = mean over h of (mean over i of ub)
 *   TV_REDUCE_MAX:  score[j] = mean over h of (max over i of ub)
 *   TV_REDUCE_LAST: score[j] = mean over h of ub(n_nodes - 1, h, j)
 * accumulated in fp32.  The selected list is the union, ascending and
 * without duplicates, of
 *   sinks   0 .. n_sink_blocks - 1,
 *   window  the last n_window_blocks blocks below nv,
 *   the top_k blocks of the rest by score (equal scores: lower id first),
 * each clipped to [0, nv).  It is written to block_idx[b][0 .. n_blocks[b]-1]
 * and the rest of the row is set to -1: the format tv_tree_attention's
 * partial mode reads (same block_size).
 *
 * Layouts: q bf16 [batch][n_nodes][n_q_heads][head_dim]; summaries as
 *   written by tv_block_summaries for this cache_capacity and block_size;
 *   prefix_len int32 [batch]; block_idx int32 [batch][max_blocks];
 *   n_blocks int32 [batch]; scores fp32 [batch][ceil(capacity / block_size)]
 *   or NULL (entries j >= nv are not written).
 * Supported: head_dim 64 or 128; TV_REDUCE_MAX needs n_q_heads / n_kv_heads
 *   <= TV_MAX_SELECT_GROUP; max_blocks >= n_sink_blocks + n_window_blocks + top_k;
 *   at most TV_MAX_SELECT_BLOCKS blocks in min(capacity, max_prefix_len)
 *   (TV_ERR_UNSUPPORTED, and a workspace size of 0, beyond).
 * Fallback: prefix_len outside [0, min(capacity, max_prefix_len)] is clamped
 *   to that range (TV_DERR_BAD_PREFIX).  NaN or infinite inputs give an
 *   unspecified (but valid, ascending) list.
 * Workspace: tv_select_blocks_workspace_size(desc) bytes, 256-byte aligned.
 */
enum { TV_REDUCE_MEAN = 0, TV_REDUCE_MAX = 1, TV_REDUCE_LAST = 2 };
#define TV_MAX_SELECT_GROUP 64
#define TV_MAX_SELECT_BLOCKS 32768

typedef struct {
  int32_t batch, n_nodes, n_q_heads, n_kv_heads, head_dim;
  int32_t cache_capacity;   /* rows per (sequence, kv head) of the summarised cache */
  int32_t max_prefix_len;   /* host-side upper bound of prefix_len[] (grid sizing) */
  int32_t block_size;       /* tokens per block (>= 1) */
  int32_t n_sink_blocks, n_window_blocks, top_k;  /* each >= 0 */
  int32_t reduction;        /* TV_REDUCE_MEAN, TV_REDUCE_MAX or TV_REDUCE_LAST */
  int32_t max_blocks;       /* columns of block_idx */
  int32_t reserved;         /* must be 0 */
} tv_select_desc;

size_t tv_select_blocks_workspace_size(const tv_select_desc* desc);
tv_status tv_select_blocks(const tv_select_desc* desc, const void* q, const void* summaries,
                           const int32_t* prefix_len, int32_t* block_idx, int32_t* n_blocks,
                           float* scores, void* workspace, size_t workspace_bytes,
                           int32_t* dev_err, hipStream_t stream);

/*
 * SpecPV partial-verification buffer and rectification (host functions).
 *
 * Source: SpecPV Sec. 3.3 "Rectified with Full Verification": tokens
 * accepted by partial verification are partially verified; when the partial
 * cache's buffer overflows, a full verification re-checks them, prepended to
 * the new candidates, over the full KV, and the partial cache is rebuilt.
 * App. C sizes the buffer as one step's tokens plus 20; App. D: buffer 20.
 *
 * The buffer holds the step's candidates plus up to buffer_size partially
 * verified tokens (the cache rows committed by partial steps since the last
 * full verification).  These functions take HOST pointers, touch no device
 * and enqueue nothing.
 *
 * tv_specpv_needs_rectification: 1 if the next step must be a rectifying full
 *   verification (n_partial > buffer_size), 0 if it may be partial, -1 if a
 *   count is negative.
 *
 * tv_specpv_rectify_tree: the tree a rectifying step verifies.  Node i <
 *   n_buffer is buffered token i (oldest first; node 0, the last full
 *   verification's bonus token, is the root), chained to node i-1; node
 *   n_buffer is the current root (root_token, the last emitted token) under
 *   node n_buffer-1; draft node j >= 1 becomes node n_buffer + j under node
 *   n_buffer + parents[j].  parents_out and tokens_out have n_buffer + n_draft
 *   entries.  The step then runs with full attention over the fully verified
 *   prefix and commits at the fully verified length, replacing the partially
 *   verified rows.
 *   Errors: TV_ERR_NULL; TV_ERR_SHAPE if n_buffer < 1, n_draft < 1,
 *   n_buffer + n_draft > TV_MAX_NODES, or the draft tree is not topologically
 *   ordered with parents[0] == -1.
 */
int32_t tv_specpv_needs_rectification(int32_t n_partial, int32_t buffer_size);
tv_status tv_specpv_rectify_tree(const int32_t* buffer_tokens, int32_t n_buffer,
                                 int32_t root_token, const int32_t* parents,
                                 const int32_t* draft_tokens, int32_t n_draft,
                                 int32_t* parents_out, int32_t* tokens_out);

/* human-readable name of a status code (static storage) */
/*
 * tv_stream_read -- measurement aid, not a step of the method: reads
 * `bytes` (a multiple of 16) at `src` once with 16-byte loads spread over
 * the whole chip and writes one folding word per workgroup to
 * sink[0 .. TV_STREAM_READ_SINK_WORDS-1], so that timing it gives the read
 * bandwidth this device reaches, the ceiling against which the other calls'
 * bytes per second are judged.  src 16-byte aligned; sink device memory of
 * TV_STREAM_READ_SINK_WORDS words.
 */
#define TV_STREAM_READ_SINK_WORDS 2048
tv_status tv_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

const char* tv_status_string(tv_status status);
/* library version: major * 10000 + minor * 100 + patch */
int32_t tv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TREEVERIFY_H */
