"""Plain fp64 CPU oracle for target-side tree verification.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP path.

What it computes (one function per step of the verification hot path):

* ``build_mask``   -- ancestor-or-self visibility of each draft-tree node.
* ``tree_attention`` -- exact softmax attention of every tree node's query
  heads over the verified-prefix KV (full, or a listed subset of KV blocks)
  followed by the tree nodes that the node may see.
* ``greedy_accept`` -- temperature-0 acceptance: per-node vocabulary argmax,
  longest accepted root-to-node path, bonus token.
* ``commit_kv``    -- copy the accepted nodes' K/V rows into the cache.

Sources (page title, then the section the step follows):

* "SpecBlock: Block-Iterative Speculative Decoding with Dynamic Tree
  Drafting" (paperlayer.ai summary of arXiv 2605.07243v2): Abstract (whole
  tree verified in one target forward); App. A.2 "Attention Mask for
  SpecBlock" (a position sees the verified prefix, its on-path ancestors and
  itself, never off-path positions); App. A.5 "Inference procedure" (the
  longest accepted prefix is committed before the next iteration); App. E
  "Case Study" (the target contributes one bonus token after the accepted
  drafts); Sec. 4 "Experiments" (greedy decoding at temperature 0).
* papernotes.org notes on the same paper, "关键设计" item 3 (the valid-prefix
  recurrence m_{t,k+1} = m_{t,k} * 1[argmax p_{t,k} = y*_{t,k}]) and the main
  results table setting (greedy, T = 0).
* "Dynamic Speculative Decoding" (blog), "Implementation Details": per request
  the number of emitted tokens is accept_length + 1, and the last emitted
  token of request r sits at the running sum of those counts minus one.
* "SpecPV: Improving Self-Speculative Decoding for Long-Context Generation via
  Partial Verification" (paperlayer.ai summary of arXiv 2512.02337v2), Sec. 3.2
  "Partial Verification": the selected KV subset is attended as one
  continuous segment together with the candidate tokens.

Readings taken where the pages are silent (each is listed in the design notes):

* Node 0 is the root: the last committed token, whose K/V is not in the cache
  yet.  Nodes are topologically ordered (parent index < child index).
* Prefix tokens are visible to every tree node (no causal limit inside the
  verified prefix for the tree queries).
* GQA: query head h reads KV head floor(h / G), G = Hq / Hkv.
* Softmax scale defaults to 1 / sqrt(head_dim).
* A listed KV block b covers cache rows b*bs .. min((b+1)*bs, P) - 1; the
  listed blocks are concatenated in list order (a duplicate counts twice).
* accept_len counts accepted draft nodes excluding the root; the rows
  committed are the root plus the accepted drafts (accept_len + 1 rows).  The
  bonus token's K/V does not exist yet and is not committed.
* When duplicate sibling tokens accept several branches, the deepest accepted
  node wins and, among equal depths, the lowest node index.
* Argmax ties go to the lowest vocabulary index; -0 and +0 compare equal.

All floating-point arithmetic is fp64.  bf16 inputs arrive as uint16 bit
patterns and are widened exactly (bits << 16 is an fp32 bit pattern).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f64",
    "OracleInputError",
    "build_mask",
    "ancestors",
    "tree_attention",
    "argmax_lowest",
    "greedy_accept",
    "pack_accepted_tokens",
    "commit_kv",
]


class OracleInputError(ValueError):
    """Raised for inputs the method does not define (malformed trees, NaN
    logits, block ids outside the prefix, cache overflow)."""


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp64."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 data must be passed as uint16 bit patterns")
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def _check_parents(parents_row: np.ndarray) -> None:
    n = parents_row.shape[0]
    if n < 1:
        raise OracleInputError("a draft tree needs at least the root node")
    if int(parents_row[0]) != -1:
        raise OracleInputError("node 0 must be the root (parent -1)")
    for i in range(1, n):
        p = int(parents_row[i])
        if not (0 <= p < i):
            raise OracleInputError(
                f"node {i} has parent {p}; parents must precede children")


def ancestors(parents_row: np.ndarray, i: int) -> list[int]:
    """Ancestor-or-self set of node i, listed from i up to the root."""
    out = [i]
    j = i
    while int(parents_row[j]) >= 0:
        j = int(parents_row[j])
        out.append(j)
    return out


# ---------------------------------------------------------------------------
# O1: tree mask
# ---------------------------------------------------------------------------

def build_mask(parents: np.ndarray):
    """Packed ancestor-or-self bitmask and depth of every draft-tree node.

    Follows SpecBlock App. A.2: a node sees the nodes on its own root path
    (its ancestors) and itself; nodes off that path are hidden.  The prefix
    part of the visibility is handled by ``tree_attention``.

    parents: int [B][N], parents[b][0] == -1 and 0 <= parents[b][i] < i.
    Returns mask uint32 [B][N][W] with W = ceil(N / 32) (bit j of row i lives
    in word j // 32 at bit position j % 32) and depth int32 [B][N].
    """
    parents = np.asarray(parents)
    if parents.ndim != 2:
        raise OracleInputError("parents must be [batch][n_nodes]")
    bsz, n = parents.shape
    w = (n + 31) // 32
    mask = np.zeros((bsz, n, w), dtype=np.uint32)
    depth = np.zeros((bsz, n), dtype=np.int32)
    for b in range(bsz):
        _check_parents(parents[b])
        for i in range(n):
            anc = ancestors(parents[b], i)
            depth[b, i] = len(anc) - 1
            for j in anc:
                mask[b, i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return mask, depth


def _mask_bit(mask_row: np.ndarray, j: int) -> bool:
    return bool((int(mask_row[j // 32]) >> (j % 32)) & 1)


# ---------------------------------------------------------------------------
# O2: tree attention
# ---------------------------------------------------------------------------

def _visible_prefix_rows(p_len: int, block_idx_row, n_blk, block_size):
    """Cache rows of the prefix segment one sequence attends to.

    Full mode (no block list): rows 0 .. P-1.
    Partial mode (SpecPV Sec. 3.2): the listed blocks in list order, each
    clipped to the verified prefix, concatenated into one segment.
    """
    if block_idx_row is None:
        return np.arange(p_len, dtype=np.int64)
    rows = []
    for t in range(n_blk):
        blk = int(block_idx_row[t])
        start = blk * block_size
        if blk < 0 or start >= p_len:
            raise OracleInputError(
                f"block {blk} does not start inside the verified prefix ({p_len})")
        stop = min(start + block_size, p_len)
        rows.extend(range(start, stop))
    return np.asarray(rows, dtype=np.int64)


def tree_attention(q, k_cache, v_cache, k_tree, v_tree, prefix_len, mask, *,
                   block_idx=None, n_blocks=None, block_size=None, scale=None):
    """Exact tree-masked GQA attention in fp64.

    Layouts (all bf16 arrays as uint16 bit patterns):
      q        [B][N][Hq][D]
      k_cache  [B][Hkv][cap][D]   (v_cache the same)
      k_tree   [B][N][Hkv][D]     (v_tree the same)
      prefix_len int [B]; mask uint32 [B][N][W] from ``build_mask``.
      Partial mode: block_idx int [B][max_blocks], n_blocks int [B],
      block_size int.

    For batch b, node i, query head h (kv head g = h // G) the visible keys
    are the prefix segment followed by the tree nodes j whose bit is set in
    mask[b][i] (SpecBlock App. A.2; SpecPV Sec. 3.2).  With s_t the scaled dot
    products: o = sum_t e^{s_t - m} v_t / sum_t e^{s_t - m}, m = max_t s_t, and
    lse = m + ln sum_t e^{s_t - m}.

    Returns (o fp64 [B][N][Hq][D], lse fp64 [B][N][Hq]).
    """
    qf = bf16_to_f64(q)
    kc = np.asarray(k_cache)
    vc = np.asarray(v_cache)
    ktf = bf16_to_f64(k_tree)
    vtf = bf16_to_f64(v_tree)
    bsz, n, hq, d = qf.shape
    hkv = kc.shape[1]
    cap = kc.shape[2]
    if hq % hkv != 0:
        raise OracleInputError("query heads must be a multiple of kv heads")
    grp = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    partial = block_idx is not None
    o = np.zeros((bsz, n, hq, d), dtype=np.float64)
    lse = np.zeros((bsz, n, hq), dtype=np.float64)
    for b in range(bsz):
        p_len = int(prefix_len[b])
        if not (0 <= p_len <= cap):
            raise OracleInputError("prefix length outside the cache")
        rows = _visible_prefix_rows(
            p_len,
            block_idx[b] if partial else None,
            int(n_blocks[b]) if partial else 0,
            block_size)
        # tree visibility, one boolean row per node
        vis = np.array([[_mask_bit(mask[b, i], j) for j in range(n)]
                        for i in range(n)], dtype=bool)
        for g in range(hkv):
            kp = bf16_to_f64(kc[b, g, rows, :]) if rows.size else np.zeros((0, d))
            vp = bf16_to_f64(vc[b, g, rows, :]) if rows.size else np.zeros((0, d))
            kt = ktf[b, :, g, :]           # [N][D]
            vt = vtf[b, :, g, :]
            k_all = np.concatenate([kp, kt], axis=0)   # [R + N][D]
            v_all = np.concatenate([vp, vt], axis=0)
            for hh in range(grp):
                h = g * grp + hh
                qh = qf[b, :, h, :]                    # [N][D]
                s = (qh @ k_all.T) * scale             # [N][R + N]
                s[:, rows.size:][~vis] = -np.inf
                m = np.max(s, axis=1, keepdims=True)
                if not np.all(np.isfinite(m)):
                    raise OracleInputError("a node sees no key at all")
                w = np.exp(s - m)
                den = np.sum(w, axis=1, keepdims=True)
                o[b, :, h, :] = (w @ v_all) / den
                lse[b, :, h] = m[:, 0] + np.log(den[:, 0])
    return o, lse


# ---------------------------------------------------------------------------
# O3: greedy acceptance
# ---------------------------------------------------------------------------

def argmax_lowest(row: np.ndarray) -> int:
    """Index of the largest value, lowest index among equal values.

    Values compare as real numbers (so -0 equals +0).  NaN is undefined for
    the method and raises.
    """
    r = np.asarray(row)
    if r.dtype == np.uint16:
        r = bf16_to_f64(r)
    else:
        r = r.astype(np.float64)
    if np.isnan(r).any():
        raise OracleInputError("NaN logit")
    return int(np.argmax(r))   # numpy returns the first occurrence


def greedy_accept(logits: np.ndarray, parents: np.ndarray, draft_tokens: np.ndarray):
    """Temperature-0 verification of a draft tree.

    1. a[i] = argmax of node i's target logits (lowest index on ties): the
       target's greedy next token after the path ending at node i.
    2. The root is accepted; node i >= 1 is accepted iff its parent is
       accepted and its draft token equals a[parent] -- the tree form of the
       valid-prefix recurrence (papernotes, key design 3).
    3. The committed path ends at the deepest accepted node (lowest index
       among equal depths): the longest accepted prefix (SpecBlock A.5).
    4. accept_len = that node's depth; the bonus token is a[end node]
       (SpecBlock App. E).

    logits: [B][N][V] (uint16 bf16 bits or float); parents, draft_tokens:
    int [B][N] (draft_tokens[b][0] is ignored).
    Returns (argmax int32 [B][N], accept_len int32 [B],
             path int32 [B][N] root first, -1 padded, bonus int32 [B]).
    """
    logits = np.asarray(logits)
    parents = np.asarray(parents)
    draft_tokens = np.asarray(draft_tokens)
    bsz, n = parents.shape
    amax = np.zeros((bsz, n), dtype=np.int32)
    acc_len = np.zeros(bsz, dtype=np.int32)
    path = np.full((bsz, n), -1, dtype=np.int32)
    bonus = np.zeros(bsz, dtype=np.int32)
    for b in range(bsz):
        _check_parents(parents[b])
        for i in range(n):
            amax[b, i] = argmax_lowest(logits[b, i])
        acc = [False] * n
        depth = [0] * n
        acc[0] = True
        for i in range(1, n):
            p = int(parents[b, i])
            depth[i] = depth[p] + 1
            acc[i] = acc[p] and int(draft_tokens[b, i]) == int(amax[b, p])
        best = 0
        for i in range(n):
            if acc[i] and depth[i] > depth[best]:
                best = i          # strict '>' keeps the lowest index on ties
        chain = ancestors(parents[b], best)[::-1]   # root first
        acc_len[b] = depth[best]
        path[b, :len(chain)] = chain
        bonus[b] = amax[b, best]
    return amax, acc_len, path, bonus


def pack_accepted_tokens(draft_tokens, accept_len, path, bonus):
    """Per-request emitted tokens, packed back to back.

    Request r emits its accepted draft tokens (path[1..accept_len], the root
    is already committed) followed by the bonus token: accept_len + 1 tokens.
    The last emitted token of request r sits at index cumsum(accept_len+1)[r]-1
    ("Dynamic Speculative Decoding", Implementation Details).
    Returns (tokens int32 [sum(accept_len+1)], last_index int64 [B]).
    """
    toks = []
    for b in range(len(accept_len)):
        for r in range(1, int(accept_len[b]) + 1):
            toks.append(int(draft_tokens[b][int(path[b][r])]))
        toks.append(int(bonus[b]))
    counts = np.asarray(accept_len, dtype=np.int64) + 1
    last = np.cumsum(counts) - 1
    return np.asarray(toks, dtype=np.int32), last


# ---------------------------------------------------------------------------
# O4: KV commit
# ---------------------------------------------------------------------------

def commit_kv(k_tree, v_tree, path, accept_len, prefix_len, k_cache, v_cache):
    """Append the accepted path's K/V rows to the cache (SpecBlock A.5).

    For r = 0 .. accept_len and every kv head h:
      cache[b][h][P_b + r] = tree[b][path[b][r]][h]
    and the new prefix length is P_b + accept_len + 1.  Bit patterns are
    copied unchanged.  Returns new (k_cache, v_cache, new_prefix_len); the
    inputs are not modified.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    bsz, hkv, cap, _ = kc.shape
    new_len = np.zeros(bsz, dtype=np.int32)
    for b in range(bsz):
        p_len = int(prefix_len[b])
        a = int(accept_len[b])
        if p_len < 0 or p_len + a + 1 > cap:
            raise OracleInputError("commit would overflow the cache")
        for r in range(a + 1):
            node = int(path[b][r])
            for h in range(hkv):
                kc[b, h, p_len + r, :] = k_tree[b, node, h, :]
                vc[b, h, p_len + r, :] = v_tree[b, node, h, :]
        new_len[b] = p_len + a + 1
    return kc, vc, new_len
