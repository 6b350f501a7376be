"""Plain fp64 CPU oracle for SpecPV's retrieval of KV blocks.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP path.

What it computes (source: "SpecPV: Improving Self-Speculative Decoding for
Long-Context Generation via Partial Verification", paperlayer.ai summary of
arXiv 2512.02337v2):

* ``block_summaries`` -- per KV block and KV head, the element-wise maximum
  and minimum key (Sec. 3.2 "Partial Verification": key-state summaries are
  cached to speed up retrieval and are built from element-wise max and min
  key states).
* ``block_scores``    -- each candidate token's query state scores each block;
  the per-query scores of a block are folded into one importance score by a
  reduction: mean, max or last (Sec. 3.2; App. C "Ablation Study": mean works
  best).
* ``select_blocks``   -- the partial KV segment keeps the initial sink blocks,
  the retrieved blocks and a local window at the end of the prefix (Sec. 3.2;
  App. D "Generation Settings": blocks of 16 tokens, 32 sink tokens, a
  128-token window).

Readings where the pages are silent (each is listed in the design notes):

* Only tokens inside the verified prefix [0, P) enter a summary; block j
  covers tokens j*bs .. min((j+1)*bs, P) - 1 and the prefix has
  ceil(P / bs) blocks.  When a block's extreme value is zero its sign is not
  part of the result.
* The score of query q against a block is the largest q.k over all keys k
  that lie between the block's min and max key in every coordinate: each
  coordinate contributes the larger of q_d*max_d and q_d*min_d.  It is an
  upper bound of q.k for every token of the block.  No softmax scale is
  applied (a positive scale does not change the ranking).
* The candidate tokens are the tree nodes.  For each query head the reduction
  runs over the nodes ("last" is node N-1, the last node in the tree's
  order); the per-head results are then averaged over all query heads,
  because one block list serves every head of the sequence.
* Sinks are blocks 0 .. n_sink-1 and the window is the last n_window blocks
  of the prefix; the top_k highest-scoring of the remaining blocks are
  retrieved (equal scores: lower block index first).  The list is the union,
  ascending and without duplicates.

All arithmetic is fp64; bf16 inputs arrive as uint16 bit patterns.
"""

from __future__ import annotations

import numpy as np

from .tree_verify import OracleInputError, bf16_to_f64

__all__ = ["REDUCTIONS", "num_blocks", "block_summaries", "ub_score", "block_scores",
           "select_blocks", "specpv_select"]

REDUCTIONS = ("mean", "max", "last")


def num_blocks(prefix_len: int, block_size: int) -> int:
    """Blocks that hold at least one verified-prefix token."""
    if block_size < 1:
        raise OracleInputError("block size must be positive")
    return -(-int(prefix_len) // block_size)


def block_summaries(k_cache, prefix_len, block_size: int):
    """Element-wise max and min key of every block (SpecPV Sec. 3.2).

    k_cache  uint16 (bf16) [B][Hkv][cap][D]; prefix_len int [B].
    Returns (kmax, kmin, n_valid): kmax and kmin fp64 [B][Hkv][nb_cap][D]
    with nb_cap = ceil(cap / block_size), NaN for blocks past the prefix;
    n_valid int64 [B] = ceil(P_b / block_size).
    """
    kc = np.asarray(k_cache)
    bsz, hkv, cap, d = kc.shape
    nb_cap = num_blocks(cap, block_size)
    kmax = np.full((bsz, hkv, nb_cap, d), np.nan)
    kmin = np.full((bsz, hkv, nb_cap, d), np.nan)
    n_valid = np.zeros(bsz, dtype=np.int64)
    for b in range(bsz):
        p = int(prefix_len[b])
        if not 0 <= p <= cap:
            raise OracleInputError("prefix length outside the cache")
        n_valid[b] = num_blocks(p, block_size)
        for j in range(n_valid[b]):
            rows = bf16_to_f64(kc[b, :, j * block_size:min((j + 1) * block_size, p), :])
            kmax[b, :, j, :] = rows.max(axis=1)
            kmin[b, :, j, :] = rows.min(axis=1)
    return kmax, kmin, n_valid


def ub_score(q, kmax, kmin):
    """Largest q.k over the box kmin <= k <= kmax (last axis is the head dim).

    Each coordinate independently takes the extreme that gives the larger
    product, so the sum is reached by a corner of the box and bounds q.k for
    every key inside it.
    """
    return np.sum(np.maximum(q * kmax, q * kmin), axis=-1)


def _reduce(per_node: np.ndarray, reduction: str) -> np.ndarray:
    """Fold the node axis (axis 0) of per-query scores into one value."""
    if reduction == "mean":
        return per_node.mean(axis=0)
    if reduction == "max":
        return per_node.max(axis=0)
    if reduction == "last":
        return per_node[-1]
    raise OracleInputError(f"unknown reduction {reduction!r}")


def block_scores(q, kmax, kmin, n_valid, reduction: str = "mean", *, blocks=None,
                 magnitude: bool = False):
    """Importance score of each block (SpecPV Sec. 3.2, App. C).

    q uint16 (bf16) [B][N][Hq][D]; kmax, kmin from ``block_summaries``.
    For sequence b and block j: for every query head h (KV head h // G) and
    node i the bound ub(q[b,i,h], block j of that KV head); reduce over the
    nodes; average over the heads.  Returns fp64 [B][nb_cap], NaN past
    n_valid[b].  ``blocks`` restricts the work to the listed block indices of
    every sequence (the others stay NaN).

    With ``magnitude`` the same reduction is applied to sum_d |q_d| *
    max(|max_d|, |min_d|) instead: a bound on the size of the terms, used to
    derive rounding tolerances.
    """
    qf = bf16_to_f64(q)
    bsz, n, hq, d = qf.shape
    hkv = kmax.shape[1]
    if hq % hkv:
        raise OracleInputError("query heads must be a multiple of kv heads")
    grp = hq // hkv
    out = np.full((bsz, kmax.shape[2]), np.nan)
    for b in range(bsz):
        nv = int(n_valid[b])
        js = np.arange(nv) if blocks is None else np.asarray(
            [j for j in blocks if 0 <= j < nv], dtype=np.int64)
        if js.size == 0:
            continue
        acc = np.zeros(js.size)
        for h in range(hq):
            g = h // grp
            hi = kmax[b, g, js, :]                           # [J][D]
            lo = kmin[b, g, js, :]
            qh = qf[b, :, h, :]                              # [N][D]
            if magnitude:
                per_node = np.abs(qh) @ np.maximum(np.abs(hi), np.abs(lo)).T
            else:
                per_node = ub_score(qh[:, None, :], hi[None, :, :], lo[None, :, :])  # [N][J]
            acc += _reduce(per_node, reduction)
        out[b, js] = acc / hq
    return out


def select_blocks(scores_row, n_valid: int, n_sink: int, n_window: int, top_k: int):
    """Blocks of one sequence's partial KV segment (SpecPV Sec. 3.2, App. D).

    Sinks: blocks 0 .. n_sink-1.  Window: the last n_window blocks below
    n_valid.  Retrieved: the top_k blocks of the rest by score, equal scores
    taken in ascending block order.  Returns the union as an ascending int
    array.
    """
    if min(n_sink, n_window, top_k) < 0:
        raise OracleInputError("negative selection size")
    n_valid = int(n_valid)
    sink = set(range(min(n_sink, n_valid)))
    window = set(range(max(n_valid - n_window, 0), n_valid))
    rest = [j for j in range(n_valid) if j not in sink and j not in window]
    vals = [float(scores_row[j]) for j in rest]
    if any(v != v for v in vals):
        raise OracleInputError("NaN block score")
    ranked = sorted(zip(vals, rest), key=lambda t: (-t[0], t[1]))
    picked = {j for _, j in ranked[:top_k]}
    return np.asarray(sorted(sink | window | picked), dtype=np.int64)


def specpv_select(q, k_cache, prefix_len, *, block_size: int, n_sink: int, n_window: int,
                  top_k: int, reduction: str = "mean"):
    """Summaries, scores and the selected block list of every sequence.

    Returns (lists, scores, kmax, kmin, n_valid) with lists a Python list of
    ascending int arrays, one per sequence.
    """
    kmax, kmin, n_valid = block_summaries(k_cache, prefix_len, block_size)
    scores = block_scores(q, kmax, kmin, n_valid, reduction)
    lists = [select_blocks(scores[b], n_valid[b], n_sink, n_window, top_k)
             for b in range(len(n_valid))]
    return lists, scores, kmax, kmin, n_valid
