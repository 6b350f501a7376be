"""Seeded synthetic inputs for tree verification.

This module only draws random data in the shapes and distributions of the
workloads the pages describe; it performs none of the verification
arithmetic (no masks, no attention, no argmax, no path walk, no commit).
Both the HIP path and the CPU oracle consume exactly the bit patterns it
returns.

Workloads (one seeded generator each):

* ``tiny``           batch 1, Hq 4, Hkv 1, D 64, prefix 256, 8-node tree of
                     depth 3 (1-3 children per internal node), fp32 logits
                     over a 1024-token vocabulary, draft = target token with
                     probability 0.7.
* ``8b_layer``       batch 1, Hq 32, Hkv 8, D 128, prefix 1000, EAGLE-style
                     60-node tree of depth 8 (top-4 expansion pruned by seeded
                     path scores), bf16 logits over 128256, probability 0.75.
* ``specblock_tree`` same head shape, prefix 4096, tree grown by 3 block
                     expansions of K = 4 dependent positions with per-position
                     sibling counts [2, 4, 10, 0] drawn with probabilities
                     0.55/0.25/0.15/0.05, capped at 96 nodes; rank-1 nodes
                     carry the target token with probability 0.8.
* ``batched``        16 sequences, ragged prefixes uniform in [1000, 1600],
                     independent 32-node trees of depth 6, probability 0.7.
* ``long_context``   batch 1, prefix 60000, 60-node depth-8 tree; a partial
                     KV list of 64-token blocks (2 sink blocks, the last 16
                     blocks and 46 distinct random others).

SpecPV retrieval settings (App. D "Generation Settings": 16-token blocks,
32 sink tokens, a 128-token local window; Sec. 4.3: a 4096-token partial KV
budget) are the ``SPECPV_*`` constants.  ``make_select_case`` draws small
seeded cases for block selection, optionally with planted relevant blocks:
every query of a sequence leans toward one random direction, and one token of
each planted block carries a large multiple of that direction.

Sources for the shapes: "Dynamic Speculative Decoding" (Problem Context:
~1000-token prompts; Benchmark Table: (steps, topk, draft tokens) triples);
SpecBlock (Sec. 4 setup: 8B-class GQA targets at batch 1; papernotes key
design 2: rank buckets and sibling counts [2, 4, 10, 0]); SpecPV (Sec. 4.1:
32K-60K contexts; App. D: KV blocks, sink tokens and a local window).

Target tokens are planted, not computed: each logits row draws N(0, s^2)
values, clipped just below a cap, and the cap value is written at one chosen
index (and, for a tenth of the rows, at a second, higher index, so ties occur).
The drafter then proposes the planted token of the parent node with the
workload's probability, otherwise a uniform random id.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# cap for bf16 logits with std sqrt(2): 8.0 and the bf16 value just below it
_BF16_CAP = 8.0
_BF16_BELOW_CAP = 7.96875
_TIE_FRACTION = 0.1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even) as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (for generator checks)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    n_nodes: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    logits_dtype: str                 # "bf16" or "f32"
    parents: np.ndarray               # int32 [B][N]
    draft_tokens: np.ndarray          # int32 [B][N]
    logits: np.ndarray                # uint16 or float32 [B][N][V]
    q: np.ndarray                     # uint16 [B][N][Hq][D]
    k_tree: np.ndarray                # uint16 [B][N][Hkv][D]
    v_tree: np.ndarray
    k_cache: np.ndarray               # uint16 [B][Hkv][cap][D], NaN past P_b
    v_cache: np.ndarray
    prefix_len: np.ndarray            # int32 [B]
    capacity: int
    planted_target: np.ndarray        # int32 [B][N] (generator bookkeeping)
    block_size: int = 0
    block_idx: np.ndarray | None = None   # int32 [B][max_blocks]
    n_blocks: np.ndarray | None = None    # int32 [B]

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_len.max()) if self.batch else 0

    @property
    def max_blocks(self) -> int:
        return 0 if self.block_idx is None else int(self.block_idx.shape[1])

    def without_blocks(self) -> "Workload":
        return dataclasses.replace(self, block_size=0, block_idx=None, n_blocks=None)


# ---------------------------------------------------------------------------
# tree shapes
# ---------------------------------------------------------------------------

def _bfs_relabel(parents: list[int]) -> np.ndarray:
    """Relabel a topologically ordered tree in breadth-first order (children
    visited in creation order)."""
    n = len(parents)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parents[i]].append(i)
    order = [0]
    head = 0
    while head < len(order):
        order.extend(children[order[head]])
        head += 1
    new_of = {old: new for new, old in enumerate(order)}
    out = np.full(n, -1, dtype=np.int32)
    for old in range(1, n):
        out[new_of[old]] = new_of[parents[old]]
    return out


def tiny_tree(rng: np.random.Generator) -> np.ndarray:
    """Root plus a depth-3 spine, then 4 nodes hung under uniformly chosen
    nodes of depth < 3 that have fewer than 3 children; 8 nodes, BFS order."""
    parents = [-1, 0, 1, 2]
    depth = [0, 1, 2, 3]
    nchild = [1, 1, 1, 0]
    for _ in range(4):
        cands = [i for i in range(len(parents)) if depth[i] < 3 and nchild[i] < 3]
        p = int(cands[rng.integers(len(cands))])
        parents.append(p)
        depth.append(depth[p] + 1)
        nchild.append(0)
        nchild[p] += 1
    return _bfs_relabel(parents)


def eagle_tree(rng: np.random.Generator, steps: int, topk: int, n_nodes: int,
               want_depth: int) -> np.ndarray:
    """EAGLE-style dynamic tree: every frontier node gets ``topk`` children
    whose probabilities are a sorted softmax of ``topk`` N(0, 1.5^2) draws;
    a child's score is its parent's score plus ln p.  The next frontier is
    the ``topk`` best children of the step.  After ``steps`` steps the
    ``n_nodes - 1`` best candidates (ties broken by creation order) are kept
    with the root; scores fall along every path, so the kept set is closed
    under taking parents.  Redrawn until the kept tree reaches ``want_depth``.
    """
    for _attempt in range(1000):
        parents = [-1]
        score = [0.0]
        depth = [0]
        frontier = [0]
        for _s in range(steps):
            new = []
            for f in frontier:
                z = rng.normal(0.0, 1.5, size=topk)
                e = np.exp(z - z.max())
                p = np.sort(e / e.sum())[::-1]
                for c in range(topk):
                    parents.append(f)
                    score.append(score[f] + math.log(max(p[c], 1e-300)))
                    depth.append(depth[f] + 1)
                    new.append(len(parents) - 1)
            new.sort(key=lambda i: (-score[i], i))
            frontier = new[:topk]
        cands = sorted(range(1, len(parents)), key=lambda i: (-score[i], i))
        keep = sorted([0] + cands[:n_nodes - 1])
        if max(depth[i] for i in keep) < want_depth:
            continue
        remap = {old: new for new, old in enumerate(keep)}
        kept_parents = [-1] + [remap[parents[i]] for i in keep[1:]]
        return _bfs_relabel(kept_parents)
    raise RuntimeError("eagle_tree: depth never reached")


def specblock_tree(rng: np.random.Generator, k_block: int = 4, m_blocks: int = 3,
                   counts=(2, 4, 10, 0), probs=(0.55, 0.25, 0.15, 0.05),
                   cap: int = 96):
    """Block-iterative tree: each block runs K dependent positions from a
    start node; at each position a rank bucket is drawn and that many
    siblings are added under the current tip, the rank-1 sibling becoming the
    new tip (a bucket with zero siblings ends the chain).  Block 1 starts at
    the root; each later block starts from every rank-1 node of the previous
    expansion whose bucket was the rank-1 bucket, in creation order.  Nodes
    stay in creation order; growth stops at ``cap`` nodes.

    Returns (parents int32 [N], rank1 bool [N]).
    """
    parents = [-1]
    rank1 = [False]
    starts = [0]
    for _blk in range(m_blocks):
        next_starts = []
        for s in starts:
            tip = s
            for _k in range(k_block):
                b = int(rng.choice(len(counts), p=probs))
                cnt = counts[b]
                if cnt == 0:
                    break
                first = None
                for r in range(cnt):
                    if len(parents) >= cap:
                        break
                    parents.append(tip)
                    rank1.append(r == 0)
                    if r == 0:
                        first = len(parents) - 1
                if first is None:
                    break
                if b == 0:
                    next_starts.append(first)
                tip = first
                if len(parents) >= cap:
                    break
            if len(parents) >= cap:
                break
        starts = next_starts
        if len(parents) >= cap or not starts:
            break
    return np.asarray(parents, dtype=np.int32), np.asarray(rank1, dtype=bool)


def random_tree(rng: np.random.Generator, n_nodes: int) -> np.ndarray:
    """Uniform random recursive tree: parent of node i uniform in [0, i)."""
    parents = np.full(n_nodes, -1, dtype=np.int32)
    for i in range(1, n_nodes):
        parents[i] = int(rng.integers(i))
    return parents


def chain_tree(n_nodes: int) -> np.ndarray:
    return np.arange(-1, n_nodes - 1, dtype=np.int32)


# ---------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------

def planted_logits(rng: np.random.Generator, rows: int, vocab: int, dtype: str,
                   std: float, tie_fraction: float = _TIE_FRACTION, targets=None):
    """Logit rows with a planted maximum.

    Each row draws N(0, std^2), clipped just below a cap; the cap is written
    at a uniform random index (or at ``targets[r]`` when given) and, for
    ``tie_fraction`` of rows, also at a second, higher index.  Returns
    (logits [rows][vocab], planted int32 [rows]); the planted index is the
    lowest index holding the cap.
    """
    if targets is None:
        target = rng.integers(0, vocab, size=rows).astype(np.int32)
    else:
        target = np.asarray(targets, dtype=np.int32).copy()
    x = rng.normal(0.0, std, size=(rows, vocab)).astype(np.float32)
    if dtype == "bf16":
        np.minimum(x, np.float32(_BF16_BELOW_CAP), out=x)
        out = f32_to_bf16_bits(x)
        cap_val = f32_to_bf16_bits(np.array([_BF16_CAP], dtype=np.float32))[0]
    else:
        cap_f = np.float32(std * 5.0)
        np.minimum(x, np.nextafter(cap_f, np.float32(0)), out=x)
        out = x
        cap_val = cap_f
    tie = rng.random(rows) < tie_fraction
    partner = rng.integers(0, vocab, size=rows)
    for r in range(rows):
        out[r, target[r]] = cap_val
        if tie[r] and target[r] < vocab - 1:
            hi = int(target[r]) + 1 + int(partner[r]) % (vocab - 1 - int(target[r]))
            out[r, hi] = cap_val
    return out, target


def draft_tokens_for(rng: np.random.Generator, parents: np.ndarray, planted: np.ndarray,
                     vocab: int, p_match, match_mask=None) -> np.ndarray:
    """Node j >= 1 proposes its parent's planted target token with
    probability ``p_match`` (only where ``match_mask`` is true, if given),
    else a uniform random id.  Node 0 (the root) carries a random id."""
    n = parents.shape[0]
    out = rng.integers(0, vocab, size=n).astype(np.int32)
    u = rng.random(n)
    for j in range(1, n):
        allowed = True if match_mask is None else bool(match_mask[j])
        if allowed and u[j] < p_match:
            out[j] = planted[parents[j]]
    return out


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def kv_cache(rng: np.random.Generator, batch: int, hkv: int, capacity: int, d: int,
             prefix_len: np.ndarray) -> np.ndarray:
    """bf16 N(0,1) cache rows below each sequence's prefix length, bf16 NaN
    (0x7FC0) in every row at or past it."""
    out = np.full((batch, hkv, capacity, d), BF16_NAN, dtype=np.uint16)
    for b in range(batch):
        p = int(prefix_len[b])
        if p:
            out[b, :, :p, :] = normal_bf16(rng, (hkv, p, d))
    return out


def capacity_for(max_prefix: int, n_nodes: int) -> int:
    return ((max_prefix + n_nodes + 63) // 64) * 64


def specpv_block_list(rng: np.random.Generator, prefix_len: int, block_size: int,
                      n_sink: int, n_window: int, n_random: int) -> np.ndarray:
    """Sink blocks, the last ``n_window`` blocks and ``n_random`` distinct
    random blocks in between, sorted ascending (SpecPV App. D layout with the
    block size of the long-context workload)."""
    n_total = (prefix_len + block_size - 1) // block_size
    sink = list(range(n_sink))
    window = list(range(n_total - n_window, n_total))
    middle = np.arange(n_sink, n_total - n_window)
    pick = rng.choice(middle, size=n_random, replace=False)
    return np.asarray(sorted(sink + window + [int(x) for x in pick]), dtype=np.int32)


# SpecPV App. D: blocks of 16 tokens, 32 sink tokens (2 blocks), a 128-token
# window (8 blocks); Sec. 4.3: a 4096-token budget, so 256 blocks of which
# 246 are retrieved.
SPECPV_BLOCK_SIZE = 16
SPECPV_SINK_BLOCKS = 2
SPECPV_WINDOW_BLOCKS = 8
SPECPV_BUDGET_TOKENS = 4096
SPECPV_TOP_K = SPECPV_BUDGET_TOKENS // SPECPV_BLOCK_SIZE - SPECPV_SINK_BLOCKS - SPECPV_WINDOW_BLOCKS


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

WORKLOADS = ("tiny", "8b_layer", "specblock_tree", "batched", "long_context")
_SEED = {name: 1001 + i for i, name in enumerate(WORKLOADS)}


def _streams(seed: int):
    # fixed order: tree, logits, draft, q, k_tree, v_tree, k_cache, v_cache/blocks
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(8)]


def _assemble(name, rs, parents_list, vocab, ldt, std, p_match, hq, hkv, d,
              prefix_len, match_masks=None):
    batch = len(parents_list)
    n = max(len(p) for p in parents_list)
    if any(len(p) != n for p in parents_list):
        raise ValueError("all trees of a batch must have the same node count")
    parents = np.stack(parents_list).astype(np.int32)
    logits, planted = planted_logits(rs[1], batch * n, vocab, ldt, std)
    logits = logits.reshape(batch, n, vocab)
    planted = planted.reshape(batch, n)
    draft = np.stack([
        draft_tokens_for(rs[2], parents[b], planted[b], vocab, p_match,
                         None if match_masks is None else match_masks[b])
        for b in range(batch)])
    q = normal_bf16(rs[3], (batch, n, hq, d))
    k_tree = normal_bf16(rs[4], (batch, n, hkv, d))
    v_tree = normal_bf16(rs[5], (batch, n, hkv, d))
    prefix_len = np.asarray(prefix_len, dtype=np.int32)
    cap = capacity_for(int(prefix_len.max()), n)
    k_cache = kv_cache(rs[6], batch, hkv, cap, d, prefix_len)
    v_cache = kv_cache(rs[7], batch, hkv, cap, d, prefix_len)
    return Workload(name=name, batch=batch, n_nodes=n, n_q_heads=hq, n_kv_heads=hkv,
                    head_dim=d, vocab=vocab, logits_dtype=ldt, parents=parents,
                    draft_tokens=draft, logits=logits, q=q, k_tree=k_tree,
                    v_tree=v_tree, k_cache=k_cache, v_cache=v_cache,
                    prefix_len=prefix_len, capacity=cap, planted_target=planted)


def make_workload(name: str) -> Workload:
    """Generate one of the five named workloads (deterministic per name)."""
    rs = _streams(_SEED[name])
    if name == "tiny":
        return _assemble(name, rs, [tiny_tree(rs[0])], 1024, "f32", 1.0, 0.7,
                         4, 1, 64, [256])
    if name == "8b_layer":
        return _assemble(name, rs, [eagle_tree(rs[0], 8, 4, 60, 8)], 128256, "bf16",
                         math.sqrt(2.0), 0.75, 32, 8, 128, [1000])
    if name == "specblock_tree":
        parents, rank1 = specblock_tree(rs[0])
        return _assemble(name, rs, [parents], 128256, "bf16", math.sqrt(2.0), 0.8,
                         32, 8, 128, [4096], match_masks=[rank1])
    if name == "batched":
        seq_rngs = [np.random.Generator(np.random.PCG64(s))
                    for s in np.random.SeedSequence(_SEED[name] * 7919).spawn(16)]
        trees = [eagle_tree(r, 6, 4, 32, 6) for r in seq_rngs]
        plens = rs[0].integers(1000, 1601, size=16)
        return _assemble(name, rs, trees, 128256, "bf16", math.sqrt(2.0), 0.7,
                         32, 8, 128, plens)
    if name == "long_context":
        wl = _assemble(name, rs, [eagle_tree(rs[0], 8, 4, 60, 8)], 128256, "bf16",
                       math.sqrt(2.0), 0.75, 32, 8, 128, [60000])
        brng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(_SEED[name] * 104729)))
        blocks = specpv_block_list(brng, 60000, 64, 2, 16, 46)
        wl.block_size = 64
        wl.block_idx = blocks[None, :].copy()
        wl.n_blocks = np.array([blocks.shape[0]], dtype=np.int32)
        return wl
    raise KeyError(name)


def make_random_case(seed: int, *, batch: int, n_nodes: int, hq: int, hkv: int,
                     d: int, prefix_lens, vocab: int = 1000, ldt: str = "bf16",
                     p_match: float = 0.6, tree: str = "random", block_size: int = 0,
                     blocks_per_seq=None, name: str = "random") -> Workload:
    """Small seeded case for parity sweeps: random recursive trees (or chains),
    arbitrary prefix lengths, optional random partial block lists."""
    rs = _streams(seed)
    trees = []
    for _b in range(batch):
        if tree == "chain":
            trees.append(chain_tree(n_nodes))
        else:
            trees.append(random_tree(rs[0], n_nodes))
    std = math.sqrt(2.0) if ldt == "bf16" else 1.0
    wl = _assemble(name, rs, trees, vocab, ldt, std, p_match, hq, hkv, d,
                   list(prefix_lens))
    if block_size:
        brng = np.random.Generator(np.random.PCG64(seed * 31 + 7))
        lists = []
        for b in range(batch):
            p = int(wl.prefix_len[b])
            n_avail = (p + block_size - 1) // block_size
            want = n_avail if blocks_per_seq is None else min(blocks_per_seq, n_avail)
            pick = brng.choice(n_avail, size=want, replace=False) if n_avail else np.zeros(0, int)
            lists.append(np.sort(pick).astype(np.int32))
        max_blocks = max(1, max(len(x) for x in lists))
        bidx = np.full((batch, max_blocks), -1, dtype=np.int32)
        for b, x in enumerate(lists):
            bidx[b, :len(x)] = x
        wl.block_size = block_size
        wl.block_idx = bidx
        wl.n_blocks = np.array([len(x) for x in lists], dtype=np.int32)
    return wl


def make_select_case(seed: int, *, batch: int, n_nodes: int, hq: int, hkv: int, d: int,
                     prefix_lens, block_size: int, n_planted: int = 0,
                     query_lean: float = 2.0, key_lean: float | None = None) -> Workload:
    """Seeded case for block selection: N(0,1) bf16 queries and keys, plus,
    when ``n_planted`` > 0, planted relevant blocks.

    For each sequence a random unit direction u is drawn; every query gets
    ``query_lean * u`` added, and one random token in each of ``n_planted``
    distinct random blocks below the prefix gets ``key_lean * u`` added to its
    key in every KV head (default key_lean = 8 * sqrt(d)).  The planted block
    ids are returned in ``wl.block_idx`` / ``wl.n_blocks`` (bookkeeping only,
    not an input of the method).
    """
    wl = make_random_case(seed, batch=batch, n_nodes=n_nodes, hq=hq, hkv=hkv, d=d,
                          prefix_lens=prefix_lens, name="select")
    wl.block_size = block_size
    if not n_planted:
        return wl
    if key_lean is None:
        key_lean = 8.0 * math.sqrt(d)
    rng = np.random.Generator(np.random.PCG64(seed * 7 + 3))
    q = bf16_bits_to_f32(wl.q)
    planted = np.full((batch, n_planted), -1, dtype=np.int32)
    counts = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        u = rng.standard_normal(d).astype(np.float32)
        u /= np.float32(np.linalg.norm(u))
        q[b] += np.float32(query_lean) * u
        p = int(wl.prefix_len[b])
        n_avail = (p + block_size - 1) // block_size
        take = min(n_planted, n_avail)
        blocks = np.sort(rng.choice(n_avail, size=take, replace=False)) if take else []
        for t, blk in enumerate(blocks):
            lo, hi = int(blk) * block_size, min((int(blk) + 1) * block_size, p)
            row = int(rng.integers(lo, hi))
            k = bf16_bits_to_f32(wl.k_cache[b, :, row, :])
            wl.k_cache[b, :, row, :] = f32_to_bf16_bits(k + np.float32(key_lean) * u)
            planted[b, t] = blk
        counts[b] = take
    wl.q = f32_to_bf16_bits(q)
    wl.block_idx, wl.n_blocks = planted, counts
    return wl


# ---------------------------------------------------------------------------
# SpecPV multi-step scenarios (partial steps and rectifying full steps)
# ---------------------------------------------------------------------------

def _step_rng(seed: int, step: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, step, stream])))


def specpv_draft(seed: int, step: int, n_nodes: int, vocab: int, p_match: float):
    """The draft side of one step: a random recursive tree of ``n_nodes``, the
    target token planted in each node's logits row, and draft tokens (a child
    proposes its parent's planted token with probability ``p_match``).
    Returns (parents, planted, draft_tokens); draft_tokens[0] is a placeholder
    for the root."""
    rng = _step_rng(seed, step, 0)
    parents = random_tree(rng, n_nodes)
    planted = rng.integers(0, vocab, size=n_nodes).astype(np.int32)
    draft = draft_tokens_for(rng, parents, planted, vocab, p_match)
    return parents, planted, draft


def specpv_step_inputs(seed: int, step: int, tokens, n_chain: int, planted_draft, *, vocab: int,
                       hq: int, hkv: int, d: int, p_keep: float):
    """Queries, tree K/V and bf16 logits for the nodes of one step's tree.

    ``tokens`` are the tree's node tokens; the first ``n_chain`` nodes are a
    chain of previously emitted tokens (empty for a partial step) and the rest
    is the draft tree, whose rows plant ``planted_draft``.  Chain row k plants
    the token of node k + 1 with probability ``p_keep`` (the partial step's
    choice survives re-verification), else a uniform random id."""
    tokens = np.asarray(tokens, dtype=np.int32)
    n = tokens.shape[0]
    rng = _step_rng(seed, step, 1 + n_chain)
    targets = np.empty(n, dtype=np.int32)
    keep = rng.random(max(n_chain, 1)) < p_keep
    other = rng.integers(0, vocab, size=max(n_chain, 1))
    for k in range(n_chain):
        targets[k] = tokens[k + 1] if keep[k] else other[k]
    targets[n_chain:] = np.asarray(planted_draft, dtype=np.int32)
    logits, _ = planted_logits(rng, n, vocab, "bf16", math.sqrt(2.0), targets=targets)
    q = normal_bf16(rng, (1, n, hq, d))
    k_tree = normal_bf16(rng, (1, n, hkv, d))
    v_tree = normal_bf16(rng, (1, n, hkv, d))
    return q, k_tree, v_tree, logits.reshape(1, n, vocab)


def long_context_with_tree(parents, name: str = "long_context_tree") -> Workload:
    """The long-context shape (batch 1, 60000-token prefix, 32 query / 8 KV
    heads of 128, 128256-token bf16 logits) verifying the given tree, with
    fresh seeded queries, tree K/V, logits and draft tokens for its nodes."""
    parents = np.asarray(parents, dtype=np.int32)
    rs = _streams(_SEED["long_context"] * 3 + parents.shape[0])
    return _assemble(name, rs, [parents], 128256, "bf16", math.sqrt(2.0), 0.75, 32, 8, 128,
                     [60000])


# ---------------------------------------------------------------------------
# sampling (temperature > 0) cases
# ---------------------------------------------------------------------------

def sampling_logits(rng: np.random.Generator, rows: int, vocab: int, dtype: str, targets,
                    lean=(9.0, 16.0)) -> np.ndarray:
    """Logit rows shaped like a language model's at sampling time: N(0, 1)
    background, the planted target token at U[lean] above 0 and a runner-up
    token 0.5-3 below it, so that the target's probability ranges from a few
    percent to nearly one.  bf16 (uint16 bits) or fp32 [rows][vocab]."""
    x = rng.standard_normal(size=(rows, vocab), dtype=np.float32)
    top = rng.uniform(lean[0], lean[1], size=rows).astype(np.float32)
    gap = rng.uniform(0.5, 3.0, size=rows).astype(np.float32)
    other = rng.integers(0, vocab, size=rows)
    for r in range(rows):
        x[r, other[r]] = top[r] - gap[r]
        x[r, int(targets[r])] = top[r]
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def make_sampling_case(seed: int, *, batch: int, n_nodes: int, vocab: int, dtype: str = "bf16",
                       p_match: float = 0.8, tree: str = "eagle", lean=(9.0, 16.0)):
    """Trees, draft tokens and logits for stochastic verification.  Returns
    (parents [B][N], draft_tokens [B][N], logits [B][N][V])."""
    rs = _streams(seed * 13 + 5)
    trees = []
    for _ in range(batch):
        if tree == "chain" or n_nodes == 1:
            trees.append(chain_tree(n_nodes))
        elif tree == "random":
            trees.append(random_tree(rs[0], n_nodes))
        else:
            depth = max(1, min(8, n_nodes - 1))
            trees.append(eagle_tree(rs[0], depth, 4, n_nodes, depth))
    parents = np.stack(trees).astype(np.int32)
    planted = rs[1].integers(0, vocab, size=(batch, n_nodes)).astype(np.int32)
    logits = sampling_logits(rs[2], batch * n_nodes, vocab, dtype, planted.reshape(-1), lean)
    draft = np.stack([draft_tokens_for(rs[3], parents[b], planted[b], vocab, p_match)
                      for b in range(batch)])
    return parents, draft, logits.reshape(batch, n_nodes, vocab)
