"""Pins for the fp64 block-selection oracle (SpecPV Sec. 3.2, App. C, App. D).

Each check compares the oracle with something other than itself: the defining
properties of an element-wise max and min (containment and attainment), brute
force over the corners of the key box, brute-force counting for the top-k
rule, hand-worked selections and planted relevant blocks.  All CPU.
"""

import itertools
import statistics

import numpy as np
import pytest

import oracle
from oracle import OracleInputError
from tree_verification_attention_tv_amd import workloads as W


def widen(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def block_rows(wl, b, g, j):
    p = int(wl.prefix_len[b])
    bs = wl.block_size
    return widen(wl.k_cache[b, g, j * bs:min((j + 1) * bs, p), :])


CASES = [
    # seed, batch, n_nodes, hq, hkv, d, prefix_lens, block_size
    (1, 1, 5, 4, 2, 4, [23], 4),
    (2, 2, 3, 2, 1, 4, [16, 9], 8),
    (3, 1, 1, 2, 2, 4, [7], 1),
    (4, 3, 6, 6, 3, 4, [0, 5, 33], 5),
]


# ---------------------------------------------------------------------------
# summaries
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", CASES)
def test_p13_summary_contains_and_attains_every_coordinate(case):
    seed, batch, n, hq, hkv, d, plens, bs = case
    wl = W.make_select_case(seed, batch=batch, n_nodes=n, hq=hq, hkv=hkv, d=d,
                            prefix_lens=plens, block_size=bs, n_planted=1)
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, bs)
    for b in range(batch):
        p = int(wl.prefix_len[b])
        assert nv[b] == (p + bs - 1) // bs
        assert np.all(np.isnan(kmax[b, :, nv[b]:])) and np.all(np.isnan(kmin[b, :, nv[b]:]))
        for g in range(hkv):
            for j in range(nv[b]):
                rows = block_rows(wl, b, g, j)
                assert rows.shape[0] >= 1
                for dd in range(d):
                    col = [float(x) for x in rows[:, dd]]
                    # every token lies inside [min, max], and both ends are some token
                    assert all(kmin[b, g, j, dd] <= x <= kmax[b, g, j, dd] for x in col)
                    assert kmax[b, g, j, dd] in col and kmin[b, g, j, dd] in col


def test_summaries_ignore_rows_past_the_prefix():
    # the generator puts bf16 NaN in every cache row at or past the prefix
    wl = W.make_select_case(5, batch=1, n_nodes=2, hq=2, hkv=1, d=4, prefix_lens=[10],
                            block_size=4)
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, 4)
    assert nv[0] == 3
    assert np.all(np.isfinite(kmax[0, :, :3])) and np.all(np.isfinite(kmin[0, :, :3]))


# ---------------------------------------------------------------------------
# scores
# ---------------------------------------------------------------------------

def corner_max(qv, hi, lo):
    """Largest q.k over the 2^D corners of the box [lo, hi] (brute force)."""
    best = -np.inf
    for pick in itertools.product((0, 1), repeat=len(qv)):
        corner = [hi[t] if pick[t] else lo[t] for t in range(len(qv))]
        best = max(best, sum(float(a) * float(c) for a, c in zip(qv, corner)))
    return best


def brute_scores(wl, reduction):
    """Scores by nested loops over sequences, blocks, heads and nodes, with the
    bound taken as a maximum over corners and the head's KV group written out."""
    bs = wl.block_size
    q = widen(wl.q)
    grp = wl.n_q_heads // wl.n_kv_heads
    out = {}
    for b in range(wl.batch):
        p = int(wl.prefix_len[b])
        for j in range((p + bs - 1) // bs):
            per_head = []
            for h in range(wl.n_q_heads):
                rows = block_rows(wl, b, h // grp, j)
                hi, lo = rows.max(axis=0), rows.min(axis=0)
                per_node = [corner_max(q[b, i, h], hi, lo) for i in range(wl.n_nodes)]
                if reduction == "mean":
                    per_head.append(statistics.fmean(per_node))
                elif reduction == "max":
                    per_head.append(max(per_node))
                else:
                    per_head.append(per_node[wl.n_nodes - 1])
            out[(b, j)] = statistics.fmean(per_head)
    return out


@pytest.mark.parametrize("reduction", ["mean", "max", "last"])
@pytest.mark.parametrize("case", CASES)
def test_p14_scores_equal_corner_brute_force(case, reduction):
    seed, batch, n, hq, hkv, d, plens, bs = case
    wl = W.make_select_case(seed, batch=batch, n_nodes=n, hq=hq, hkv=hkv, d=d,
                            prefix_lens=plens, block_size=bs, n_planted=1)
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, bs)
    sc = oracle.block_scores(wl.q, kmax, kmin, nv, reduction)
    want = brute_scores(wl, reduction)
    for (b, j), v in want.items():
        assert sc[b, j] == pytest.approx(v, rel=1e-12, abs=1e-12)
    for b in range(batch):
        assert np.all(np.isnan(sc[b, nv[b]:]))


@pytest.mark.parametrize("seed", range(4))
def test_p14_bound_holds_for_every_token(seed):
    # one node and one head: the block score is the bound of that query itself
    wl = W.make_select_case(seed, batch=1, n_nodes=1, hq=1, hkv=1, d=16, prefix_lens=[45],
                            block_size=6, n_planted=2)
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, 6)
    sc = oracle.block_scores(wl.q, kmax, kmin, nv, "mean")
    q = widen(wl.q)[0, 0, 0]
    tight = 0
    for j in range(nv[0]):
        dots = block_rows(wl, 0, 0, j) @ q
        assert np.all(dots <= sc[0, j] + 1e-9)
        tight += bool(np.max(dots) < sc[0, j] - 1e-6)
    assert tight > 0      # with several tokens per block the bound is usually loose


def test_p14_single_token_block_is_exact_dot_product():
    # block size 1: the box is one point, so the bound is q.k itself
    wl = W.make_select_case(9, batch=1, n_nodes=3, hq=2, hkv=1, d=16, prefix_lens=[5],
                            block_size=1)
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, 1)
    sc = oracle.block_scores(wl.q, kmax, kmin, nv, "mean")
    q = widen(wl.q)[0]                       # [N][Hq][D]
    k = widen(wl.k_cache[0, 0, :5, :])       # [5][D]
    want = np.einsum("nhd,jd->j", q, k) / (3 * 2)
    np.testing.assert_allclose(sc[0, :5], want, rtol=1e-12, atol=1e-12)


def test_reductions_coincide_for_one_node():
    wl = W.make_select_case(11, batch=1, n_nodes=1, hq=4, hkv=2, d=8, prefix_lens=[30],
                            block_size=4, n_planted=1)
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, 4)
    s = [oracle.block_scores(wl.q, kmax, kmin, nv, r) for r in oracle.REDUCTIONS]
    np.testing.assert_array_equal(s[0], s[1])
    np.testing.assert_array_equal(s[0], s[2])


def test_score_block_subset_matches_full_scoring():
    wl = W.make_select_case(12, batch=2, n_nodes=3, hq=4, hkv=2, d=8, prefix_lens=[50, 21],
                            block_size=4)
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, 4)
    full = oracle.block_scores(wl.q, kmax, kmin, nv, "max")
    part = oracle.block_scores(wl.q, kmax, kmin, nv, "max", blocks=[0, 5, 12])
    for b in range(2):
        for j in range(full.shape[1]):
            if j in (0, 5, 12) and j < nv[b]:
                assert part[b, j] == full[b, j]
            else:
                assert np.isnan(part[b, j])


def test_magnitude_bounds_the_terms():
    wl = W.make_select_case(13, batch=1, n_nodes=4, hq=4, hkv=2, d=8, prefix_lens=[40],
                            block_size=8, n_planted=1)
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, 8)
    for red in oracle.REDUCTIONS:
        s = oracle.block_scores(wl.q, kmax, kmin, nv, red)
        m = oracle.block_scores(wl.q, kmax, kmin, nv, red, magnitude=True)
        assert np.all(np.abs(s[0, :nv[0]]) <= m[0, :nv[0]] + 1e-12)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def brute_select(scores, n_valid, n_sink, n_window, top_k):
    """Keep block j if it is a sink, in the window, or fewer than top_k other
    candidates come before it (higher score, or equal score and lower id)."""
    keep = []
    cands = [j for j in range(n_valid) if j >= n_sink and j < n_valid - n_window]
    for j in range(n_valid):
        if j < n_sink or j >= n_valid - n_window:
            keep.append(j)
            continue
        ahead = sum(1 for c in cands
                    if scores[c] > scores[j] or (scores[c] == scores[j] and c < j))
        if ahead < top_k:
            keep.append(j)
    return keep


def test_p17_hand_worked_selection():
    scores = [5.0, 1.0, 3.0, 3.0, 2.0, 9.0, 0.0]
    # sink {0}, window {6}; candidates 1..5 -> 5 (9.0) then 2 (3.0, beats 3 on id)
    assert list(oracle.select_blocks(scores, 7, 1, 1, 2)) == [0, 2, 5, 6]
    assert list(oracle.select_blocks(scores, 7, 1, 1, 3)) == [0, 2, 3, 5, 6]
    assert list(oracle.select_blocks(scores, 7, 0, 0, 1)) == [5]
    assert list(oracle.select_blocks(scores, 7, 2, 3, 0)) == [0, 1, 4, 5, 6]
    # a block cannot be chosen twice and the window may overlap the sinks
    assert list(oracle.select_blocks(scores, 3, 2, 2, 5)) == [0, 1, 2]
    assert list(oracle.select_blocks(scores, 0, 2, 8, 5)) == []
    # every candidate fits
    assert list(oracle.select_blocks(scores, 7, 1, 1, 99)) == list(range(7))


@pytest.mark.parametrize("seed", range(30))
def test_p17_selection_equals_brute_force_counting(seed):
    rng = np.random.default_rng(seed)
    nv = int(rng.integers(0, 40))
    # few distinct values, so ties are common
    scores = rng.integers(-3, 4, size=max(nv, 1)).astype(np.float64)
    n_sink, n_window, top_k = (int(x) for x in rng.integers(0, 6, size=3))
    got = oracle.select_blocks(scores, nv, n_sink, n_window, top_k)
    assert list(got) == brute_select(scores, nv, n_sink, n_window, top_k)
    assert len(set(got.tolist())) == len(got)
    fixed = set(range(min(n_sink, nv))) | set(range(max(nv - n_window, 0), nv))
    assert len(got) == len(fixed) + min(top_k, nv - len(fixed))


def test_selection_rejects_nan_and_negative_sizes():
    with pytest.raises(OracleInputError):
        oracle.select_blocks([0.0, np.nan, 1.0, 2.0], 4, 1, 1, 1)
    with pytest.raises(OracleInputError):
        oracle.select_blocks([0.0], 1, -1, 0, 0)


@pytest.mark.parametrize("reduction", ["mean", "max", "last"])
@pytest.mark.parametrize("seed", range(3))
def test_p18_planted_blocks_are_retrieved(seed, reduction):
    wl = W.make_select_case(100 + seed, batch=2, n_nodes=6, hq=8, hkv=2, d=64,
                            prefix_lens=[400, 333], block_size=16, n_planted=3)
    lists, sc, _, _, nv = oracle.specpv_select(wl.q, wl.k_cache, wl.prefix_len, block_size=16,
                                               n_sink=1, n_window=2, top_k=3,
                                               reduction=reduction)
    for b in range(2):
        planted = set(int(x) for x in wl.block_idx[b, :wl.n_blocks[b]])
        assert planted <= set(int(x) for x in lists[b])
        assert {0, nv[b] - 2, nv[b] - 1} <= set(int(x) for x in lists[b])


def test_specpv_settings_from_the_pages():
    # App. D: 16-token blocks, 32 sink tokens, 128-token window; 4096-token budget
    assert W.SPECPV_BLOCK_SIZE * W.SPECPV_SINK_BLOCKS == 32
    assert W.SPECPV_BLOCK_SIZE * W.SPECPV_WINDOW_BLOCKS == 128
    assert (W.SPECPV_SINK_BLOCKS + W.SPECPV_WINDOW_BLOCKS + W.SPECPV_TOP_K) * \
        W.SPECPV_BLOCK_SIZE == W.SPECPV_BUDGET_TOKENS
