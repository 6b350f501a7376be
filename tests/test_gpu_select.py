"""Parity of SpecPV block selection on the GPU with the fp64 oracle.

* Summaries: bit-exact values (a block's max and min are bf16 values of its
  keys; a zero may differ in sign only).  Records outside the updated range
  are untouched.
* Scores: |gpu - oracle| <= (N*G + 2*D + Hq + 64) * 2^-24 * M per block, M the
  same reduction over sum_d |q_d| * max(|hi_d|, |lo_d|): the fp32 rounding
  bound of the query fold (N*G terms), the 2D-term dot product or MFMA
  accumulation, and the sums over heads.
* Selection: bit-exact against the oracle's selection run on the GPU's own
  fp32 scores (same inputs, same comparisons), and valid against the fp64
  scores: no unselected candidate beats a selected one by more than the two
  tolerances.  Where the fp64 ranking has a clear gap at the cut (planted
  blocks), the lists are identical.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W

from .gpu_util import (DevWorkload, bf16_host, bf16_to_f64, check_attention_close, dev_bf16,
                       dev_i32, oracle_attention)

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F7F  # a finite bf16 pattern no summary of N(0,1) keys produces
U32 = 2.0 ** -24


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def summaries_gpu(dw, bs, *, first_token=None, sentinel=True):
    shape = binding.summaries_shape(dw.k_cache, bs)
    s = torch.empty(shape, dtype=torch.bfloat16, device=dw.k_cache.device)
    if sentinel:
        s.view(torch.int16).fill_(SENTINEL)
    err = torch.zeros(1, dtype=torch.int32, device=s.device)
    binding.block_summaries(dw.k_cache, dw.prefix_len, block_size=bs, first_token=first_token,
                            max_tokens=dw.wl.capacity, summaries=s, dev_err=err)
    return s, err


def check_summaries(s_gpu, wl, bs, blocks=None):
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, bs)
    got = bf16_to_f64(s_gpu)                      # [B][Hkv][nb][2][D]
    raw = bf16_host(s_gpu)
    for b in range(wl.batch):
        js = range(nv[b]) if blocks is None else [j for j in blocks if j < nv[b]]
        js = np.asarray(list(js), dtype=np.int64)
        if js.size:
            assert np.array_equal(got[b, :, js, 0, :], kmax[b, :, js, :]), f"max, seq {b}"
            assert np.array_equal(got[b, :, js, 1, :], kmin[b, :, js, :]), f"min, seq {b}"
        assert np.all(raw[b, :, nv[b]:] == SENTINEL), f"records past the prefix written, seq {b}"
    return kmax, kmin, nv


def score_tol(wl, mag):
    grp = wl.n_q_heads // wl.n_kv_heads
    return (wl.n_nodes * grp + 2 * wl.head_dim + wl.n_q_heads + 64) * U32 * mag


def run_select(dw, summ, bs, n_sink, n_window, top_k, reduction, max_blocks=None):
    err = torch.zeros(1, dtype=torch.int32, device=summ.device)
    bidx, nblk, sc = binding.select_blocks(
        dw.q, summ, dw.prefix_len, cache_capacity=dw.wl.capacity,
        max_prefix_len=dw.wl.max_prefix_len, block_size=bs, n_sink=n_sink, n_window=n_window,
        top_k=top_k, reduction=reduction, max_blocks=max_blocks, want_scores=True, dev_err=err)
    torch.cuda.synchronize()
    return bidx.cpu().numpy(), nblk.cpu().numpy(), sc.cpu().numpy().astype(np.float64), \
        int(err.item())


def check_selection(wl, bidx, nblk, sc_gpu, s64, tol, nv, n_sink, n_window, top_k,
                    exact_when_gapped=False):
    for b in range(wl.batch):
        got = bidx[b, :nblk[b]]
        assert np.all(bidx[b, nblk[b]:] == -1), "tail of the list not cleared"
        want_on_gpu_scores = oracle.select_blocks(sc_gpu[b], nv[b], n_sink, n_window, top_k)
        assert np.array_equal(got, want_on_gpu_scores), f"seq {b}: selection rule differs"
        # valid against fp64 scores
        lo, hi = min(n_sink, nv[b]), max(nv[b] - n_window, min(n_sink, nv[b]))
        cand = np.arange(lo, hi)
        chosen = np.isin(cand, got)
        if chosen.any() and (~chosen).any():
            worst_in = np.min(s64[b, cand[chosen]] + tol[b, cand[chosen]])
            best_out = np.max(s64[b, cand[~chosen]] - tol[b, cand[~chosen]])
            assert worst_in >= best_out, f"seq {b}: a clearly better block was left out"
        if exact_when_gapped:
            want = oracle.select_blocks(s64[b], nv[b], n_sink, n_window, top_k)
            assert np.array_equal(got, want), f"seq {b}: differs from the fp64 selection"


# ---------------------------------------------------------------------------
# summaries
# ---------------------------------------------------------------------------

SUM_CASES = [
    # seed, batch, hq, hkv, d, prefix_lens, block_size
    (1, 1, 4, 2, 128, [257], 16),
    (2, 3, 8, 2, 64, [0, 1, 100], 16),
    (3, 2, 4, 4, 128, [64, 1000], 64),
    (4, 2, 2, 1, 128, [37, 5], 1),
    (5, 1, 8, 8, 64, [333], 7),
]


@pytest.mark.parametrize("case", SUM_CASES)
def test_summaries_match_oracle(case):
    seed, batch, hq, hkv, d, plens, bs = case
    _say(f"[summaries] seed {seed} batch {batch} d {d} prefix {plens} block {bs}")
    wl = W.make_select_case(seed, batch=batch, n_nodes=4, hq=hq, hkv=hkv, d=d,
                            prefix_lens=plens, block_size=bs, n_planted=2)
    dw = DevWorkload(wl)
    s, err = summaries_gpu(dw, bs)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_summaries(s, wl, bs)


def test_summaries_incremental_update_after_commit():
    _say("[summaries] incremental update")
    bs = 16
    wl = W.make_select_case(21, batch=2, n_nodes=4, hq=8, hkv=2, d=128, prefix_lens=[300, 47],
                            block_size=bs)
    dw = DevWorkload(wl)
    old = dw.prefix_len.clone()
    s, _ = summaries_gpu(dw, bs)
    # the next step commits 13 and 40 rows: write them to the cache and grow the prefix
    grow = np.array([13, 40], dtype=np.int32)
    rng = np.random.default_rng(5)
    for b in range(2):
        p0 = int(wl.prefix_len[b])
        rows = W.normal_bf16(rng, (wl.n_kv_heads, int(grow[b]), wl.head_dim))
        wl.k_cache[b, :, p0:p0 + grow[b], :] = rows
        dw.k_cache[b, :, p0:p0 + grow[b], :] = dev_bf16(rows)
    wl.prefix_len = wl.prefix_len + grow
    dw.prefix_len = dev_i32(wl.prefix_len)
    before = bf16_host(s).copy()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.block_summaries(dw.k_cache, dw.prefix_len, block_size=bs, first_token=old,
                            max_tokens=int(grow.max()), summaries=s, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_summaries(s, wl, bs)
    after = bf16_host(s)
    for b in range(2):
        first = int(old[b].item()) // bs
        assert np.array_equal(after[b, :, :first], before[b, :, :first]), "untouched blocks changed"


def test_summaries_bad_prefix_skips_the_sequence():
    _say("[summaries] bad prefix")
    wl = W.make_select_case(22, batch=2, n_nodes=4, hq=4, hkv=2, d=64, prefix_lens=[40, 40],
                            block_size=8)
    dw = DevWorkload(wl)
    dw.prefix_len = dev_i32([40, wl.capacity + 1])
    s, err = summaries_gpu(dw, 8)
    torch.cuda.synchronize()
    assert int(err.item()) & binding.DERR_BAD_PREFIX
    raw = bf16_host(s)
    assert np.all(raw[1] == SENTINEL)
    wl.prefix_len = np.array([40, 0], dtype=np.int32)
    kmax, _, _ = oracle.block_summaries(wl.k_cache, wl.prefix_len, 8)
    assert np.array_equal(bf16_to_f64(s)[0, :, :5, 0, :], kmax[0, :, :5, :])


# ---------------------------------------------------------------------------
# scores and selection
# ---------------------------------------------------------------------------

SEL_CASES = [
    # seed, batch, n_nodes, hq, hkv, d, prefix_lens, block_size, sink, window, top_k, planted
    (31, 1, 60, 32, 8, 128, [3000], 16, 2, 8, 40, 0),
    (32, 3, 7, 8, 2, 64, [0, 90, 777], 16, 2, 3, 5, 0),
    (33, 2, 33, 16, 4, 128, [1500, 1499], 8, 1, 4, 30, 12),
    (34, 1, 17, 4, 1, 128, [513], 1, 4, 16, 64, 0),
    (35, 2, 20, 8, 8, 64, [2047, 64], 32, 2, 2, 10, 6),
    (36, 1, 256, 4, 4, 128, [640], 16, 0, 0, 7, 0),
]


@pytest.mark.parametrize("reduction", ["mean", "max", "last"])
@pytest.mark.parametrize("case", SEL_CASES)
def test_scores_and_selection_match_oracle(case, reduction):
    seed, batch, n, hq, hkv, d, plens, bs, n_sink, n_window, top_k, planted = case
    _say(f"[select] seed {seed} {reduction} batch {batch} N {n} Hq {hq} Hkv {hkv} D {d} "
         f"prefix {plens} block {bs} sink {n_sink} window {n_window} k {top_k}")
    wl = W.make_select_case(seed, batch=batch, n_nodes=n, hq=hq, hkv=hkv, d=d,
                            prefix_lens=plens, block_size=bs, n_planted=planted)
    dw = DevWorkload(wl)
    summ, _ = summaries_gpu(dw, bs)
    bidx, nblk, sc, err = run_select(dw, summ, bs, n_sink, n_window, top_k, reduction)
    assert err == 0
    kmax, kmin, nv = oracle.block_summaries(wl.k_cache, wl.prefix_len, bs)
    s64 = oracle.block_scores(wl.q, kmax, kmin, nv, reduction)
    mag = oracle.block_scores(wl.q, kmax, kmin, nv, reduction, magnitude=True)
    tol = score_tol(wl, mag)
    for b in range(batch):
        v = slice(0, nv[b])
        diff = np.abs(sc[b, v] - s64[b, v])
        assert np.all(diff <= tol[b, v]), \
            f"seq {b}: score error {diff.max():.3g} > tolerance {tol[b, v].min():.3g}"
    check_selection(wl, bidx, nblk, sc, s64, tol, nv, n_sink, n_window, top_k)
    if planted:
        for b in range(batch):
            got = set(bidx[b, :nblk[b]].tolist())
            assert set(wl.block_idx[b, :wl.n_blocks[b]].tolist()) <= got


def test_equal_scores_take_the_lowest_block_ids():
    _say("[select] all scores equal")
    bs = 16
    wl = W.make_select_case(41, batch=1, n_nodes=5, hq=8, hkv=2, d=128, prefix_lens=[16 * 300],
                            block_size=bs)
    # every block holds the same 16 keys, so every block's score is the same number
    wl.k_cache[:, :, 16:16 * 300, :] = np.tile(wl.k_cache[:, :, :16, :], (1, 1, 299, 1))
    dw = DevWorkload(wl)
    summ, _ = summaries_gpu(dw, bs)
    for red in ("mean", "max", "last"):
        bidx, nblk, sc, err = run_select(dw, summ, bs, 2, 8, 37, red)
        assert err == 0 and np.all(sc[0, :300] == sc[0, 0])
        want = list(range(2 + 37)) + list(range(292, 300))
        assert bidx[0, :nblk[0]].tolist() == want


@pytest.mark.parametrize("n_sink,n_window,top_k,plen", [
    (2, 8, 246, 0), (2, 8, 246, 20), (4, 4, 0, 800), (2, 8, 10_000, 1600), (0, 0, 3, 48),
    (50, 0, 1, 400), (0, 60, 2, 400)])
def test_selection_edge_cases(n_sink, n_window, top_k, plen):
    _say(f"[select] edge sink {n_sink} window {n_window} k {top_k} prefix {plen}")
    bs = 16
    wl = W.make_select_case(51, batch=1, n_nodes=6, hq=4, hkv=2, d=64, prefix_lens=[plen],
                            block_size=bs)
    dw = DevWorkload(wl)
    summ, _ = summaries_gpu(dw, bs)
    max_blocks = n_sink + n_window + top_k + 3
    bidx, nblk, sc, err = run_select(dw, summ, bs, n_sink, n_window, top_k, "mean", max_blocks)
    assert err == 0
    nv = (plen + bs - 1) // bs
    want = oracle.select_blocks(sc[0], nv, n_sink, n_window, top_k)
    assert bidx[0, :nblk[0]].tolist() == want.tolist()
    assert np.all(bidx[0, nblk[0]:] == -1)


def test_selection_bad_prefix_is_clamped_and_flagged():
    _say("[select] bad prefix")
    bs = 16
    wl = W.make_select_case(52, batch=2, n_nodes=6, hq=4, hkv=2, d=64, prefix_lens=[300, 300],
                            block_size=bs)
    dw = DevWorkload(wl)
    summ, _ = summaries_gpu(dw, bs)
    dw.prefix_len = dev_i32([300, -5])
    bidx, nblk, sc, err = run_select(dw, summ, bs, 1, 1, 3, "mean")
    assert err & binding.DERR_BAD_PREFIX
    assert nblk[1] == 0 and np.all(bidx[1] == -1)
    assert nblk[0] == 5


def test_selected_list_drives_partial_attention():
    _say("[select] selection -> partial attention")
    bs = 16
    wl = W.make_select_case(61, batch=2, n_nodes=12, hq=8, hkv=2, d=128, prefix_lens=[700, 433],
                            block_size=bs, n_planted=4)
    dw = DevWorkload(wl)
    summ, _ = summaries_gpu(dw, bs)
    bidx, nblk = binding.select_blocks(dw.q, summ, dw.prefix_len, cache_capacity=wl.capacity,
                                       max_prefix_len=wl.max_prefix_len, block_size=bs,
                                       n_sink=2, n_window=4, top_k=9)
    mask, _ = binding.build_tree_mask(dw.parents)
    out = binding.tree_attention(dw.q, dw.k_cache, dw.v_cache, dw.k_tree, dw.v_tree,
                                 dw.prefix_len, mask, max_prefix_len=wl.max_prefix_len,
                                 block_idx=bidx, n_blocks=nblk, block_size=bs)
    torch.cuda.synchronize()
    wl.block_idx, wl.n_blocks, wl.block_size = bidx.cpu().numpy(), nblk.cpu().numpy(), bs
    ref, _ = oracle_attention(wl, partial=True)
    check_attention_close(out, ref, "attention over the selected blocks")


@pytest.mark.parametrize("reduction", ["mean", "max"])
@pytest.mark.parametrize("plen,bs", [(100_000, 16), (131_072, 4)])
def test_many_blocks_per_sequence(plen, bs, reduction):
    # 6250 and 32768 blocks: 16 and 32 blocks per selection thread
    _say(f"[select] {plen} tokens, block {bs}, {reduction}")
    wl = W.make_select_case(71, batch=1, n_nodes=9, hq=8, hkv=2, d=64, prefix_lens=[plen],
                            block_size=bs, n_planted=5)
    dw = DevWorkload(wl)
    summ, _ = summaries_gpu(dw, bs)
    bidx, nblk, sc, err = run_select(dw, summ, bs, 3, 9, 333, reduction)
    assert err == 0
    nv = (plen + bs - 1) // bs
    want = oracle.select_blocks(sc[0], nv, 3, 9, 333)
    assert np.array_equal(bidx[0, :nblk[0]], want)
    assert set(wl.block_idx[0, :wl.n_blocks[0]].tolist()) <= set(want.tolist())
    rng = np.random.default_rng(3)
    sample = sorted(set(rng.choice(nv, 48, replace=False).tolist()) | {0, nv - 1})
    kmax, kmin, nv_o = check_summaries(summ, wl, bs, blocks=sample)
    s64 = oracle.block_scores(wl.q, kmax, kmin, nv_o, reduction, blocks=sample)
    mag = oracle.block_scores(wl.q, kmax, kmin, nv_o, reduction, blocks=sample, magnitude=True)
    assert np.all(np.abs(sc[0, sample] - s64[0, sample]) <= score_tol(wl, mag)[0, sample])


def test_too_many_blocks_is_refused():
    wl = W.make_select_case(72, batch=1, n_nodes=2, hq=2, hkv=1, d=64, prefix_lens=[40],
                            block_size=1)
    dw = DevWorkload(wl)
    summ = torch.empty(binding.summaries_shape(dw.k_cache, 1), dtype=torch.bfloat16,
                       device="cuda")
    d = binding.select_desc(dw.q, summ, cache_capacity=binding.MAX_SELECT_BLOCKS + 1,
                            max_prefix_len=binding.MAX_SELECT_BLOCKS + 1, block_size=1,
                            n_sink=1, n_window=1, top_k=1)
    assert binding.select_workspace_size(d) == 0
    d.max_prefix_len = binding.MAX_SELECT_BLOCKS
    assert binding.select_workspace_size(d) > 0


# ---------------------------------------------------------------------------
# the 60K-token long-context shape at the pages' settings, sampled
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def long_context():
    wl = W.make_workload("long_context").without_blocks()
    return wl, DevWorkload(wl)


@pytest.mark.parametrize("reduction", ["mean", "max"])
def test_long_context_selection_sampled(long_context, reduction):
    wl, dw = long_context
    bs = W.SPECPV_BLOCK_SIZE
    _say(f"[select] long_context 60000 tokens, block {bs}, {reduction}")
    summ, err = summaries_gpu(dw, bs)
    bidx, nblk, sc, err2 = run_select(dw, summ, bs, W.SPECPV_SINK_BLOCKS,
                                      W.SPECPV_WINDOW_BLOCKS, W.SPECPV_TOP_K, reduction)
    assert int(err.item()) == 0 and err2 == 0
    nv = (int(wl.prefix_len[0]) + bs - 1) // bs
    assert nblk[0] == W.SPECPV_BUDGET_TOKENS // bs
    # the selection rule, exactly, on the GPU's scores
    want = oracle.select_blocks(sc[0], nv, W.SPECPV_SINK_BLOCKS, W.SPECPV_WINDOW_BLOCKS,
                                W.SPECPV_TOP_K)
    assert np.array_equal(bidx[0, :nblk[0]], want)
    # summaries and scores of sampled blocks (every selected one and 64 others)
    rng = np.random.default_rng(7)
    sample = sorted(set(want.tolist()) | set(rng.choice(nv, 64, replace=False).tolist()))
    kmax, kmin, nv_o = check_summaries(summ, wl, bs, blocks=sample)
    s64 = oracle.block_scores(wl.q, kmax, kmin, nv_o, reduction, blocks=sample)
    mag = oracle.block_scores(wl.q, kmax, kmin, nv_o, reduction, blocks=sample, magnitude=True)
    tol = score_tol(wl, mag)
    diff = np.abs(sc[0, sample] - s64[0, sample])
    assert np.all(diff <= tol[0, sample]), f"score error {diff.max():.3g}"
