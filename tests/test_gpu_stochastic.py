"""Stochastic verification (T > 0) on the GPU against the fp64 oracle.

Both sides draw the same Philox-4x64-10 uniforms, so every accept/reject
decision and the bonus draw are fixed numbers; they can differ only where a
uniform falls within rounding distance of its threshold (the GPU computes
p in fp32).  The comparison therefore replays the oracle with the GPU's
choice at decisions closer than TOL to their threshold and requires:

* identical accepted length and path;
* the bonus equal to the oracle's, or, if the draw fell within TOL of a CDF
  boundary, the GPU's token on the other side of that boundary.

TOL = 1e-4 (absolute, on the probability scale): fp32 softmax sums over
128256 terms and the chunked prefix sums of the bonus draw are off by at most
a few 1e-6 in these inputs.

A Monte Carlo check over 3000 keys also compares the GPU's first emitted
token with the target distribution directly (chi-square), independent of the
oracle.

The filtered call (top-k / top-p, SpecPV App. D and E settings) is compared
the same way against the oracle's filtered distributions, with the filters
off it must equal the plain call bit for bit, and a Monte Carlo check
confirms that no filtered-out token is ever emitted.
"""

import sys

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import oracle.stochastic as ST
from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W

from .gpu_util import dev_bf16, dev_i32

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_run(parents, draft, logits, temperature, seed, step, dtype="bf16", stride_pad=0,
            filt=None):
    if dtype == "bf16":
        lg = dev_bf16(logits)
    else:
        lg = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    if stride_pad:
        b, n, v = lg.shape
        big = torch.zeros((b, n, v + stride_pad), dtype=lg.dtype, device="cuda")
        big[:, :, :v] = lg
        lg = big[:, :, :v]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if filt is None:
        alen, path, bonus = binding.stochastic_accept(lg, dev_i32(parents), dev_i32(draft),
                                                      temperature, seed=seed, step=step,
                                                      dev_err=err)
    else:
        alen, path, bonus = binding.stochastic_accept_filtered(
            lg, dev_i32(parents), dev_i32(draft), temperature, top_k=filt[0], top_p=filt[1],
            seed=seed, step=step, dev_err=err)
    torch.cuda.synchronize()
    return alen.cpu().numpy(), path.cpu().numpy(), bonus.cpu().numpy(), int(err.item())


def check_against_oracle(parents, draft, logits, temperature, seed, step, got, filt=(0, 1.0)):
    alen, path, bonus = got[:3]
    bsz = parents.shape[0]

    def decide(b, event, ok):
        _, u, c, unif, rest, px = event
        if abs(unif * rest - px) > TOL:
            return ok
        # near the threshold: follow the GPU (accepted c iff c is on its path after u)
        gp = list(path[b, :alen[b] + 1])
        return u in gp and gp.index(u) + 1 < len(gp) and gp[gp.index(u) + 1] == c

    a, p, y, events = ST.stochastic_accept(logits, parents, draft, temperature, seed, step,
                                           return_events=True, decide=decide, top_k=filt[0],
                                           top_p=filt[1])
    assert np.array_equal(alen, a), f"accept_len {alen} vs oracle {a}"
    assert np.array_equal(path, p)
    for b in range(bsz):
        if bonus[b] == y[b]:
            continue
        # only a draw within TOL of the boundary between the two tokens may differ
        _, u, _, unif, rest, target = events[b][-1]
        probs = ST.target_probs(logits[b, u], temperature, filt[0], filt[1])
        removed = {int(draft[b, c]) for (kind, uu, c, *_r) in events[b][:-1]
                   if kind == "child" and uu == u and 0 <= int(draft[b, c]) < probs.shape[0]}
        resid = probs.copy()
        for x in removed:
            resid[x] = 0.0
        cum = np.cumsum(resid)
        g = int(bonus[b])
        assert resid[g] > 0.0, f"seq {b}: bonus {g} is not an eligible token"
        lo_edge = cum[g] - resid[g]
        assert lo_edge - TOL <= target <= cum[g] + TOL, (
            f"seq {b}: bonus {g} (cdf {lo_edge:.6g}..{cum[g]:.6g}) vs oracle {y[b]}, "
            f"target {target:.6g}")


CASES = [
    # seed, batch, n_nodes, vocab, dtype, temperature, tree
    (1, 4, 60, 128256, "bf16", 0.6, "eagle"),
    (2, 4, 60, 128256, "bf16", 1.0, "eagle"),
    (3, 3, 96, 32000, "bf16", 0.7, "random"),
    (4, 2, 17, 1000, "f32", 0.7, "chain"),
    (5, 16, 32, 50000, "bf16", 1.0, "eagle"),
    (6, 1, 1, 128256, "bf16", 1.0, "eagle"),
    (7, 2, 256, 4099, "f32", 0.6, "random"),
]


@pytest.mark.parametrize("step", [0, 7])
@pytest.mark.parametrize("case", CASES)
def test_stochastic_matches_oracle(case, step):
    seed, batch, n, vocab, dtype, temp, tree = case
    _say(f"[stochastic] seed {seed} batch {batch} N {n} V {vocab} {dtype} T {temp} {tree} "
         f"step {step}")
    parents, draft, logits = W.make_sampling_case(seed, batch=batch, n_nodes=n, vocab=vocab,
                                                  dtype=dtype, tree=tree)
    got = gpu_run(parents, draft, logits, temp, (seed, 99), step, dtype)
    assert got[3] == 0
    check_against_oracle(parents, draft, logits, temp, (seed, 99), step, got)


def test_strided_rows_and_out_of_range_tokens():
    _say("[stochastic] strided rows, tokens out of range, repeated siblings")
    parents, draft, logits = W.make_sampling_case(11, batch=3, n_nodes=40, vocab=5003,
                                                  dtype="bf16", tree="random")
    draft[0, 5] = -1
    draft[1, 7] = 5003
    # repeated sibling tokens
    kids = [j for j in range(1, 40) if parents[2, j] == 0]
    for j in kids[1:]:
        draft[2, j] = draft[2, kids[0]]
    got = gpu_run(parents, draft, logits, 0.7, (5, 6), 3, "bf16", stride_pad=13)
    assert got[3] == 0
    check_against_oracle(parents, draft, logits, 0.7, (5, 6), 3, got)


def test_malformed_tree_falls_back_to_the_root():
    _say("[stochastic] malformed tree")
    parents, draft, logits = W.make_sampling_case(12, batch=2, n_nodes=10, vocab=777,
                                                  dtype="f32", tree="chain")
    parents[1, 4] = 7
    alen, path, bonus, err = gpu_run(parents, draft, logits, 1.0, (1, 1), 0, "f32")
    assert err & binding.DERR_BAD_PARENT
    assert alen[1] == 0 and path[1, 0] == 0 and np.all(path[1, 1:] == -1)
    # the root-only walk draws the bonus from the root's row
    root_only = ST.stochastic_accept(logits[1:2, :1], parents[1:2, :1], draft[1:2, :1], 1.0,
                                     (1, 1), 0, return_events=True)
    tgt = root_only[3][0][-1][-1]
    cum = np.cumsum(ST.target_probs(logits[1, 0], 1.0))
    g = int(bonus[1])
    assert cum[g] - (cum[g] - (cum[g - 1] if g else 0.0)) - TOL <= tgt <= cum[g] + TOL


def test_host_checks():
    parents, draft, logits = W.make_sampling_case(13, batch=1, n_nodes=4, vocab=64, dtype="f32")
    for bad_t in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(binding.TVError):
            gpu_run(parents, draft, logits, bad_t, (0, 0), 0, "f32")


def test_first_token_is_distributed_as_the_target():
    # independent of the oracle: 3000 keys, chi-square against softmax(l/T)
    _say("[stochastic] Monte Carlo of the first emitted token")
    vocab, temp = 8, 0.8
    rng = np.random.default_rng(21)
    rows = rng.normal(0, 1.5, size=(4, vocab)).astype(np.float32)
    parents = np.array([[-1, 0, 0, 0]], dtype=np.int32)
    draft = np.array([[0, 3, 5, 3]], dtype=np.int32)
    lg = torch.from_numpy(rows.copy()).cuda().view(1, 4, vocab)
    par_d, dr_d = dev_i32(parents), dev_i32(draft)
    ws = torch.empty(binding.stochastic_accept_workspace_size(1, 4, vocab), dtype=torch.uint8,
                     device="cuda")
    outs = (torch.empty(1, dtype=torch.int32, device="cuda"),
            torch.empty((1, 4), dtype=torch.int32, device="cuda"),
            torch.empty(1, dtype=torch.int32, device="cuda"))
    firsts = []
    trials = 3000
    res = torch.empty((trials, 3), dtype=torch.int32, device="cuda")
    for k in range(trials):
        binding.stochastic_accept(lg, par_d, dr_d, temp, seed=(k, 4242), step=0, workspace=ws,
                                  outputs=outs)
        res[k, 0] = outs[0][0]
        res[k, 1] = outs[1][0, 1]
        res[k, 2] = outs[2][0]
    r = res.cpu().numpy()
    for alen, node1, bonus in r:
        firsts.append(int(draft[0, node1]) if alen >= 1 else int(bonus))
    z = rows[0].astype(np.float64) / temp
    p = np.exp(z - z.max())
    p /= p.sum()
    counts = np.bincount(firsts, minlength=vocab)
    assert stats.chisquare(counts, p * trials).pvalue > 1e-4
    # the repeated sibling (node 3) is never accepted
    assert not np.any((r[:, 0] >= 1) & (r[:, 1] == 3))


# top-k / top-p: the pages' settings (SpecPV App. D: T 0.6, top-k 20, top-p
# 0.95; App. E: T 0.7 / 1.0, top-p 0.9) and edge values
FILTER_CASES = [
    # seed, batch, n_nodes, vocab, dtype, temperature, tree, top_k, top_p, logit lean
    # (lean (3, 7): top-k 20 keeps 10-21 tokens, top-p 0.9 about 55000 of 128256;
    # lean (9, 16): rows peaked on one token)
    (21, 4, 60, 128256, "bf16", 0.6, "eagle", 20, 0.95, (3.0, 7.0)),
    (22, 4, 60, 128256, "bf16", 0.7, "eagle", 0, 0.9, (3.0, 7.0)),
    (23, 2, 60, 128256, "bf16", 1.0, "eagle", 0, 0.9, (9.0, 16.0)),
    (24, 3, 96, 32000, "bf16", 0.7, "random", 50, 1.0, (3.0, 7.0)),
    (25, 2, 17, 1000, "f32", 0.7, "chain", 5, 0.8, (1.0, 3.0)),
    (26, 2, 64, 4099, "f32", 0.6, "random", 1, 1.0, (9.0, 16.0)),
    (27, 2, 33, 5003, "bf16", 1.0, "random", 3000, 0.5, (1.0, 3.0)),
    (28, 1, 1, 128256, "bf16", 0.6, "eagle", 20, 0.95, (3.0, 7.0)),
]


@pytest.mark.parametrize("case", FILTER_CASES, ids=lambda c: f"seed{c[0]}")
def test_filtered_sampling_matches_oracle(case):
    # The GPU's top-p masses are fp32 exponentials in 2^-40 fixed point: a
    # tail token whose larger tokens hold within ~1e-6 of top_p may be kept
    # on one side only.  Such tokens carry ~1e-6 of probability, so they
    # change the renormalised probabilities by far less than TOL and are
    # drawn with probability ~1e-6; the comparison below is unaffected.
    seed, batch, n, vocab, dtype, temp, tree, top_k, top_p, lean = case
    _say(f"[stochastic filtered] seed {seed} batch {batch} N {n} V {vocab} {dtype} T {temp} "
         f"top-k {top_k} top-p {top_p}")
    parents, draft, logits = W.make_sampling_case(seed, batch=batch, n_nodes=n, vocab=vocab,
                                                  dtype=dtype, tree=tree, lean=lean)
    for step in (0, 3):
        got = gpu_run(parents, draft, logits, temp, (seed, 5), step, dtype, filt=(top_k, top_p))
        assert got[3] == 0
        check_against_oracle(parents, draft, logits, temp, (seed, 5), step, got,
                             filt=(top_k, top_p))


def test_filters_off_equal_the_unfiltered_call():
    _say("[stochastic filtered] top-k 0 / >= V and top-p 1 equal tv_stochastic_accept")
    parents, draft, logits = W.make_sampling_case(3, batch=3, n_nodes=40, vocab=5000,
                                                  dtype="bf16", tree="random")
    base = gpu_run(parents, draft, logits, 0.8, (9, 9), 2, "bf16")
    for filt in ((0, 1.0), (5000, 1.0), (9999, 1.0)):
        got = gpu_run(parents, draft, logits, 0.8, (9, 9), 2, "bf16", filt=filt)
        for x, y in zip(got[:3], base[:3]):
            assert np.array_equal(x, y), filt


def test_filtered_first_token_is_distributed_as_the_filtered_target():
    # independent of the walk oracle: chi-square of the first emitted token
    _say("[stochastic filtered] Monte Carlo of the first emitted token")
    vocab, temp, top_k, top_p = 12, 0.8, 6, 0.8
    rng = np.random.default_rng(31)
    rows = rng.normal(0, 1.5, size=(4, vocab)).astype(np.float32)
    parents = np.array([[-1, 0, 0, 0]], dtype=np.int32)
    # drafts: a kept token, a filtered-out token, a repeated one
    target = ST.target_probs(rows[0], temp, top_k, top_p)
    kept, dropped = np.nonzero(target > 0)[0], np.nonzero(target == 0)[0]
    draft = np.array([[0, kept[0], dropped[0], kept[0]]], dtype=np.int32)
    lg = torch.from_numpy(rows.copy()).cuda().view(1, 4, vocab)
    par_d, dr_d = dev_i32(parents), dev_i32(draft)
    ws = torch.empty(binding.stochastic_accept_workspace_size(1, 4, vocab), dtype=torch.uint8,
                     device="cuda")
    outs = (torch.empty(1, dtype=torch.int32, device="cuda"),
            torch.empty((1, 4), dtype=torch.int32, device="cuda"),
            torch.empty(1, dtype=torch.int32, device="cuda"))
    trials = 3000
    res = torch.empty((trials, 3), dtype=torch.int32, device="cuda")
    for k in range(trials):
        binding.stochastic_accept_filtered(lg, par_d, dr_d, temp, top_k=top_k, top_p=top_p,
                                           seed=(k, 777), step=0, workspace=ws, outputs=outs)
        res[k, 0] = outs[0][0]
        res[k, 1] = outs[1][0, 1]
        res[k, 2] = outs[2][0]
    r = res.cpu().numpy()
    firsts = np.array([int(draft[0, node1]) if alen >= 1 else int(bonus) for alen, node1, bonus in r])
    # never a filtered-out token, never the filtered-out or repeated child
    assert np.all(target[firsts] > 0)
    assert not np.any((r[:, 0] >= 1) & ((r[:, 1] == 2) | (r[:, 1] == 3)))
    counts = np.bincount(firsts, minlength=vocab)[kept]
    assert stats.chisquare(counts, target[kept] * trials).pvalue > 1e-4


def test_filtered_sampling_unaligned_rows():
    # a row stride that is not a whole number of 16-byte vectors: the
    # element-wise load paths of every kernel, top-k through the slices
    _say("[stochastic filtered] strided rows (element-wise loads)")
    parents, draft, logits = W.make_sampling_case(41, batch=2, n_nodes=24, vocab=9001,
                                                  dtype="bf16", tree="random", lean=(3.0, 7.0))
    for filt in ((20, 0.95), (0, 0.9), (1, 1.0)):
        got = gpu_run(parents, draft, logits, 0.7, (41, 8), 1, "bf16", stride_pad=13, filt=filt)
        assert got[3] == 0
        check_against_oracle(parents, draft, logits, 0.7, (41, 8), 1, got, filt=filt)


# The threshold search takes two routes: top-k of at most 32 through per-slice
# candidate lists (falling back to a whole-row search when a slice has more
# than 256 candidates), everything else spread over 8192-element slices with
# one launch per key digit (bf16: two digits, fp32: three).  These cases reach
# the routes the cases above do not.
SPREAD_CASES = [
    # seed, batch, n_nodes, vocab, dtype, temperature, top_k, top_p, lean
    (51, 2, 24, 70000, "f32", 0.7, 0, 0.9, (3.0, 7.0)),     # fp32 top-p: three mass digits
    (52, 2, 16, 70000, "f32", 0.8, 200, 0.95, (3.0, 7.0)),  # fp32 count digits, then mass
    (53, 1, 9, 600000, "bf16", 0.6, 20, 0.95, (3.0, 7.0)),  # 74 slices: top-k 20 spread
    (54, 2, 12, 9001, "bf16", 1.0, 33, 1.0, (1.0, 3.0)),    # top-k just past the list route
]


@pytest.mark.parametrize("case", SPREAD_CASES, ids=lambda c: f"seed{c[0]}")
def test_filter_routes_match_oracle(case):
    seed, batch, n, vocab, dtype, temp, top_k, top_p, lean = case
    _say(f"[stochastic filtered] route case seed {seed} V {vocab} {dtype} top-k {top_k} "
         f"top-p {top_p}")
    parents, draft, logits = W.make_sampling_case(seed, batch=batch, n_nodes=n, vocab=vocab,
                                                  dtype=dtype, tree="random", lean=lean)
    got = gpu_run(parents, draft, logits, temp, (seed, 1), 0, dtype, filt=(top_k, top_p))
    assert got[3] == 0
    check_against_oracle(parents, draft, logits, temp, (seed, 1), 0, got, filt=(top_k, top_p))


def test_filter_heavy_ties_fall_back_to_the_row_search():
    # rows whose values repeat so often that a slice keeps more than 256
    # candidates at or above its bound: the per-row workgroup searches the row
    _say("[stochastic filtered] heavy ties (candidate lists overflow)")
    rng = np.random.default_rng(61)
    batch, n, vocab = 2, 10, 20000
    parents = np.stack([W.random_tree(rng, n) for _ in range(batch)]).astype(np.int32)
    draft = rng.integers(0, vocab, size=(batch, n)).astype(np.int32)
    # four distinct values, the top one shared by thousands of tokens
    vals = np.array([2.0, 1.0, 0.5, -1.0], dtype=np.float32)
    x = vals[rng.integers(0, 4, size=(batch * n, vocab))]
    logits = W.f32_to_bf16_bits(x).reshape(batch, n, vocab)
    for filt in ((20, 1.0), (20, 0.95), (5, 0.5)):
        got = gpu_run(parents, draft, logits, 0.9, (61, 2), 0, "bf16", filt=filt)
        assert got[3] == 0
        check_against_oracle(parents, draft, logits, 0.9, (61, 2), 0, got, filt=filt)


def test_masked_vocabulary_tail():
    # a padded vocabulary: the last 1000 logits of every row are -inf (never
    # kept, never drawn, never counted as mass) on every route
    _say("[stochastic] -inf logits in every row")
    parents, draft, logits = W.make_sampling_case(71, batch=2, n_nodes=20, vocab=20000,
                                                  dtype="f32", tree="random", lean=(3.0, 7.0))
    masked = logits.copy()
    masked[:, :, -1000:] = -np.inf
    # the oracle takes finite logits only: -1e4 has the same order and, at
    # this temperature, an fp64 probability of exactly 0
    finite = logits.copy()
    finite[:, :, -1000:] = -1e4
    for filt in (None, (20, 0.95), (0, 0.9), (500, 1.0)):
        got = gpu_run(parents, draft, masked, 0.8, (71, 3), 0, "f32", filt=filt)
        assert got[3] == 0
        assert np.all(got[2] < 19000), "a masked token was drawn"
        check_against_oracle(parents, draft, finite, 0.8, (71, 3), 0, got,
                             filt=(0, 1.0) if filt is None else filt)
