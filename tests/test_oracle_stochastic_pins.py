"""Pins for the stochastic-verification oracle (T > 0).

* Its Philox-4x64-10 equals numpy's Philox bit generator (a library routine);
* speculative sampling over a tree is equivalent to sampling from the target
  (SpecPV Sec. 2): Monte Carlo over many keys, chi-square against the target
  distributions, for the first emitted token and for the token after an
  accepted child;
* as T -> 0 the walk becomes greedy acceptance (the T = 0 oracle);
* duplicate and out-of-range draft tokens.
All CPU.
"""

import numpy as np
import pytest
from scipy import stats

import oracle
import oracle.stochastic as ST
from tree_verification_attention_tv_amd import workloads as W


@pytest.mark.parametrize("seed", range(6))
def test_philox_matches_numpy(seed):
    rng = np.random.default_rng(seed)
    ctr = [int(x) for x in rng.integers(0, 2 ** 62, size=4)]
    key = [int(x) for x in rng.integers(0, 2 ** 63, size=2)]
    bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(8)]
    # numpy steps the counter by one before each 4-word block
    assert ST.philox4x64_10([ctr[0] + 1] + ctr[1:], key) == raw[:4]
    assert ST.philox4x64_10([ctr[0] + 2] + ctr[1:], key) == raw[4:]


def test_uniform_grid():
    us = [ST.uniform((3, 4), 0, 0, i, 0) for i in range(200)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert all(float(u * 2 ** 24).is_integer() for u in us)


def _logits(vals):
    return np.asarray(vals, dtype=np.float32)[None, :, :]


P_ROOT = np.log(np.array([0.45, 0.2, 0.15, 0.12, 0.08]))
P_C1 = np.log(np.array([0.1, 0.6, 0.1, 0.1, 0.1]))
P_C2 = np.log(np.array([0.3, 0.05, 0.05, 0.3, 0.3]))


def _mc(parents, draft, rows, trials, temperature=1.0):
    lg = _logits(rows)
    first, second = [], []
    for t in range(trials):
        a, path, bonus = ST.stochastic_accept(lg, np.array([parents]), np.array([draft]),
                                              temperature, (t, 77), 0)
        toks = [draft[j] for j in path[0, 1:a[0] + 1]] + [int(bonus[0])]
        first.append((toks[0], path[0, 1] if a[0] >= 1 else -1))
        second.append(toks[1] if len(toks) > 1 else None)
    return first, second


def _chi2_ok(observed_tokens, probs):
    counts = np.bincount(observed_tokens, minlength=len(probs))
    exp = probs * len(observed_tokens)
    return stats.chisquare(counts, exp).pvalue


def test_first_emitted_token_follows_the_target():
    # root with three children: tokens 0, 1 and a duplicate 0
    parents, draft = [-1, 0, 0, 0], [9, 0, 1, 0]
    rows = [P_ROOT, P_C1, P_C2, P_C2]
    first, _ = _mc(parents, draft, rows, 8000)
    p = np.exp(P_ROOT)
    assert _chi2_ok(np.array([t for t, _ in first]), p) > 1e-4
    # the duplicate child (node 3) can never be accepted
    assert all(node != 3 for _, node in first)


def test_token_after_an_accepted_child_follows_its_row():
    parents, draft = [-1, 0, 0], [9, 0, 3]
    rows = [P_ROOT, P_C1, P_C2]
    first, second = _mc(parents, draft, rows, 8000)
    after_c1 = np.array([s for (t, node), s in zip(first, second) if node == 1])
    after_c2 = np.array([s for (t, node), s in zip(first, second) if node == 2])
    assert len(after_c1) > 1000 and len(after_c2) > 300
    assert _chi2_ok(after_c1, np.exp(P_C1)) > 1e-4
    assert _chi2_ok(after_c2, np.exp(P_C2)) > 1e-4
    # and the first token is still distributed as the root's row
    assert _chi2_ok(np.array([t for t, _ in first]), np.exp(P_ROOT)) > 1e-4


@pytest.mark.parametrize("seed", range(8))
def test_low_temperature_is_greedy(seed):
    rng = np.random.default_rng(seed)
    wl = W.make_random_case(seed, batch=2, n_nodes=12, hq=2, hkv=1, d=8, prefix_lens=[4, 4],
                            vocab=40, ldt="f32")
    # distinct logits so that the argmax has a margin
    logits = wl.logits + rng.permutation(40).astype(np.float32)[None, None, :] * 0.5
    g = oracle.greedy_accept(logits, wl.parents, wl.draft_tokens)
    s = ST.stochastic_accept(logits, wl.parents, wl.draft_tokens, 1e-3, (seed, 1), 5)
    assert np.array_equal(g[1], s[0]) and np.array_equal(g[2], s[1])
    assert np.array_equal(g[3], s[2])


def test_out_of_range_tokens_are_never_accepted():
    parents, draft = [-1, 0, 0], [0, -3, 5]
    rows = [np.zeros(5), np.zeros(5), np.zeros(5)]
    for t in range(300):
        a, _, bonus = ST.stochastic_accept(_logits(rows), np.array([parents]), np.array([draft]),
                                           1.0, (t, 2), 0)
        assert a[0] == 0 and 0 <= bonus[0] < 5


# ---------------------------------------------------------------------------
# top-k / top-p filters (SpecPV App. D: T 0.6, top-p 0.95, top-k 20; App. E:
# T 0.7 and 1.0, top-k off, top-p 0.9)
# ---------------------------------------------------------------------------

def test_filters_hand_worked():
    # logits 1, 3, 3, 2, -1 at T = 1: p = e^l / sum
    l = np.array([1.0, 3.0, 3.0, 2.0, -1.0], dtype=np.float32)
    e = np.exp(l.astype(np.float64) - 3.0)
    p = e / e.sum()
    # top-1: both tokens tied at the largest logit stay
    assert np.allclose(ST.target_probs(l, 1.0, top_k=1), [0, 0.5, 0.5, 0, 0], rtol=0, atol=1e-15)
    assert np.allclose(ST.target_probs(l, 1.0, top_k=2), [0, 0.5, 0.5, 0, 0], rtol=0, atol=1e-15)
    k3 = np.array([0, e[1], e[2], e[3], 0]) / (e[1] + e[2] + e[3])
    assert np.allclose(ST.target_probs(l, 1.0, top_k=3), k3, rtol=0, atol=1e-15)
    # top-p: the mass strictly above 3 is 0, above 2 is p1 + p2 = 0.793,
    # above 1 is 0.939
    assert abs(p[1] + p[2] - 0.7931691) < 1e-6
    assert np.allclose(ST.target_probs(l, 1.0, top_p=0.5), [0, 0.5, 0.5, 0, 0], atol=1e-15)
    assert np.allclose(ST.target_probs(l, 1.0, top_p=0.79), [0, 0.5, 0.5, 0, 0], atol=1e-15)
    assert np.allclose(ST.target_probs(l, 1.0, top_p=0.9), k3, atol=1e-15)
    full = np.array([e[0], e[1], e[2], e[3], 0]) / (e[:4].sum())
    assert np.allclose(ST.target_probs(l, 1.0, top_p=0.95), full, atol=1e-15)
    # top-k first, then top-p on the renormalised top-k mass: with k = 3 the
    # mass above 2 is 0.793 / 0.939 = 0.845 of the kept mass
    assert np.allclose(ST.target_probs(l, 1.0, top_k=3, top_p=0.84), [0, 0.5, 0.5, 0, 0],
                       atol=1e-15)
    assert np.allclose(ST.target_probs(l, 1.0, top_k=3, top_p=0.85), k3, atol=1e-15)
    # an exact boundary: at a huge temperature four distinct logits have
    # probability 1/4 each exactly, so the mass strictly above the third
    # token is exactly 0.5 and top-p 0.5 must drop it
    l4 = np.array([4.0, 3.0, 2.0, 1.0], dtype=np.float32)
    assert np.array_equal(ST.target_probs(l4, 1e20), [0.25] * 4)
    assert np.array_equal(ST.target_probs(l4, 1e20, top_p=0.5), [0.5, 0.5, 0, 0])
    assert np.allclose(ST.target_probs(l4, 1e20, top_p=0.75), [1 / 3, 1 / 3, 1 / 3, 0],
                       rtol=0, atol=1e-15)
    # filters off
    assert np.allclose(ST.target_probs(l, 1.0, top_k=5), p, atol=1e-15)
    assert np.allclose(ST.target_probs(l, 1.0, top_k=0, top_p=1.0), p, atol=1e-15)
    for bad in ((-1, 1.0), (0, 0.0), (0, 1.5), (0, float("nan"))):
        with pytest.raises(oracle.OracleInputError):
            ST.target_probs(l, 1.0, *bad)


def _brute_filter(l, T, k, top_p):
    """The filter rules by explicit enumeration over pairs of tokens."""
    v = len(l)
    z = [float(x) / T for x in l]
    mx = max(z)
    w = [np.exp(x - mx) for x in z]
    keep = [True] * v
    if k > 0:
        keep = [sum(1 for j in range(v) if l[j] > l[i]) < k for i in range(v)]
    if top_p < 1.0:
        tot = sum(w[i] for i in range(v) if keep[i])
        keep = [keep[i] and sum(w[j] for j in range(v) if keep[j] and l[j] > l[i]) / tot < top_p
                for i in range(v)]
    tot = sum(w[i] for i in range(v) if keep[i])
    return np.array([w[i] / tot if keep[i] else 0.0 for i in range(v)])


@pytest.mark.parametrize("seed", range(30))
def test_filters_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    v = int(rng.integers(1, 13))
    # few distinct values, so that ties are common
    l = rng.integers(-3, 4, size=v).astype(np.float32) * 0.5
    T = float(rng.choice([0.6, 0.7, 1.0]))
    k = int(rng.integers(0, v + 2))
    top_p = float(rng.choice([1.0, 0.95, 0.9, 0.5, 0.2]))
    got = ST.target_probs(l, T, top_k=k, top_p=top_p)
    want = _brute_filter(l, T, k, top_p)
    assert np.allclose(got, want, rtol=0, atol=1e-12), (l, T, k, top_p)


@pytest.mark.parametrize("seed", range(6))
def test_top1_with_a_unique_max_is_greedy(seed):
    # with a unique largest logit, top-k = 1 makes every row a point mass:
    # the walk accepts exactly the greedy path and the bonus is the argmax
    rng = np.random.default_rng(100 + seed)
    wl = W.make_random_case(seed, batch=2, n_nodes=12, hq=2, hkv=1, d=8, prefix_lens=[4, 4],
                            vocab=40, ldt="f32")
    logits = wl.logits + rng.permutation(40).astype(np.float32)[None, None, :] * 0.5
    g = oracle.greedy_accept(logits, wl.parents, wl.draft_tokens)
    for T in (0.6, 1.0):
        s = ST.stochastic_accept(logits, wl.parents, wl.draft_tokens, T, (seed, 3), 1, top_k=1)
        assert np.array_equal(g[1], s[0]) and np.array_equal(g[2], s[1])
        assert np.array_equal(g[3], s[2])
        # a tiny nucleus keeps only the most likely token too
        s = ST.stochastic_accept(logits, wl.parents, wl.draft_tokens, T, (seed, 4), 1,
                                 top_p=1e-6)
        assert np.array_equal(g[1], s[0]) and np.array_equal(g[3], s[2])


def test_filtered_first_token_follows_the_filtered_target():
    # speculative sampling stays exact under filtering: the first emitted
    # token is distributed as the filtered root distribution
    parents, draft = [-1, 0, 0, 0], [9, 0, 1, 3]
    rows = [P_ROOT, P_C1, P_C2, P_C2]
    lg = _logits(rows)
    for k, top_p in ((3, 1.0), (0, 0.7), (4, 0.9)):
        firsts = []
        for t in range(6000):
            a, path, bonus = ST.stochastic_accept(lg, np.array([parents]), np.array([draft]),
                                                  1.0, (t, 91), 0, top_k=k, top_p=top_p)
            firsts.append(draft[path[0, 1]] if a[0] >= 1 else int(bonus[0]))
        target = ST.target_probs(P_ROOT.astype(np.float32), 1.0, k, top_p)
        assert set(np.nonzero(np.bincount(firsts, minlength=5))[0]) <= \
            set(np.nonzero(target)[0])
        nz = target > 0
        counts = np.bincount(firsts, minlength=5)[nz]
        assert stats.chisquare(counts, target[nz] * len(firsts)).pvalue > 1e-4, (k, top_p)
