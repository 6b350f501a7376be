"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch each of them: a pin that still passes on a broken oracle pins nothing."""

import numpy as np
import pytest

import oracle.tree_verify as TV
from tests import test_oracle_pins as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, TV.OracleInputError, ValueError, IndexError):
        return True
    return False


def test_no_tree_masking_is_caught(monkeypatch):
    monkeypatch.setattr(TV, "_mask_bit", lambda row, j: True)
    assert _fails(pins.test_p2_per_node_gather, 0)
    assert _fails(pins.test_p1_chain_equals_causal_attention, 1, 9, 17, 4, 2)


def test_tree_part_dropped_is_caught(monkeypatch):
    monkeypatch.setattr(TV, "_mask_bit", lambda row, j: False)
    assert _fails(pins.test_p2_per_node_gather, 1)


def test_prefix_off_by_one_is_caught(monkeypatch):
    orig = TV._visible_prefix_rows
    monkeypatch.setattr(TV, "_visible_prefix_rows",
                        lambda p, *a: orig(max(p - 1, 0), *a))
    assert _fails(pins.test_p1_chain_equals_causal_attention, 3, 5, 40, 8, 1)


def test_self_bit_missing_is_caught(monkeypatch):
    monkeypatch.setattr(TV, "ancestors", _anc_without_self)
    assert _fails(pins.test_p4_specblock_a2_worked_example)


def _anc_without_self(parents, i):
    out = []
    j = i
    while int(parents[j]) >= 0:
        j = int(parents[j])
        out.append(j)
    return out


def test_last_occurrence_argmax_is_caught(monkeypatch):
    def last_argmax(row):
        r = np.asarray(row)
        r = TV.bf16_to_f64(r) if r.dtype == np.uint16 else r.astype(np.float64)
        return int(len(r) - 1 - np.argmax(r[::-1]))
    monkeypatch.setattr(TV, "argmax_lowest", last_argmax)
    monkeypatch.setattr(pins.oracle, "argmax_lowest", last_argmax)
    assert _fails(pins.test_p10_argmax_ties_and_signed_zero)
    assert any(_fails(pins.test_p3_accept_equals_path_enumeration, s) for s in range(40))


@pytest.mark.parametrize("mut", ["child_index", "no_parent_check"])
def test_wrong_acceptance_rule_is_caught(monkeypatch, mut):
    orig = TV.greedy_accept

    def broken(logits, parents, draft):
        amax, alen, path, bonus = orig(logits, parents, draft)
        parents = np.asarray(parents)
        bsz, n = parents.shape
        for b in range(bsz):
            acc, depth = [True] + [False] * (n - 1), [0] * n
            for i in range(1, n):
                p = int(parents[b, i])
                depth[i] = depth[p] + 1
                if mut == "child_index":
                    acc[i] = acc[p] and int(draft[b, i]) == int(amax[b, i])
                else:
                    acc[i] = int(draft[b, i]) == int(amax[b, p])
            best = max(range(n), key=lambda i: (acc[i], depth[i], -i))
            alen[b] = depth[best]
        return amax, alen, path, bonus

    monkeypatch.setattr(TV, "greedy_accept", broken)
    monkeypatch.setattr(pins.oracle, "greedy_accept", broken)
    assert any(_fails(pins.test_p3_accept_equals_path_enumeration, s) for s in range(40))


# ---------------------------------------------------------------------------
# block selection (SpecPV)
# ---------------------------------------------------------------------------

import oracle.block_select as BS  # noqa: E402
from tests import test_oracle_select_pins as spins  # noqa: E402


def test_bound_with_max_key_only_is_caught(monkeypatch):
    # forgetting the min key: negative query coordinates then bound nothing
    monkeypatch.setattr(BS, "ub_score", lambda q, hi, lo: (q * hi).sum(axis=-1))
    assert _fails(spins.test_p14_bound_holds_for_every_token, 0)
    assert _fails(spins.test_p14_scores_equal_corner_brute_force, spins.CASES[0], "mean")


def test_swapped_summaries_are_caught(monkeypatch):
    orig = BS.block_summaries
    swapped = lambda *a: (lambda r: (r[1], r[0], r[2]))(orig(*a))  # noqa: E731
    monkeypatch.setattr(BS, "block_summaries", swapped)
    monkeypatch.setattr(spins.oracle, "block_summaries", swapped)
    assert _fails(spins.test_p13_summary_contains_and_attains_every_coordinate, spins.CASES[0])


def test_summary_including_a_row_past_the_prefix_is_caught(monkeypatch):
    # one row too many in the last block pulls a cache row past the prefix in
    monkeypatch.setattr(BS, "num_blocks", lambda p, bs: -(-(int(p) + 1) // bs))
    assert _fails(spins.test_p13_summary_contains_and_attains_every_coordinate, spins.CASES[1])


@pytest.mark.parametrize("mut", ["first_node", "sum", "min"])
def test_wrong_reduction_is_caught(monkeypatch, mut):
    orig = BS._reduce

    def broken(per_node, reduction):
        if mut == "first_node" and reduction == "last":
            return per_node[0]
        if mut == "sum" and reduction == "mean":
            return per_node.sum(axis=0)
        if mut == "min" and reduction == "max":
            return per_node.min(axis=0)
        return orig(per_node, reduction)
    monkeypatch.setattr(BS, "_reduce", broken)
    red = {"first_node": "last", "sum": "mean", "min": "max"}[mut]
    assert _fails(spins.test_p14_scores_equal_corner_brute_force, spins.CASES[0], red)


def test_wrong_head_to_kv_group_is_caught(monkeypatch):
    orig = BS.block_scores

    def broken(q, kmax, kmin, n_valid, reduction="mean", **kw):
        # heads interleaved over KV groups instead of contiguous groups
        qq = np.asarray(q)
        hq, hkv = qq.shape[2], kmax.shape[1]
        grp = hq // hkv
        perm = [(h % hkv) * grp + h // hkv for h in range(hq)]
        return orig(qq[:, :, perm, :], kmax, kmin, n_valid, reduction, **kw)
    monkeypatch.setattr(BS, "block_scores", broken)
    monkeypatch.setattr(spins.oracle, "block_scores", broken)
    assert _fails(spins.test_p14_scores_equal_corner_brute_force, spins.CASES[3], "mean")


@pytest.mark.parametrize("mut", ["high_id_ties", "window_short", "no_sinks"])
def test_wrong_selection_rule_is_caught(monkeypatch, mut):
    orig = BS.select_blocks

    def broken(scores_row, n_valid, n_sink, n_window, top_k):
        if mut == "window_short":
            return orig(scores_row, n_valid, n_sink, max(n_window - 1, 0), top_k)
        if mut == "no_sinks":
            return orig(scores_row, n_valid, 0, n_window, top_k + n_sink)
        rest = [j for j in range(n_valid) if j >= n_sink and j < n_valid - n_window]
        ranked = sorted(rest, key=lambda j: (-float(scores_row[j]), -j))
        keep = set(range(min(n_sink, n_valid))) | set(range(max(n_valid - n_window, 0), n_valid))
        return np.asarray(sorted(keep | set(ranked[:top_k])), dtype=np.int64)
    monkeypatch.setattr(BS, "select_blocks", broken)
    monkeypatch.setattr(spins.oracle, "select_blocks", broken)
    caught = _fails(spins.test_p17_hand_worked_selection) or any(
        _fails(spins.test_p17_selection_equals_brute_force_counting, s) for s in range(30))
    assert caught


# ---------------------------------------------------------------------------
# SpecPV buffer and rectification
# ---------------------------------------------------------------------------

import oracle.specpv_policy as SPP  # noqa: E402
from tests import test_oracle_specpv_pins as ppins  # noqa: E402


def test_buffer_rule_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(SPP, "needs_rectification", lambda n, size: n >= size)
    assert _fails(ppins.test_buffer_rule_from_the_pages)


@pytest.mark.parametrize("mut", ["no_root", "reversed_chain"])
def test_wrong_rectifying_tree_is_caught(monkeypatch, mut):
    orig = SPP.rectify_tree

    def broken(buffer_tokens, root_token, parents, draft_tokens):
        if mut == "reversed_chain":
            return orig(list(buffer_tokens)[::-1], root_token, parents, draft_tokens)
        # the draft tree hung under the last buffered token, the root dropped
        par, tok = orig(list(buffer_tokens)[:-1] or list(buffer_tokens), buffer_tokens[-1],
                        parents, draft_tokens)
        return par, tok
    monkeypatch.setattr(SPP, "rectify_tree", broken)
    caught = _fails(ppins.test_rectify_tree_hand_worked) or any(
        _fails(ppins.test_rectifying_acceptance_equals_chain_then_tree, s) for s in range(40))
    assert caught


# ---------------------------------------------------------------------------
# stochastic verification (T > 0)
# ---------------------------------------------------------------------------

import inspect  # noqa: E402

import oracle.stochastic as STO  # noqa: E402
from tests import test_oracle_stochastic_pins as spins2  # noqa: E402


def _walk_with(old, new):
    src = inspect.getsource(STO._walk)
    assert old in src
    ns = dict(STO.__dict__)
    exec(src.replace(old, new), ns)
    return ns["_walk"]


@pytest.mark.parametrize("old,new", [
    ("ok = unif * rest < px", "ok = unif < px"),                  # no renormalisation
    ("resid[x] = 0.0", "pass"),                                   # rejected tokens kept
    ("target = unif * rest", "target = unif"),                    # bonus draw unscaled
    ("hits = np.nonzero(cum > target)[0]", "hits = np.array([int(np.argmax(resid))])"),
])
def test_wrong_speculative_sampling_is_caught(monkeypatch, old, new):
    monkeypatch.setattr(STO, "_walk", _walk_with(old, new))
    assert _fails(spins2.test_first_emitted_token_follows_the_target) or \
        _fails(spins2.test_token_after_an_accepted_child_follows_its_row)


def test_wrong_philox_constant_is_caught(monkeypatch):
    monkeypatch.setattr(STO, "_M1", STO._M1 ^ 4)
    assert _fails(spins2.test_philox_matches_numpy, 0)


def _filter_with(old, new):
    src = inspect.getsource(STO.target_probs)
    assert old in src
    ns = dict(STO.__dict__)
    exec(src.replace(old, new), ns)
    return ns["target_probs"]


def _mass_above_with(old, new):
    src = inspect.getsource(STO._mass_above)
    assert old in src
    ns = dict(STO.__dict__)
    exec(src.replace(old, new), ns)
    return ns["_mass_above"]


@pytest.mark.parametrize("old,new", [
    ("keep &= _count_above(l) < top_k", "keep &= _count_above(l) <= top_k"),  # k+1 kept
    ("keep &= mass_above < top_p", "keep &= mass_above <= top_p"),           # boundary kept
    ("q = q / q.sum()", "pass"),                        # top-p on the unrenormalised mass
    ("return f / f.sum()", "return f"),                 # kept mass not renormalised
    ("mass_above = _mass_above(l, q)", "mass_above = _mass_above(l, p)"),  # top-p before top-k
])
def test_wrong_filter_is_caught(monkeypatch, old, new):
    monkeypatch.setattr(STO, "target_probs", _filter_with(old, new))
    caught = _fails(spins2.test_filters_hand_worked) or any(
        _fails(spins2.test_filters_match_brute_force, s) for s in range(30))
    assert caught


@pytest.mark.parametrize("old,new", [
    ("out[order[i:j]] = run          # mass strictly above this value",
     "out[order[i:j]] = run + qs[i:j].sum()"),          # ties counted as above
    ("while j < ls.size and ls[j] == ls[i]:", "while j < ls.size and j == i:"),  # ties split
])
def test_wrong_mass_above_is_caught(monkeypatch, old, new):
    monkeypatch.setattr(STO, "_mass_above", _mass_above_with(old, new))
    caught = _fails(spins2.test_filters_hand_worked) or any(
        _fails(spins2.test_filters_match_brute_force, s) for s in range(30))
    assert caught
