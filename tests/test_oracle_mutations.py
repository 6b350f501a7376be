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
