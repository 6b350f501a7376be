"""Pins for the SpecPV buffer / rectification oracle (SpecPV Sec. 3.3, App. C,
App. D), and CPU parity of the library's host-side policy with it.

The rectifying tree's acceptance is checked against a different
decomposition: re-verify the chain token by token, then, only if the whole
chain survives, accept in the draft tree alone.  All CPU.
"""

import numpy as np
import pytest

import oracle
import oracle.specpv_policy as SP
from oracle import OracleInputError
from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W


def test_buffer_rule_from_the_pages():
    # App. D: buffer size 20; App. C: capacity = one step's tokens + 20
    assert not SP.needs_rectification(0, 20)
    assert not SP.needs_rectification(20, 20)
    assert SP.needs_rectification(21, 20)
    n_step = 60
    for waiting in range(0, 100):
        fits = waiting + n_step <= n_step + 20
        assert SP.needs_rectification(waiting, 20) == (not fits)
    with pytest.raises(OracleInputError):
        SP.needs_rectification(-1, 20)


def test_rectify_tree_hand_worked():
    par, tok = SP.rectify_tree([7, 8, 9], 10, [-1, 0, 0, 1], [99, 11, 12, 13])
    assert par.tolist() == [-1, 0, 1, 2, 3, 3, 4]
    assert tok.tolist() == [7, 8, 9, 10, 11, 12, 13]
    # one buffered token: the chain is just the old bonus above the root
    par, tok = SP.rectify_tree([5], 6, [-1], [0])
    assert par.tolist() == [-1, 0] and tok.tolist() == [5, 6]
    with pytest.raises(OracleInputError):
        SP.rectify_tree([], 1, [-1], [0])
    with pytest.raises(OracleInputError):
        SP.rectify_tree([1], 1, [-1, 1], [0, 0])


def _greedy_next(logits_bits):
    return [oracle.argmax_lowest(r) for r in logits_bits]


@pytest.mark.parametrize("seed", range(40))
def test_rectifying_acceptance_equals_chain_then_tree(seed):
    rng = np.random.default_rng(seed)
    vocab, n_draft = 50, int(rng.integers(1, 12))
    n_buf = int(rng.integers(1, 9))
    parents, planted, draft = W.specpv_draft(seed, 0, n_draft, vocab, 0.7)
    buf = rng.integers(0, vocab, size=n_buf).astype(np.int32)
    root = int(rng.integers(0, vocab))
    par, tok = SP.rectify_tree(buf, root, parents, draft)
    _, _, _, logits = W.specpv_step_inputs(seed, 0, tok, n_buf, planted, vocab=vocab, hq=1,
                                           hkv=1, d=8, p_keep=0.8)
    amax, alen, path, bonus = oracle.greedy_accept(logits, par[None, :], tok[None, :])
    g = _greedy_next(logits[0])
    # chain re-verification, token by token (the root is chain node n_buf)
    chain = list(buf) + [root]
    kept = SP.first_chain_mismatch(chain, g)
    if kept < n_buf:
        assert alen[0] == kept
        assert path[0, :kept + 1].tolist() == list(range(kept + 1))
        assert bonus[0] == g[kept]
    else:
        # the whole chain survived: the draft tree alone decides the rest,
        # with its root's row being chain node n_buf's row
        sub_logits = logits[:, n_buf:, :]
        d_tok = np.asarray(tok[n_buf:])[None, :]
        _, a2, p2, b2 = oracle.greedy_accept(sub_logits, parents[None, :], d_tok)
        assert alen[0] == n_buf + a2[0]
        want = list(range(n_buf)) + [n_buf + int(x) for x in p2[0, :a2[0] + 1]]
        assert path[0, :alen[0] + 1].tolist() == want
        assert bonus[0] == b2[0]


# ---------------------------------------------------------------------------
# the library's host functions against the oracle (no GPU needed)
# ---------------------------------------------------------------------------

def test_library_buffer_rule_matches_oracle():
    for waiting in range(0, 50):
        for size in (0, 1, 20, 45):
            assert binding.specpv_needs_rectification(waiting, size) == \
                SP.needs_rectification(waiting, size)
    with pytest.raises(binding.TVError):
        binding.specpv_needs_rectification(-1, 20)


@pytest.mark.parametrize("seed", range(25))
def test_library_rectify_tree_matches_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    n_draft, n_buf = int(rng.integers(1, 60)), int(rng.integers(1, 90))
    parents, _, draft = W.specpv_draft(seed, 3, n_draft, 1000, 0.5)
    buf = rng.integers(0, 1000, size=n_buf)
    root = int(rng.integers(0, 1000))
    got = binding.specpv_rectify_tree(buf, root, parents, draft)
    want = SP.rectify_tree(buf, root, parents, draft)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_library_rectify_tree_rejects_bad_input():
    with pytest.raises(binding.TVError):
        binding.specpv_rectify_tree([], 1, [-1], [0])
    with pytest.raises(binding.TVError):
        binding.specpv_rectify_tree([1], 1, [-1, 1], [0, 0])
    with pytest.raises(binding.TVError):
        binding.specpv_rectify_tree(np.zeros(200), 1, np.r_[-1, np.zeros(56, int)], np.zeros(57))
