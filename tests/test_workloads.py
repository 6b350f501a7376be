"""Seeded generators: determinism, shapes and the stated properties of each
workload (parity unpinned: the distributions are synthetic)."""

import numpy as np
import pytest

import oracle
from tree_verification_attention_tv_amd import workloads as W


@pytest.fixture(scope="module")
def small_workloads():
    return {n: W.make_workload(n) for n in ("tiny", "8b_layer", "specblock_tree")}


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 1.0 + 2 ** -8], dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits)
    # exact values stay, halfway cases go to even mantissa
    assert back[0] == 1.0 and back[3] == -2.5
    assert back[1] == 1.0                  # 1 + 2^-8 is halfway -> even (1.0)
    assert back[2] == 1.015625             # 1 + 3*2^-8 halfway -> even (1 + 2^-6)
    assert abs(back[4] - 3.0e-3) / 3.0e-3 < 2 ** -8


def test_deterministic(small_workloads):
    again = W.make_workload("8b_layer")
    a = small_workloads["8b_layer"]
    for f in ("parents", "draft_tokens", "q", "k_tree", "v_tree", "k_cache", "logits"):
        assert np.array_equal(getattr(a, f), getattr(again, f))


def test_tiny_properties(small_workloads):
    wl = small_workloads["tiny"]
    assert wl.parents.shape == (1, 8)
    _, depth = oracle.build_mask(wl.parents)
    assert depth.max() == 3
    kids = np.bincount(wl.parents[0, 1:], minlength=8)
    assert np.all(kids[kids > 0] <= 3)
    assert wl.logits.dtype == np.float32 and wl.logits.shape == (1, 8, 1024)
    assert wl.q.shape == (1, 8, 4, 64) and wl.k_cache.shape[1:] == (1, 320, 64)


def test_8b_tree(small_workloads):
    wl = small_workloads["8b_layer"]
    assert wl.parents.shape == (1, 60)
    _, depth = oracle.build_mask(wl.parents)
    assert depth.max() == 8
    # breadth-first labels: depth never decreases with the index
    assert np.all(np.diff(depth[0]) >= 0)
    assert wl.q.shape == (1, 60, 32, 128) and wl.k_cache.shape == (1, 8, 1088, 128)


def test_specblock_tree(small_workloads):
    wl = small_workloads["specblock_tree"]
    n = wl.n_nodes
    assert 2 <= n <= 96
    oracle.build_mask(wl.parents)    # well formed
    kids = np.bincount(wl.parents[0, 1:], minlength=n)
    assert set(np.unique(kids)) <= {0, 2, 4, 6, 8, 10, 12, 14, 16, 18, 20}


def test_planted_targets_are_the_argmax(small_workloads):
    for wl in small_workloads.values():
        flat = wl.logits.reshape(-1, wl.vocab)
        planted = wl.planted_target.reshape(-1)
        for r in range(0, flat.shape[0], 7):
            assert oracle.argmax_lowest(flat[r]) == planted[r]


def test_cache_poisoned_past_prefix(small_workloads):
    wl = small_workloads["8b_layer"]
    assert np.all(wl.k_cache[:, :, 1000:] == W.BF16_NAN)
    assert np.all(wl.v_cache[:, :, 1000:] == W.BF16_NAN)
    assert not np.any(wl.k_cache[:, :, :1000] == W.BF16_NAN)


def test_match_rate_near_stated_probability(small_workloads):
    wl = small_workloads["8b_layer"]
    par = wl.parents[0]
    hits = [wl.draft_tokens[0, j] == wl.planted_target[0, par[j]] for j in range(1, 60)]
    assert 0.5 < np.mean(hits) < 0.95


def test_specpv_block_list_layout():
    rng = np.random.default_rng(5)
    blocks = W.specpv_block_list(rng, 60000, 64, 2, 16, 46)
    assert blocks.shape == (64,)
    assert list(blocks[:2]) == [0, 1]
    assert list(blocks[-16:]) == list(range(922, 938))
    assert len(set(blocks.tolist())) == 64 and np.all(np.diff(blocks) > 0)
    # the last block holds 60000 - 937*64 = 32 tokens: 4064 visible tokens
    visible = sum(min(64, 60000 - b * 64) for b in blocks)
    assert visible == 4064
