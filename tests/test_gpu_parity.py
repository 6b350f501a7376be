"""Parity of the HIP path with the fp64 oracle on seeded inputs.

Bit-exact: masks, depths, argmax, accepted length / path / bonus, committed
cache rows.  bf16 attention output: |gpu - oracle| <= 2e-2 + 1e-2 |oracle|
elementwise, plus max_abs_err / max|oracle| <= 1e-2.
"""

import math
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

NAMED = ["tiny", "8b_layer", "specblock_tree", "batched", "long_context"]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def workloads():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = DevWorkload(W.make_workload(name))
        return cache[name]
    return get


def mask_np(mask_t):
    return mask_t.cpu().numpy().view(np.uint32)


# ---------------------------------------------------------------------------
# a1 mask
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", NAMED)
def test_mask_named(workloads, name):
    _say(f"[mask] {name}")
    dw = workloads(name)
    mask, depth = binding.build_tree_mask(dw.parents)
    ref_mask, ref_depth = oracle.build_mask(dw.wl.parents)
    assert np.array_equal(mask_np(mask), ref_mask)
    assert np.array_equal(depth.cpu().numpy(), ref_depth)


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 64, 65, 100, 255, 256])
def test_mask_random_sizes(n):
    _say(f"[mask] random n={n}")
    rng = np.random.default_rng(n)
    parents = np.stack([W.random_tree(rng, n) for _ in range(3)] + [W.chain_tree(n)])
    mask, depth = binding.build_tree_mask(dev_i32(parents))
    ref_mask, ref_depth = oracle.build_mask(parents)
    assert np.array_equal(mask_np(mask), ref_mask)
    assert np.array_equal(depth.cpu().numpy(), ref_depth)


def test_mask_malformed_fallback():
    _say("[mask] malformed parents")
    parents = np.array([[-1, 0, 1, 2], [-1, 0, 3, 1], [0, 0, 1, 2]], dtype=np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    mask, depth = binding.build_tree_mask(dev_i32(parents), dev_err=err)
    m = mask_np(mask)
    ref, _ = oracle.build_mask(parents[:1])
    assert np.array_equal(m[0], ref[0])
    for b in (1, 2):   # self-only rows, depth 0
        assert list(m[b, :, 0]) == [1, 2, 4, 8]
        assert np.all(depth[b].cpu().numpy() == 0)
    assert int(err.item()) == binding.DERR_BAD_PARENT


# ---------------------------------------------------------------------------
# a2-a4 attention
# ---------------------------------------------------------------------------

def _run_attention_case(dw, partial=False, label="", **kw):
    wl = dw.wl
    mask, _ = binding.build_tree_mask(dw.parents)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = dw.attention(mask, partial=partial, want_lse=True, dev_err=err, **kw)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle_attention(wl, partial=partial,
                                      scale=kw.get("scale") or None)
    e, rel = check_attention_close(out, ref_o, label)
    lse_err = np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse).max()
    assert lse_err < 2e-3, f"{label}: lse err {lse_err}"
    assert int(err.item()) == 0
    return out, e, rel


@pytest.mark.parametrize("name,partial", [(n, False) for n in NAMED] + [("long_context", True)])
def test_attention_named(workloads, name, partial):
    _say(f"[attention] {name} partial={partial}")
    dw = workloads(name)
    out, e, rel = _run_attention_case(dw, partial=partial, label=name)
    _say(f"  max_abs_err={e:.3g} rel={rel:.3g}")


ATTN_CASES = [
    # seed, batch, n, hq, hkv, d, prefix lens, block_size, blocks/seq, tree
    (1, 1, 8, 4, 1, 64, [256], 0, None, "random"),
    (2, 1, 60, 32, 8, 128, [1000], 0, None, "random"),
    (3, 2, 17, 8, 2, 128, [95, 33], 0, None, "random"),      # ragged tail, tiny prefix
    (4, 3, 5, 6, 3, 64, [0, 1, 64], 0, None, "random"),       # empty prefix, G=2
    (5, 1, 100, 32, 8, 128, [700], 0, None, "random"),        # 400 rows -> 2 row groups
    (6, 1, 256, 16, 4, 128, [129], 0, None, "random"),        # 1024 rows -> 4 row groups
    (7, 1, 33, 32, 8, 128, [1500], 0, None, "chain"),
    (8, 2, 12, 32, 8, 128, [900, 450], 16, 20, "random"),     # partial, bs 16
    (9, 1, 9, 8, 1, 64, [300], 64, None, "random"),           # partial, every block
    (10, 4, 32, 32, 8, 128, [1000, 1600, 1203, 1377], 0, None, "random"),
    (11, 1, 3, 2, 2, 128, [5000], 0, None, "random"),
    (12, 1, 47, 4, 4, 64, [777], 48, 7, "random"),            # bs not a multiple of 32
    # 280 and 332 rows (a second row group of 24 and 76 rows) with a grid
    # filled by the prefix splits, full and partial mode
    (13, 1, 70, 8, 2, 128, [9000], 0, None, "random"),
    (14, 1, 83, 32, 8, 128, [6000], 32, 160, "random"),       # partial, 5120 listed slots
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[f"case{c[0]}" for c in ATTN_CASES])
def test_attention_random(case):
    seed, bsz, n, hq, hkv, d, plens, bs, bps, tree = case
    _say(f"[attention] random case {case}")
    wl = W.make_random_case(seed, batch=bsz, n_nodes=n, hq=hq, hkv=hkv, d=d, prefix_lens=plens,
                            block_size=bs, blocks_per_seq=bps, tree=tree)
    dw = DevWorkload(wl)
    _run_attention_case(dw, partial=bool(bs), label=f"case{seed}")


@pytest.mark.parametrize("placement", [binding.TREE_IN_LAST_SPLIT, binding.TREE_OWN_WORKGROUP])
@pytest.mark.parametrize("case", [c for c in ATTN_CASES if c[0] in (2, 3, 4, 8, 10, 12, 13)],
                         ids=lambda c: f"case{c[0]}")
def test_attention_tree_placements(case, placement):
    seed, bsz, n, hq, hkv, d, plens, bs, bps, tree = case
    _say(f"[attention] tree placement {placement} case {seed}")
    wl = W.make_random_case(seed, batch=bsz, n_nodes=n, hq=hq, hkv=hkv, d=d, prefix_lens=plens,
                            block_size=bs, blocks_per_seq=bps, tree=tree)
    _run_attention_case(DevWorkload(wl), partial=bool(bs), label=f"case{seed}-p{placement}",
                        tree_placement=placement)


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 7, 31])
def test_attention_split_counts(workloads, splits):
    _say(f"[attention] 8b_layer splits={splits}")
    _run_attention_case(workloads("8b_layer"), label=f"splits{splits}", num_splits=splits)


@pytest.mark.parametrize("splits", [1, 3, 6, 12])
def test_attention_split_counts_d64(splits):
    """Head dim 64 with 1..13 partials per row: both merge forms (one lane
    per output chunk up to 8 partials, one wave per row above) at D = 64."""
    _say(f"[attention] d64 splits={splits}")
    wl = W.make_random_case(41, batch=2, n_nodes=20, hq=8, hkv=2, d=64, prefix_lens=[900, 517])
    _run_attention_case(DevWorkload(wl), label=f"d64-splits{splits}", num_splits=splits)


@pytest.mark.parametrize("d,splits", [(128, 40), (128, 75), (64, 75)])
def test_attention_many_partials(d, splits):
    """Rows with more partials than the merge keeps in flight per lane group
    (8 per group): 38 splits of 64 tokens, and 75 splits of 32 tokens (two
    or three rounds of loads at D = 128, two at D = 64)."""
    _say(f"[attention] d{d} splits={splits}")
    wl = W.make_random_case(43, batch=2, n_nodes=12, hq=8, hkv=2, d=d, prefix_lens=[2400, 2263])
    _run_attention_case(DevWorkload(wl), label=f"d{d}-splits{splits}", num_splits=splits)


def test_attention_explicit_scale(workloads):
    _say("[attention] explicit scale")
    _run_attention_case(workloads("tiny"), label="scale", scale=0.3)


def test_attention_deterministic(workloads):
    _say("[attention] determinism")
    dw = workloads("8b_layer")
    mask, _ = binding.build_tree_mask(dw.parents)
    a = dw.attention(mask)
    b = dw.attention(mask)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_bad_block_is_skipped():
    _say("[attention] bad block ids")
    wl = W.make_random_case(31, batch=1, n_nodes=6, hq=8, hkv=2, d=128, prefix_lens=[200],
                            block_size=32, blocks_per_seq=4)
    good = wl.block_idx.copy()
    dw = DevWorkload(wl)
    bad = good.copy()
    bad = np.concatenate([bad, np.array([[-3, 50]], dtype=np.int32)], axis=1)   # both invalid
    dw.block_idx = dev_i32(bad)
    dw.n_blocks = dev_i32(np.array([6], dtype=np.int32))
    wl.block_idx = bad
    mask, _ = binding.build_tree_mask(dw.parents)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = dw.attention(mask, partial=True, dev_err=err)
    torch.cuda.synchronize()
    wl.block_idx, wl.n_blocks = good, np.array([4], dtype=np.int32)
    ref, _ = oracle_attention(wl, partial=True)
    check_attention_close(out, ref, "bad-block")
    assert int(err.item()) & binding.DERR_BAD_BLOCK


@pytest.mark.parametrize("placement", [binding.TREE_IN_LAST_SPLIT, binding.TREE_OWN_WORKGROUP])
def test_attention_tree_split_with_only_invalid_blocks(placement):
    # Every block id of the last prefix split is invalid.  With the tree
    # folded into that split it must still produce the tree's partial; with
    # the tree in its own workgroup the split contributes nothing.
    _say(f"[attention] last split all-invalid blocks, tree placement {placement}")
    wl = W.make_random_case(33, batch=1, n_nodes=9, hq=8, hkv=2, d=128, prefix_lens=[300],
                            block_size=32, blocks_per_seq=4)
    good = wl.block_idx.copy()
    dw = DevWorkload(wl)
    bad = np.concatenate([good, np.array([[-1, 1000, -7, 99]], dtype=np.int32)], axis=1)
    dw.block_idx = dev_i32(bad)
    dw.n_blocks = dev_i32(np.array([8], dtype=np.int32))
    wl.block_idx = bad
    mask, _ = binding.build_tree_mask(dw.parents)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = dw.attention(mask, partial=True, dev_err=err, num_splits=2, tree_placement=placement)
    torch.cuda.synchronize()
    wl.block_idx, wl.n_blocks = good, np.array([4], dtype=np.int32)
    ref, _ = oracle_attention(wl, partial=True)
    check_attention_close(out, ref, "tree-split-invalid-blocks")
    assert int(err.item()) & binding.DERR_BAD_BLOCK


# ---------------------------------------------------------------------------
# a5-a6 acceptance
# ---------------------------------------------------------------------------

def _check_accept(dw_parents, dw_draft, logits_t, host_logits, parents, draft, label=""):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    amax, alen, path, bonus = binding.greedy_accept(logits_t, dw_parents, dw_draft, dev_err=err)
    torch.cuda.synchronize()
    r_amax, r_alen, r_path, r_bonus = oracle.greedy_accept(host_logits, parents, draft)
    assert np.array_equal(amax.cpu().numpy(), r_amax), label
    assert np.array_equal(alen.cpu().numpy(), r_alen), label
    assert np.array_equal(path.cpu().numpy(), r_path), label
    assert np.array_equal(bonus.cpu().numpy(), r_bonus), label
    assert int(err.item()) == 0
    return r_alen


@pytest.mark.parametrize("name", NAMED)
def test_accept_named(workloads, name):
    _say(f"[accept] {name}")
    dw = workloads(name)
    wl = dw.wl
    alen = _check_accept(dw.parents, dw.draft, dw.logits, wl.logits, wl.parents,
                         wl.draft_tokens, name)
    _say(f"  accept_len={list(alen)}")


@pytest.mark.parametrize("seed", range(6))
def test_accept_ties_and_duplicates(seed):
    """Tiny vocabulary with many exact ties and duplicate sibling tokens."""
    _say(f"[accept] ties seed={seed}")
    rng = np.random.default_rng(seed)
    bsz, n, v = 5, int(rng.integers(2, 200)), int(rng.integers(3, 3000))
    parents = np.stack([W.random_tree(rng, n) for _ in range(bsz)])
    vals = rng.integers(-3, 3, size=(bsz, n, v)).astype(np.float32) * 0.5
    host = W.f32_to_bf16_bits(vals)
    zero_rows = rng.random((bsz, n)) < 0.2            # rows of +0/-0 only
    host[zero_rows] = np.where(rng.random((int(zero_rows.sum()), v)) < 0.5, 0x0000, 0x8000)
    amax_ref, _, _, _ = oracle.greedy_accept(host, parents, np.zeros((bsz, n), np.int32))
    draft = np.zeros((bsz, n), dtype=np.int32)
    for b in range(bsz):
        for j in range(1, n):
            draft[b, j] = amax_ref[b, parents[b, j]] if rng.random() < 0.8 else rng.integers(v)
    _check_accept(dev_i32(parents), dev_i32(draft), dev_bf16(host), host, parents, draft,
                  f"ties{seed}")


def test_accept_fp32_and_strided_rows():
    _say("[accept] fp32 strided")
    rng = np.random.default_rng(7)
    bsz, n, v, stride = 2, 40, 5000, 5004
    parents = np.stack([W.random_tree(rng, n) for _ in range(bsz)])
    full = rng.normal(size=(bsz, n, stride)).astype(np.float32)
    full[..., v:] = 100.0   # padding past the vocabulary must be ignored
    host = full[..., :v]
    amax_ref, _, _, _ = oracle.greedy_accept(host, parents, np.zeros((bsz, n), np.int32))
    draft = np.array([[amax_ref[b, parents[b, j]] if j else 0 for j in range(n)]
                      for b in range(bsz)], dtype=np.int32)
    dev_full = torch.from_numpy(full).cuda()
    _check_accept(dev_i32(parents), dev_i32(draft), dev_full[..., :v], host, parents, draft,
                  "fp32-strided")
    # odd stride: scalar path
    dev_odd = torch.from_numpy(np.ascontiguousarray(full[..., :v + 1])).cuda()
    _check_accept(dev_i32(parents), dev_i32(draft), dev_odd[..., :v], host, parents, draft,
                  "fp32-odd")


def test_accept_malformed_parents():
    _say("[accept] malformed parents")
    parents = np.array([[-1, 0, 1], [-1, 2, 0]], dtype=np.int32)
    logits = W.f32_to_bf16_bits(np.random.default_rng(0).normal(size=(2, 3, 50)).astype(np.float32))
    draft = np.zeros((2, 3), dtype=np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    amax, alen, path, bonus = binding.greedy_accept(dev_bf16(logits), dev_i32(parents),
                                                    dev_i32(draft), dev_err=err)
    torch.cuda.synchronize()
    assert int(alen[1]) == 0 and list(path[1].cpu().numpy()) == [0, -1, -1]
    assert int(bonus[1]) == oracle.argmax_lowest(logits[1, 0])
    assert int(err.item()) == binding.DERR_BAD_PARENT


def test_accept_many_short_sequences():
    # many short sequences: one walk workgroup each
    _say("[accept] 1100 sequences")
    bsz, n, v = 1100, 3, 96
    parents, draft, logits = W.make_sampling_case(77, batch=bsz, n_nodes=n, vocab=v, dtype="f32")
    got = binding.greedy_accept(torch.from_numpy(logits).cuda(), dev_i32(parents), dev_i32(draft))
    torch.cuda.synchronize()
    ref = oracle.greedy_accept(logits, parents, draft)
    for k, (x, y) in enumerate(zip(got, ref)):
        assert np.array_equal(x.cpu().numpy(), y), f"output {k}"


def test_accept_workspace_reused_across_calls():
    """One workspace and one set of output buffers serve consecutive calls
    with different inputs: nothing from a previous call leaks into the next
    (outputs are scrambled in between, so a stale result shows)."""
    _say("[accept] one workspace, several calls")
    rng = np.random.default_rng(17)
    bsz, n, v = 3, 40, 70000
    ws = torch.empty(binding.accept_workspace_size(bsz, n, v), dtype=torch.uint8, device="cuda")
    outs = tuple(torch.empty(sh, dtype=torch.int32, device="cuda")
                 for sh in ((bsz, n), (bsz,), (bsz, n), (bsz,)))
    for call in range(4):
        parents = np.full((bsz, n), -1, dtype=np.int32)
        for b in range(bsz):
            for i in range(1, n):
                parents[b, i] = rng.integers(0, i)
        logits = W.f32_to_bf16_bits(rng.normal(size=(bsz, n, v)).astype(np.float32))
        amax_ref, _, _, _ = oracle.greedy_accept(logits, parents, np.zeros((bsz, n), np.int32))
        draft = np.zeros((bsz, n), dtype=np.int32)
        for b in range(bsz):
            for i in range(1, n):
                draft[b, i] = amax_ref[b, parents[b, i]] if rng.random() < 0.8 else rng.integers(v)
        for t in outs:
            t.fill_(-7)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        amax, alen, path, bonus = binding.greedy_accept(dev_bf16(logits), dev_i32(parents),
                                                        dev_i32(draft), workspace=ws, dev_err=err,
                                                        outputs=outs)
        torch.cuda.synchronize()
        r_amax, r_alen, r_path, r_bonus = oracle.greedy_accept(logits, parents, draft)
        assert np.array_equal(amax.cpu().numpy(), r_amax), f"call {call}"
        assert np.array_equal(alen.cpu().numpy(), r_alen), f"call {call}"
        assert np.array_equal(path.cpu().numpy(), r_path), f"call {call}"
        assert np.array_equal(bonus.cpu().numpy(), r_bonus), f"call {call}"
        assert int(err.item()) == 0


# ---------------------------------------------------------------------------
# a7 commit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", NAMED)
def test_commit_named(workloads, name):
    # long_context: the accepted rows land at cache rows 60000 and after
    _say(f"[commit] {name}")
    dw = workloads(name)
    wl = dw.wl
    _, alen, path, _ = oracle.greedy_accept(wl.logits, wl.parents, wl.draft_tokens)
    kc = dw.k_cache.clone()
    vc = dw.v_cache.clone()
    plen = dw.prefix_len.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    newp = binding.commit_kv(dw.k_tree, dw.v_tree, dev_i32(path), dev_i32(alen), plen, kc, vc,
                             new_prefix_len=plen, dev_err=err)   # aliasing allowed
    torch.cuda.synchronize()
    rk, rv, rp = oracle.commit_kv(wl.k_tree, wl.v_tree, path, alen, wl.prefix_len,
                                  wl.k_cache, wl.v_cache)
    assert np.array_equal(newp.cpu().numpy(), rp)
    assert np.array_equal(bf16_host(kc), rk)
    assert np.array_equal(bf16_host(vc), rv)
    assert int(err.item()) == 0


def test_commit_overflow_and_bad_path():
    _say("[commit] overflow / bad path")
    wl = W.make_random_case(41, batch=3, n_nodes=5, hq=4, hkv=2, d=64, prefix_lens=[10, 20, 30])
    dw = DevWorkload(wl)
    cap = wl.capacity
    plen = np.array([10, cap - 2, 30], dtype=np.int32)          # seq 1 overflows
    alen = np.array([2, 3, 1], dtype=np.int32)
    path = np.array([[0, 1, 2, -1, -1], [0, 1, 2, 3, -1], [0, 9, -1, -1, -1]], dtype=np.int32)
    kc, vc = dw.k_cache.clone(), dw.v_cache.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    newp = binding.commit_kv(dw.k_tree, dw.v_tree, dev_i32(path), dev_i32(alen), dev_i32(plen),
                             kc, vc, dev_err=err)
    torch.cuda.synchronize()
    assert list(newp.cpu().numpy()) == [13, cap - 2, 30]
    e = int(err.item())
    assert e & binding.DERR_CAPACITY and e & binding.DERR_BAD_PATH
    rk, _, _ = oracle.commit_kv(wl.k_tree, wl.v_tree, path[:1], alen[:1], plen[:1],
                                wl.k_cache[:1], wl.v_cache[:1])
    got = bf16_host(kc)
    assert np.array_equal(got[:1], rk)
    assert np.array_equal(got[1:], wl.k_cache[1:])     # untouched


# ---------------------------------------------------------------------------
# whole step
# ---------------------------------------------------------------------------

def test_full_step_8b(workloads):
    """mask -> attention -> accept -> commit on one stream, all checked."""
    _say("[step] 8b_layer")
    dw = workloads("8b_layer")
    wl = dw.wl
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    mask, _ = binding.build_tree_mask(dw.parents, dev_err=err)
    out = dw.attention(mask, dev_err=err)
    amax, alen, path, bonus = binding.greedy_accept(dw.logits, dw.parents, dw.draft, dev_err=err)
    kc, vc = dw.k_cache.clone(), dw.v_cache.clone()
    newp = binding.commit_kv(dw.k_tree, dw.v_tree, path, alen, dw.prefix_len, kc, vc,
                             dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref_o, _ = oracle_attention(wl)
    check_attention_close(out, ref_o, "step")
    _, r_alen, r_path, r_bonus = oracle.greedy_accept(wl.logits, wl.parents, wl.draft_tokens)
    assert np.array_equal(alen.cpu().numpy(), r_alen)
    assert np.array_equal(path.cpu().numpy(), r_path)
    rk, rv, rp = oracle.commit_kv(wl.k_tree, wl.v_tree, r_path, r_alen, wl.prefix_len,
                                  wl.k_cache, wl.v_cache)
    assert np.array_equal(bf16_host(kc), rk) and np.array_equal(newp.cpu().numpy(), rp)


def test_attention_large_score_jump_recomputes():
    """A later tile scores far above the first tile of its split (a row sum
    far beyond 2^100 relative to the first reference): the split must fall
    back to the exact two-pass computation and still match the oracle."""
    _say("[attention] score jump")
    wl = W.make_random_case(51, batch=1, n_nodes=5, hq=8, hkv=2, d=128, prefix_lens=[300])
    big = W.f32_to_bf16_bits(np.full(128, 6.0, dtype=np.float32))
    wl.q[:] = big                      # q.k = 128*36 at the boosted keys
    wl.k_cache[0, :, 200:230] = big    # inside a later tile of the same split
    _run_attention_case(DevWorkload(wl), label="score-jump", num_splits=1)


def test_attention_first_block_invalid_then_valid():
    _say("[attention] first listed block invalid")
    wl = W.make_random_case(52, batch=1, n_nodes=7, hq=8, hkv=2, d=128, prefix_lens=[400],
                            block_size=32, blocks_per_seq=5)
    good_idx, good_n = wl.block_idx.copy(), wl.n_blocks.copy()
    dw = DevWorkload(wl)
    bad = np.concatenate([np.array([[1000]], dtype=np.int32), good_idx], axis=1)
    dw.block_idx = dev_i32(bad)
    dw.n_blocks = dev_i32(good_n + 1)
    wl.block_idx = bad
    mask, _ = binding.build_tree_mask(dw.parents)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = dw.attention(mask, partial=True, dev_err=err, num_splits=1)
    torch.cuda.synchronize()
    wl.block_idx, wl.n_blocks = good_idx, good_n
    ref, _ = oracle_attention(wl, partial=True)
    check_attention_close(out, ref, "first-block-invalid")
    assert int(err.item()) & binding.DERR_BAD_BLOCK


# ---------------------------------------------------------------------------
# a1 fused into a2/a3: the mask built by the attention's tree workgroups
# ---------------------------------------------------------------------------

def _fused_vs_standalone(dw, partial, parents=None, label=""):
    wl = dw.wl
    par = dw.parents if parents is None else parents
    err1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    mask, depth = binding.build_tree_mask(par, dev_err=err1)
    ref = dw.attention(mask, partial=partial)
    b, n = par.shape
    mask_out = torch.full((b, n, (n + 31) // 32), -5, dtype=torch.int32, device="cuda")
    depth_out = torch.full((b, n), -5, dtype=torch.int32, device="cuda")
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = binding.tree_attention(
        dw.q, dw.k_cache, dw.v_cache, dw.k_tree, dw.v_tree, dw.prefix_len, None,
        max_prefix_len=wl.max_prefix_len, block_idx=dw.block_idx if partial else None,
        n_blocks=dw.n_blocks if partial else None, block_size=wl.block_size if partial else 0,
        parents=par, mask_out=mask_out, depth_out=depth_out, dev_err=err2)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{label}: outputs differ"
    assert torch.equal(mask_out, mask), f"{label}: mask_out differs"
    assert torch.equal(depth_out, depth), f"{label}: depth_out differs"
    assert int(err1.item()) == int(err2.item())
    return int(err2.item())


@pytest.mark.parametrize("name", NAMED)
def test_fused_mask_matches_standalone(workloads, name):
    _say(f"[fused mask] {name}")
    dw = workloads(name)
    assert _fused_vs_standalone(dw, False, label=name) == 0
    if dw.wl.block_idx is not None:
        assert _fused_vs_standalone(dw, True, label=name + " partial") == 0


def test_fused_mask_rectifying_tree_two_row_groups():
    # 81 nodes x 4 heads = 324 rows: two row groups of the attention grid
    _say("[fused mask] 81-node tree, two row groups")
    wl = W.make_random_case(31, batch=2, n_nodes=81, hq=8, hkv=2, d=128,
                            prefix_lens=[700, 1300], tree="random")
    assert _fused_vs_standalone(DevWorkload(wl), False, label="81 nodes") == 0


def test_fused_mask_malformed_tree_fallback():
    _say("[fused mask] malformed tree")
    wl = W.make_random_case(32, batch=3, n_nodes=20, hq=4, hkv=2, d=64,
                            prefix_lens=[100, 50, 77])
    dw = DevWorkload(wl)
    bad = wl.parents.copy()
    bad[1, 7] = 9
    err = _fused_vs_standalone(dw, False, parents=dev_i32(bad), label="malformed")
    assert err & binding.DERR_BAD_PARENT


# ---------------------------------------------------------------------------
# a6 + a7 in one call: the walk workgroup commits the accepted rows
# ---------------------------------------------------------------------------

def _accept_commit_vs_two_calls(dw, prefix=None, parents=None, alias=False, label=""):
    wl = dw.wl
    par = dw.parents if parents is None else parents
    pre = dw.prefix_len if prefix is None else prefix
    kc1, vc1 = dw.k_cache.clone(), dw.v_cache.clone()
    kc2, vc2 = dw.k_cache.clone(), dw.v_cache.clone()
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    amax, alen, path, bonus = binding.greedy_accept(dw.logits, par, dw.draft, dev_err=e1)
    newp1 = binding.commit_kv(dw.k_tree, dw.v_tree, path, alen, pre, kc1, vc1, dev_err=e1)
    pre2 = pre.clone()
    got = binding.greedy_accept_commit(dw.logits, par, dw.draft, dw.k_tree, dw.v_tree, pre2, kc2,
                                       vc2, new_prefix_len=pre2 if alias else None, dev_err=e2)
    torch.cuda.synchronize()
    for k, (x, y) in enumerate(zip(got[:4], (amax, alen, path, bonus))):
        assert torch.equal(x, y), f"{label}: acceptance output {k} differs"
    assert torch.equal(got[4], newp1), f"{label}: new prefix differs"
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), f"{label}: K cache differs"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), f"{label}: V cache differs"
    assert int(e1.item()) == int(e2.item()), f"{label}: error bits differ"
    return int(e2.item())


@pytest.mark.parametrize("name", NAMED)
def test_accept_commit_matches_two_calls(workloads, name):
    _say(f"[accept+commit] {name}")
    assert _accept_commit_vs_two_calls(workloads(name), label=name) == 0


@pytest.mark.parametrize("name", NAMED)
def test_accept_commit_vs_oracle(workloads, name):
    # the fused call against the oracle's acceptance followed by its commit
    _say(f"[accept+commit vs oracle] {name}")
    dw = workloads(name)
    wl = dw.wl
    kc, vc = dw.k_cache.clone(), dw.v_cache.clone()
    pre = dw.prefix_len.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    amax, alen, path, bonus, newp = binding.greedy_accept_commit(
        dw.logits, dw.parents, dw.draft, dw.k_tree, dw.v_tree, pre, kc, vc, dev_err=err)
    torch.cuda.synchronize()
    r_amax, r_alen, r_path, r_bonus = oracle.greedy_accept(wl.logits, wl.parents, wl.draft_tokens)
    assert np.array_equal(amax.cpu().numpy(), r_amax)
    assert np.array_equal(alen.cpu().numpy(), r_alen)
    assert np.array_equal(path.cpu().numpy(), r_path)
    assert np.array_equal(bonus.cpu().numpy(), r_bonus)
    rk, rv, rp = oracle.commit_kv(wl.k_tree, wl.v_tree, r_path, r_alen, wl.prefix_len,
                                  wl.k_cache, wl.v_cache)
    assert np.array_equal(newp.cpu().numpy(), rp)
    assert np.array_equal(bf16_host(kc), rk)
    assert np.array_equal(bf16_host(vc), rv)
    assert int(err.item()) == 0


def test_accept_commit_edge_cases(workloads):
    _say("[accept+commit] aliasing, overflow, bad prefix, malformed tree")
    dw = workloads("batched")
    wl = dw.wl
    assert _accept_commit_vs_two_calls(dw, alias=True, label="alias") == 0
    cap = wl.capacity
    full = dev_i32([cap - 1] + [int(x) for x in wl.prefix_len[1:]])
    assert _accept_commit_vs_two_calls(dw, prefix=full, label="overflow") & binding.DERR_CAPACITY
    badp = dev_i32([-3] + [int(x) for x in wl.prefix_len[1:]])
    assert _accept_commit_vs_two_calls(dw, prefix=badp, label="bad prefix") & \
        binding.DERR_BAD_PREFIX
    par = wl.parents.copy()
    par[2, 5] = 17
    assert _accept_commit_vs_two_calls(dw, parents=dev_i32(par), label="malformed") & \
        binding.DERR_BAD_PARENT


@pytest.mark.parametrize("case", [c for c in ATTN_CASES if c[0] in (3, 4, 5, 6, 8, 12, 14)],
                         ids=lambda c: f"case{c[0]}")
def test_fused_mask_random_cases(case):
    # 1 to 4 row groups, empty prefixes, partial mode with ragged blocks
    seed, bsz, n, hq, hkv, d, plens, bs, bps, tree = case
    _say(f"[fused mask] random case {case}")
    wl = W.make_random_case(seed, batch=bsz, n_nodes=n, hq=hq, hkv=hkv, d=d, prefix_lens=plens,
                            block_size=bs, blocks_per_seq=bps, tree=tree)
    assert _fused_vs_standalone(DevWorkload(wl), bool(bs), label=f"case{seed}") == 0
