"""Parity of the 32-row attention schedule (TV_ATTN_KERNEL_WIDE) with the fp64
oracle, on the same seeded cases as the 16-row schedule: the five named
workloads (full and partial KV), the random shapes (ragged tails, empty
prefixes, several row groups, partial blocks of 16, 48 and 64 tokens), both
tree placements, forced split counts, the exact recompute after a score
jump, invalid block ids, and the mask built in-kernel from the parent array.
Tolerance as everywhere: |gpu - oracle| <= 2e-2 + 1e-2 |oracle|, lse within
2e-3."""

import numpy as np
import pytest
import torch

from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W

from .gpu_util import DevWorkload, check_attention_close, dev_i32, oracle_attention
from .test_gpu_parity import ATTN_CASES, NAMED, _run_attention_case, _say

pytestmark = pytest.mark.gpu

WIDE = dict(kernel=binding.KERNEL_WIDE)


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


@pytest.mark.parametrize("name,partial", [(n, False) for n in NAMED] + [("long_context", True)])
def test_wide_named(workloads, name, partial):
    _say(f"[wide attention] {name} partial={partial}")
    _, e, rel = _run_attention_case(workloads(name), partial=partial, label=f"wide {name}", **WIDE)
    _say(f"  max_abs_err={e:.3g} rel={rel:.3g}")


@pytest.mark.parametrize("case", ATTN_CASES, ids=[f"case{c[0]}" for c in ATTN_CASES])
def test_wide_random(case):
    seed, bsz, n, hq, hkv, d, plens, bs, bps, tree = case
    _say(f"[wide attention] random case {case}")
    wl = W.make_random_case(seed, batch=bsz, n_nodes=n, hq=hq, hkv=hkv, d=d, prefix_lens=plens,
                            block_size=bs, blocks_per_seq=bps, tree=tree)
    _run_attention_case(DevWorkload(wl), partial=bool(bs), label=f"wide case{seed}", **WIDE)


@pytest.mark.parametrize("placement", [binding.TREE_IN_LAST_SPLIT, binding.TREE_OWN_WORKGROUP])
@pytest.mark.parametrize("case", [c for c in ATTN_CASES if c[0] in (2, 3, 4, 8, 10, 12)],
                         ids=lambda c: f"case{c[0]}")
def test_wide_tree_placements(case, placement):
    seed, bsz, n, hq, hkv, d, plens, bs, bps, tree = case
    _say(f"[wide attention] tree placement {placement} case {seed}")
    wl = W.make_random_case(seed, batch=bsz, n_nodes=n, hq=hq, hkv=hkv, d=d, prefix_lens=plens,
                            block_size=bs, blocks_per_seq=bps, tree=tree)
    _run_attention_case(DevWorkload(wl), partial=bool(bs), label=f"wide case{seed}-p{placement}",
                        tree_placement=placement, **WIDE)


@pytest.mark.parametrize("splits", [1, 2, 7, 31])
def test_wide_split_counts(workloads, splits):
    _say(f"[wide attention] 8b_layer splits={splits}")
    _run_attention_case(workloads("8b_layer"), label=f"wide splits{splits}", num_splits=splits,
                        **WIDE)


def test_wide_long_context_split_counts(workloads):
    # few, long splits: many tiles per workgroup through the whole DMA ring
    for splits in (3, 64):
        _say(f"[wide attention] long_context splits={splits}")
        _run_attention_case(workloads("long_context"), label=f"wide lc splits{splits}",
                            num_splits=splits, **WIDE)


def test_wide_score_jump_recomputes():
    _say("[wide attention] score jump")
    wl = W.make_random_case(51, batch=1, n_nodes=5, hq=8, hkv=2, d=128, prefix_lens=[300])
    big = W.f32_to_bf16_bits(np.full(128, 6.0, dtype=np.float32))
    wl.q[:] = big
    wl.k_cache[0, :, 200:230] = big
    _run_attention_case(DevWorkload(wl), label="wide score-jump", num_splits=1, **WIDE)


def test_wide_bad_blocks_are_skipped():
    _say("[wide attention] bad block ids")
    wl = W.make_random_case(31, batch=1, n_nodes=6, hq=8, hkv=2, d=128, prefix_lens=[200],
                            block_size=32, blocks_per_seq=4)
    good = wl.block_idx.copy()
    dw = DevWorkload(wl)
    bad = np.concatenate([good, np.array([[-3, 50]], dtype=np.int32)], axis=1)
    dw.block_idx = dev_i32(bad)
    dw.n_blocks = dev_i32(np.array([6], dtype=np.int32))
    wl.block_idx = bad
    mask, _ = binding.build_tree_mask(dw.parents)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = dw.attention(mask, partial=True, dev_err=err, **WIDE)
    torch.cuda.synchronize()
    wl.block_idx, wl.n_blocks = good, np.array([4], dtype=np.int32)
    ref, _ = oracle_attention(wl, partial=True)
    check_attention_close(out, ref, "wide bad-block")
    assert int(err.item()) & binding.DERR_BAD_BLOCK


def _wide_fused_vs_standalone(dw, partial, label):
    wl = dw.wl
    err1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    mask, depth = binding.build_tree_mask(dw.parents, dev_err=err1)
    ref = dw.attention(mask, partial=partial, **WIDE)
    b, n = dw.parents.shape
    mask_out = torch.full((b, n, (n + 31) // 32), -5, dtype=torch.int32, device="cuda")
    depth_out = torch.full((b, n), -5, dtype=torch.int32, device="cuda")
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = binding.tree_attention(
        dw.q, dw.k_cache, dw.v_cache, dw.k_tree, dw.v_tree, dw.prefix_len, None,
        max_prefix_len=wl.max_prefix_len, block_idx=dw.block_idx if partial else None,
        n_blocks=dw.n_blocks if partial else None, block_size=wl.block_size if partial else 0,
        parents=dw.parents, mask_out=mask_out, depth_out=depth_out, dev_err=err2, **WIDE)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{label}: outputs differ"
    assert torch.equal(mask_out, mask), f"{label}: mask_out differs"
    assert torch.equal(depth_out, depth), f"{label}: depth_out differs"
    assert int(err1.item()) == int(err2.item()) == 0


@pytest.mark.parametrize("name", NAMED)
def test_wide_fused_mask_matches_standalone(workloads, name):
    _say(f"[wide fused mask] {name}")
    dw = workloads(name)
    _wide_fused_vs_standalone(dw, False, f"wide {name}")
    if dw.wl.block_idx is not None:
        _wide_fused_vs_standalone(dw, True, f"wide {name} partial")


def test_wide_rectifying_tree_rows():
    # 81 nodes x 4 heads = 324 rows: two row groups
    _say("[wide attention] 81-node tree")
    wl = W.make_random_case(31, batch=2, n_nodes=81, hq=8, hkv=2, d=128,
                            prefix_lens=[700, 1300], tree="random")
    _run_attention_case(DevWorkload(wl), label="wide 81 nodes", **WIDE)
    _wide_fused_vs_standalone(DevWorkload(wl), False, "wide 81 nodes fused")


def test_wide_deterministic(workloads):
    _say("[wide attention] determinism")
    dw = workloads("long_context")
    mask, _ = binding.build_tree_mask(dw.parents)
    a = dw.attention(mask, **WIDE)
    b = dw.attention(mask, **WIDE)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_wide_merge_counters_left_zero_and_workspace_reused():
    # the in-launch merge waits on counters at the start of the workspace:
    # every call must leave them zero, so one workspace serves calls of
    # different descriptors in turn
    _say("[wide attention] merge counters")
    ws = None
    for seed, bsz, plens in ((61, 3, [900, 0, 2500]), (62, 1, [4000]), (63, 3, [50, 700, 1])):
        wl = W.make_random_case(seed, batch=bsz, n_nodes=20, hq=8, hkv=2, d=128, prefix_lens=plens)
        dw = DevWorkload(wl)
        desc = binding.attn_desc(dw.q, dw.k_cache, max_prefix_len=wl.max_prefix_len, kernel=binding.KERNEL_WIDE)
        need = binding.attention_workspace_size(desc)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 4 << 20), dtype=torch.uint8, device="cuda")
        mask, _ = binding.build_tree_mask(dw.parents)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = dw.attention(mask, workspace=ws, dev_err=err, **WIDE)
        torch.cuda.synchronize()
        ref, _ = oracle_attention(wl)
        check_attention_close(out, ref, f"wide reuse seed {seed}")
        assert int(err.item()) == 0
        assert int(ws[:binding.ATTN_WS_COUNTER_BYTES].count_nonzero().item()) == 0, "counters not reset"


def test_wide_many_units_merge_in_second_launch():
    # batch * kv heads beyond the counter area: partials merged by a second launch
    _say("[wide attention] 520 x 8 units")
    bsz = 520
    rng = np.random.default_rng(5)
    plens = rng.integers(0, 70, size=bsz).tolist()
    wl = W.make_random_case(64, batch=bsz, n_nodes=3, hq=8, hkv=8, d=64, prefix_lens=plens, tree="chain")
    _run_attention_case(DevWorkload(wl), label="wide 520x8", **WIDE)


def test_attention_workspace_holds_the_counters():
    # every descriptor's workspace (either schedule) starts with the merge counters
    for kernel in (binding.KERNEL_SPLIT16, binding.KERNEL_WIDE):
        for bsz, n, cap in ((1, 5, 64), (4, 60, 60000), (16, 32, 1600)):
            d = binding.AttnDesc()
            d.batch, d.n_nodes, d.n_q_heads, d.n_kv_heads, d.head_dim = bsz, n, 32, 8, 128
            d.cache_capacity, d.max_prefix_len, d.kernel = cap, cap, kernel
            size = binding.attention_workspace_size(d)
            parts = bsz * n * 32  # at least one partial row per output row
            assert size >= binding.ATTN_WS_COUNTER_BYTES + parts * (128 * 2 + 8)
