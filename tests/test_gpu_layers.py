"""Multi-layer commit on the GPU: tv_commit_kv_layers and
tv_greedy_accept_commit_layers.

Every layer's cache must equal the oracle's commit of that layer's tree rows
(bit for bit), and the calls must equal the one-layer calls made once per
layer: outputs, caches, new prefix lengths and error bits.  Two cache
layouts: layer-major [L][B][Hkv][cap][D] and sequence-major
[B][L][Hkv][cap][D] seen through a permuted view.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W

from .gpu_util import bf16_host, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(seed, n_layers, layout, batch=3, n=24, hkv=4, d=128, prefix_lens=(50, 120, 7)):
    wl = W.make_random_case(seed, batch=batch, n_nodes=n, hq=hkv * 2, hkv=hkv, d=d,
                            prefix_lens=list(prefix_lens), vocab=500, p_match=0.7)
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    cap = wl.capacity
    kt = np.stack([W.f32_to_bf16_bits(rng.standard_normal((batch, n, hkv, d)).astype(np.float32))
                   for _ in range(n_layers)])
    vt = np.stack([W.f32_to_bf16_bits(rng.standard_normal((batch, n, hkv, d)).astype(np.float32))
                   for _ in range(n_layers)])
    kc = np.stack([W.kv_cache(rng, batch, hkv, cap, d, wl.prefix_len) for _ in range(n_layers)])
    vc = np.stack([W.kv_cache(rng, batch, hkv, cap, d, wl.prefix_len) for _ in range(n_layers)])
    return wl, kt, vt, kc, vc


def _dev_caches(kc, vc, layout):
    """Device caches [L][B][Hkv][cap][D] (a view in the sequence-major layout)."""
    if layout == "layer":
        return dev_bf16(kc), dev_bf16(vc)
    kb = dev_bf16(np.ascontiguousarray(kc.transpose(1, 0, 2, 3, 4)))
    vb = dev_bf16(np.ascontiguousarray(vc.transpose(1, 0, 2, 3, 4)))
    return kb.permute(1, 0, 2, 3, 4), vb.permute(1, 0, 2, 3, 4)


@pytest.mark.parametrize("layout", ["layer", "sequence"])
@pytest.mark.parametrize("n_layers", [1, 3, 5])
def test_commit_layers_matches_oracle_and_per_layer_calls(n_layers, layout):
    _say(f"[layers] commit, {n_layers} layers, {layout}-major caches")
    wl, kt, vt, kc, vc = _case(7 + n_layers, n_layers, layout)
    amax, alen, path, _ = oracle.greedy_accept(wl.logits, wl.parents, wl.draft_tokens)
    k_tree, v_tree = dev_bf16(kt), dev_bf16(vt)
    k1, v1 = _dev_caches(kc, vc, layout)
    k2, v2 = _dev_caches(kc, vc, layout)
    pth, aln, pre = dev_i32(path), dev_i32(alen), dev_i32(wl.prefix_len)
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    newp = binding.commit_kv_layers(k_tree, v_tree, pth, aln, pre, k1, v1, dev_err=e1)
    for l in range(n_layers):
        np2 = binding.commit_kv(k_tree[l], v_tree[l], pth, aln, pre, k2[l], v2[l], dev_err=e2)
    torch.cuda.synchronize()
    assert int(e1.item()) == 0 and int(e2.item()) == 0
    assert torch.equal(newp, np2)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    for l in range(n_layers):
        rk, rv, rn = oracle.commit_kv(kt[l], vt[l], path, alen, wl.prefix_len, kc[l], vc[l])
        assert np.array_equal(bf16_host(k1[l]), rk), f"layer {l}: K cache"
        assert np.array_equal(bf16_host(v1[l]), rv), f"layer {l}: V cache"
        assert np.array_equal(newp.cpu().numpy(), rn)


def _accept_commit_vs_calls(wl, kt, vt, kc, vc, layout, prefix=None, parents=None, label=""):
    n_layers = kt.shape[0]
    lg = dev_bf16(wl.logits) if wl.logits_dtype == "bf16" else torch.from_numpy(wl.logits).cuda()
    par = dev_i32(wl.parents if parents is None else parents)
    dr = dev_i32(wl.draft_tokens)
    pre = dev_i32(wl.prefix_len if prefix is None else prefix)
    k_tree, v_tree = dev_bf16(kt), dev_bf16(vt)
    k1, v1 = _dev_caches(kc, vc, layout)
    k2, v2 = _dev_caches(kc, vc, layout)
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = binding.greedy_accept_commit_layers(lg, par, dr, k_tree, v_tree, pre, k1, v1,
                                              dev_err=e1)
    amax, alen, path, bonus = binding.greedy_accept(lg, par, dr, dev_err=e2)
    for l in range(n_layers):
        newp = binding.commit_kv(k_tree[l], v_tree[l], path, alen, pre, k2[l], v2[l], dev_err=e2)
    torch.cuda.synchronize()
    for k, (x, y) in enumerate(zip(got[:4], (amax, alen, path, bonus))):
        assert torch.equal(x, y), f"{label}: acceptance output {k} differs"
    assert torch.equal(got[4], newp), f"{label}: new prefix differs"
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16)), f"{label}: K caches differ"
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16)), f"{label}: V caches differ"
    assert int(e1.item()) == int(e2.item()), f"{label}: error bits differ"
    return int(e1.item()), got


@pytest.mark.parametrize("layout", ["layer", "sequence"])
@pytest.mark.parametrize("n_layers", [1, 4])
def test_accept_commit_layers_matches_separate_calls(n_layers, layout):
    _say(f"[layers] accept+commit, {n_layers} layers, {layout}-major caches")
    wl, kt, vt, kc, vc = _case(31 + n_layers, n_layers, layout)
    err, got = _accept_commit_vs_calls(wl, kt, vt, kc, vc, layout, label="plain")
    assert err == 0
    # and the oracle's acceptance
    amax, alen, path, bonus = oracle.greedy_accept(wl.logits, wl.parents, wl.draft_tokens)
    assert np.array_equal(got[1].cpu().numpy(), alen)
    assert np.array_equal(got[2].cpu().numpy(), path)
    assert np.array_equal(got[3].cpu().numpy(), bonus)


def test_accept_commit_layers_edge_cases():
    _say("[layers] overflow, bad prefix, malformed tree")
    wl, kt, vt, kc, vc = _case(77, 3, "layer")
    cap = wl.capacity
    full = wl.prefix_len.copy()
    full[1] = cap  # no room for even the root row
    err, _ = _accept_commit_vs_calls(wl, kt, vt, kc, vc, "layer", prefix=full, label="overflow")
    assert err & binding.DERR_CAPACITY
    bad = wl.prefix_len.copy()
    bad[0] = -2
    err, _ = _accept_commit_vs_calls(wl, kt, vt, kc, vc, "sequence", prefix=bad, label="bad")
    assert err & binding.DERR_BAD_PREFIX
    par = wl.parents.copy()
    par[2, 5] = 9
    err, _ = _accept_commit_vs_calls(wl, kt, vt, kc, vc, "layer", parents=par, label="malformed")
    assert err & binding.DERR_BAD_PARENT


def test_commit_layers_aliasing():
    _say("[layers] new_prefix_len aliasing")
    wl, kt, vt, kc, vc = _case(5, 2, "layer")
    amax, alen, path, _ = oracle.greedy_accept(wl.logits, wl.parents, wl.draft_tokens)
    k_tree, v_tree = dev_bf16(kt), dev_bf16(vt)
    k1, v1 = _dev_caches(kc, vc, "layer")
    pre = dev_i32(wl.prefix_len)
    with pytest.raises(binding.TVError):
        binding.commit_kv_layers(k_tree, v_tree, dev_i32(path), dev_i32(alen), pre, k1, v1,
                                 new_prefix_len=pre)
    # one layer: the alias is allowed, as for tv_commit_kv
    binding.commit_kv_layers(k_tree[:1], v_tree[:1], dev_i32(path), dev_i32(alen), pre, k1[:1],
                             v1[:1], new_prefix_len=pre)
    torch.cuda.synchronize()
    assert np.array_equal(pre.cpu().numpy(), wl.prefix_len + alen + 1)
    rk, _, _ = oracle.commit_kv(kt[0], vt[0], path, alen, wl.prefix_len, kc[0], vc[0])
    assert np.array_equal(bf16_host(k1[0]), rk)
