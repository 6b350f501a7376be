"""Every kernel writes its outputs and nothing else.

Each output here is a view into a larger device buffer whose leading and
trailing guard regions hold a sentinel bit pattern.  After the call the guards
must hold the sentinel still, and the outputs must equal those of the same call
into freshly allocated tensors (bit for bit: the kernels' sums run in a fixed
order).  The caches of the commit calls are guarded the same way, and every
cache row the accepted path does not own must be unchanged.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W

from .gpu_util import DevWorkload, dev_i32

pytestmark = pytest.mark.gpu

G = 4096  # guard elements on each side of an output
SENTINEL = {torch.int32: 0x7FC01234, torch.float32: 0x7FC01234, torch.bfloat16: 0x7FC3,
            torch.int16: 0x7FC3}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.int16) else t.view(torch.int32)


class Guarded:
    """A contiguous view of `shape` inside a buffer with G sentinel elements
    on each side."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape))
        self.big = torch.empty(self.n + 2 * G, dtype=dtype, device="cuda")
        _bits(self.big).fill_(SENTINEL[dtype])
        self.view = self.big[G:G + self.n].view(shape)

    def check(self, name):
        torch.cuda.synchronize()
        raw = _bits(self.big)
        ref = raw[0].item()
        head, tail = raw[:G], raw[G + self.n:]
        assert bool((head == ref).all()), f"{name}: the leading guard was written"
        assert bool((tail == ref).all()), f"{name}: the trailing guard was written"


def _same(name, a, b):
    assert torch.equal(_bits(a.contiguous()), _bits(b.contiguous())), f"{name} differs"


# ---- attention ---------------------------------------------------------------------------

ATTN = [
    # seed, batch, n, hq, hkv, d, prefix lens, block_size, blocks/seq
    (3, 2, 17, 8, 2, 128, [95, 33], 0, None),
    (5, 1, 100, 32, 8, 128, [700], 0, None),
    (4, 3, 5, 6, 3, 64, [0, 1, 64], 0, None),
    (8, 2, 12, 32, 8, 128, [900, 450], 16, 20),
]


@pytest.mark.parametrize("kernel", [binding.KERNEL_SPLIT16, binding.KERNEL_WIDE])
@pytest.mark.parametrize("case", ATTN, ids=lambda c: f"case{c[0]}")
def test_attention_writes_only_its_outputs(case, kernel):
    seed, bsz, n, hq, hkv, d, plens, bs, bps = case
    _say(f"[guards] attention case {seed} kernel {kernel}")
    wl = W.make_random_case(seed, batch=bsz, n_nodes=n, hq=hq, hkv=hkv, d=d, prefix_lens=plens,
                            block_size=bs, blocks_per_seq=bps)
    dw = DevWorkload(wl)
    partial = bool(bs)
    w = (n + 31) // 32
    out = Guarded((bsz, n, hq, d), torch.bfloat16)
    lse = Guarded((bsz, n, hq), torch.float32)
    mask_out = Guarded((bsz, n, w), torch.int32)
    depth_out = Guarded((bsz, n), torch.int32)
    dw.attention(None, partial=partial, kernel=kernel, want_lse=True, out=out.view,
                 lse=lse.view, parents=dw.parents, mask_out=mask_out.view,
                 depth_out=depth_out.view)
    for name, g in (("out", out), ("lse", lse), ("mask_out", mask_out), ("depth_out", depth_out)):
        g.check(name)
    m2 = torch.empty((bsz, n, w), dtype=torch.int32, device="cuda")
    d2 = torch.empty((bsz, n), dtype=torch.int32, device="cuda")
    o2, l2 = dw.attention(None, partial=partial, kernel=kernel, want_lse=True,
                          parents=dw.parents, mask_out=m2, depth_out=d2)
    _same("out", out.view, o2)
    _same("lse", lse.view, l2)
    _same("mask_out", mask_out.view, m2)
    _same("depth_out", depth_out.view, d2)


def test_tree_mask_writes_only_its_outputs():
    _say("[guards] tv_build_tree_mask")
    wl = W.make_random_case(6, batch=2, n_nodes=70, hq=4, hkv=1, d=64, prefix_lens=[8, 9])
    par = dev_i32(wl.parents)
    bsz, n = wl.parents.shape
    w = (n + 31) // 32
    mask = Guarded((bsz, n, w), torch.int32)
    depth = Guarded((bsz, n), torch.int32)
    lib = binding.lib()
    st = lib.tv_build_tree_mask(ctypes.c_void_p(par.data_ptr()), bsz, n,
                                ctypes.c_void_p(mask.view.data_ptr()),
                                ctypes.c_void_p(depth.view.data_ptr()), None,
                                binding._stream(par.device))
    assert st == 0
    mask.check("mask")
    depth.check("depth")
    m2, d2 = binding.build_tree_mask(par)
    _same("mask", mask.view, m2)
    _same("depth", depth.view, d2)


# ---- acceptance --------------------------------------------------------------------------

def _accept_outputs(bsz, n):
    return [Guarded((bsz, n), torch.int32), Guarded((bsz,), torch.int32),
            Guarded((bsz, n), torch.int32), Guarded((bsz,), torch.int32)]


@pytest.mark.parametrize("name", ["tiny", "8b_layer"])
def test_greedy_accept_writes_only_its_outputs(name):
    _say(f"[guards] greedy acceptance {name}")
    dw = DevWorkload(W.make_workload(name))
    bsz, n = dw.wl.parents.shape
    g = _accept_outputs(bsz, n)
    binding.greedy_accept(dw.logits, dw.parents, dw.draft, outputs=tuple(x.view for x in g))
    for nm, x in zip(("target_argmax", "accept_len", "accept_path", "bonus"), g):
        x.check(nm)
    ref = binding.greedy_accept(dw.logits, dw.parents, dw.draft)
    for nm, x, r in zip(("target_argmax", "accept_len", "accept_path", "bonus"), g, ref):
        _same(nm, x.view, r)


def _guarded_cache(k_cache):
    """The cache inside a guarded buffer: (Guarded, view of the same shape)."""
    g = Guarded(tuple(k_cache.shape), torch.bfloat16)
    g.view.copy_(k_cache)
    return g


def _owned_rows(alen, path, plen, cap, bsz):
    """[B][cap] booleans: the rows the commit of each accepted path writes."""
    own = np.zeros((bsz, cap), dtype=bool)
    for b in range(bsz):
        own[b, plen[b]:plen[b] + alen[b] + 1] = True
    return own


@pytest.mark.parametrize("name", ["tiny", "batched"])
def test_accept_commit_writes_only_its_rows(name):
    _say(f"[guards] greedy acceptance + commit {name}")
    dw = DevWorkload(W.make_workload(name))
    bsz, n = dw.wl.parents.shape
    cap = dw.k_cache.shape[2]
    kc, vc = _guarded_cache(dw.k_cache), _guarded_cache(dw.v_cache)
    k0, v0 = dw.k_cache.clone(), dw.v_cache.clone()
    g = _accept_outputs(bsz, n)
    newp = Guarded((bsz,), torch.int32)
    binding.greedy_accept_commit(dw.logits, dw.parents, dw.draft, dw.k_tree, dw.v_tree,
                                 dw.prefix_len, kc.view, vc.view, new_prefix_len=newp.view,
                                 outputs=tuple(x.view for x in g))
    for nm, x in zip(("target_argmax", "accept_len", "accept_path", "bonus"), g):
        x.check(nm)
    newp.check("new_prefix_len")
    kc.check("k_cache")
    vc.check("v_cache")
    alen = g[1].view.cpu().numpy()
    path = g[2].view.cpu().numpy()
    plen = dw.wl.prefix_len
    own = torch.from_numpy(_owned_rows(alen, path, plen, cap, bsz)).cuda()
    keep = ~own[:, None, :, None].expand_as(k0)
    assert torch.equal(_bits(kc.view)[keep], _bits(k0)[keep]), "k_cache rows off the path changed"
    assert torch.equal(_bits(vc.view)[keep], _bits(v0)[keep]), "v_cache rows off the path changed"
    # the path's rows hold the accepted nodes' tree rows
    for b in range(bsz):
        for r in range(alen[b] + 1):
            node = path[b, r]
            assert torch.equal(_bits(kc.view[b, :, plen[b] + r]), _bits(dw.k_tree[b, node]))
            assert torch.equal(_bits(vc.view[b, :, plen[b] + r]), _bits(dw.v_tree[b, node]))


@pytest.mark.parametrize("filt", [None, (20, 0.95), (0, 0.9)], ids=["plain", "k20p95", "p90"])
def test_stochastic_accept_writes_only_its_outputs(filt):
    _say(f"[guards] stochastic acceptance {filt}")
    parents, draft, logits = W.make_sampling_case(11, batch=3, n_nodes=40, vocab=50000,
                                                  dtype="bf16", tree="eagle", lean=(3.0, 7.0))
    lg = torch.from_numpy(np.ascontiguousarray(logits).view(np.int16)).cuda().view(torch.bfloat16)
    par, dr = dev_i32(parents), dev_i32(draft)
    bsz, n = parents.shape
    g = [Guarded((bsz,), torch.int32), Guarded((bsz, n), torch.int32),
         Guarded((bsz,), torch.int32)]
    kw = dict(seed=(5, 6), step=2)
    if filt is None:
        binding.stochastic_accept(lg, par, dr, 0.8, outputs=tuple(x.view for x in g), **kw)
        ref = binding.stochastic_accept(lg, par, dr, 0.8, **kw)
    else:
        binding.stochastic_accept_filtered(lg, par, dr, 0.8, top_k=filt[0], top_p=filt[1],
                                           outputs=tuple(x.view for x in g), **kw)
        ref = binding.stochastic_accept_filtered(lg, par, dr, 0.8, top_k=filt[0],
                                                 top_p=filt[1], **kw)
    for nm, x, r in zip(("accept_len", "accept_path", "bonus"), g, ref):
        x.check(nm)
        _same(nm, x.view, r)


def test_commit_kv_writes_only_its_rows():
    _say("[guards] tv_commit_kv")
    dw = DevWorkload(W.make_workload("tiny"))
    bsz, n = dw.wl.parents.shape
    cap = dw.k_cache.shape[2]
    amax, alen, path, bonus = binding.greedy_accept(dw.logits, dw.parents, dw.draft)
    kc, vc = _guarded_cache(dw.k_cache), _guarded_cache(dw.v_cache)
    k0 = dw.k_cache.clone()
    newp = Guarded((bsz,), torch.int32)
    binding.commit_kv(dw.k_tree, dw.v_tree, path, alen, dw.prefix_len, kc.view, vc.view,
                      new_prefix_len=newp.view)
    newp.check("new_prefix_len")
    kc.check("k_cache")
    vc.check("v_cache")
    own = torch.from_numpy(_owned_rows(alen.cpu().numpy(), path.cpu().numpy(),
                                       dw.wl.prefix_len, cap, bsz)).cuda()
    keep = ~own[:, None, :, None].expand_as(k0)
    assert torch.equal(_bits(kc.view)[keep], _bits(k0)[keep])
