"""tv_tree_attention_noalloc (the workspace is the library's own device
array) against tv_tree_attention with a caller workspace: identical bits on
the same inputs, on two calls in a row with the second smaller, for both
schedules; an over-size descriptor is refused before any launch."""

import pytest
import torch

from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W

from .gpu_util import DevWorkload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _both(dw, kernel, partial=False):
    wl = dw.wl
    kw = dict(max_prefix_len=wl.max_prefix_len, kernel=kernel,
              block_idx=dw.block_idx if partial else None,
              n_blocks=dw.n_blocks if partial else None,
              block_size=wl.block_size if partial else 0)
    args = (dw.q, dw.k_cache, dw.v_cache, dw.k_tree, dw.v_tree, dw.prefix_len, None)
    err1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref, ref_lse = binding.tree_attention(*args, parents=dw.parents, want_lse=True, dev_err=err1,
                                          **kw)
    out = torch.full_like(dw.q, float("nan"))
    lse = torch.full(dw.q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.tree_attention_noalloc(*args, parents=dw.parents, out=out, lse=lse, dev_err=err2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "outputs differ"
    assert torch.equal(lse, ref_lse), "lse differs"
    assert int(err1.item()) == int(err2.item()) == 0


@pytest.mark.parametrize("kernel", [binding.KERNEL_SPLIT16, binding.KERNEL_WIDE])
def test_noalloc_matches_workspace_call_twice(kernel):
    # the 60000-token prefix first, then a smaller call reusing the same array
    for name, partial in (("long_context", False), ("8b_layer", False), ("long_context", True)):
        _say(f"[noalloc] kernel={kernel} {name} partial={partial}")
        _both(DevWorkload(W.make_workload(name)), kernel, partial)
    _say(f"[noalloc] kernel={kernel} small random case")
    wl = W.make_random_case(71, batch=3, n_nodes=9, hq=8, hkv=2, d=64, prefix_lens=[0, 77, 300])
    _both(DevWorkload(wl), kernel)


def test_noalloc_refuses_oversize_descriptor():
    _say("[noalloc] over-size descriptor")
    bsz, n, hq, hkv, d, cap = 128, 60, 32, 8, 128, 64
    q = torch.zeros(bsz, n, hq, d, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(bsz, hkv, cap, d, dtype=torch.bfloat16, device="cuda")
    kt = torch.zeros(bsz, n, hkv, d, dtype=torch.bfloat16, device="cuda")
    plen = torch.full((bsz,), cap, dtype=torch.int32, device="cuda")
    par = torch.arange(-1, n - 1, dtype=torch.int32, device="cuda").repeat(bsz, 1)
    desc = binding.attn_desc(q, kc, max_prefix_len=cap)
    assert binding.attention_workspace_size(desc) > binding.ATTN_NOALLOC_SCRATCH_BYTES
    out = torch.empty_like(q)
    with pytest.raises(binding.TVError) as info:
        binding.tree_attention_noalloc(q, kc, kc, kt, kt, plen, None, parents=par,
                                       max_prefix_len=cap, out=out)
    assert info.value.status == 4  # TV_ERR_WORKSPACE
