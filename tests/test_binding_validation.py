"""Host-side operand checks of the Python binding (no GPU needed).

The binding raises ValueError/TypeError on a malformed operand before any
launch: a wrong shape there would otherwise become an out-of-bounds device
access.  The validators are pure functions of shapes, dtypes, strides and
devices, so they run here on CPU tensors; the GPU suite repeats a few of the
cases through the public calls.
"""

import pytest
import torch

from tree_verification_attention_tv_amd import binding as B

bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32


def attn_ops(b=2, n=5, hq=8, hkv=2, d=64, cap=96):
    return dict(
        q=torch.zeros(b, n, hq, d, dtype=bf),
        k_cache=torch.zeros(b, hkv, cap, d, dtype=bf),
        v_cache=torch.zeros(b, hkv, cap, d, dtype=bf),
        k_tree=torch.zeros(b, n, hkv, d, dtype=bf),
        v_tree=torch.zeros(b, n, hkv, d, dtype=bf),
        prefix_len=torch.zeros(b, dtype=i32),
        mask=torch.zeros(b, n, (n + 31) // 32, dtype=i32),
    )


def call_attn(ops, **kw):
    B.validate_attention(ops["q"], ops["k_cache"], ops["v_cache"], ops["k_tree"], ops["v_tree"],
                         ops["prefix_len"], ops["mask"], **kw)


def test_attention_good_operands_pass():
    ops = attn_ops()
    call_attn(ops)
    call_attn(ops, out=torch.zeros_like(ops["q"]), lse=torch.zeros(2, 5, 8, dtype=f32),
              block_idx=torch.zeros(2, 3, dtype=i32), n_blocks=torch.zeros(2, dtype=i32),
              workspace=torch.zeros(16, dtype=torch.uint8), dev_err=torch.zeros(1, dtype=i32))
    ops["mask"] = None
    call_attn(ops, parents=torch.zeros(2, 5, dtype=i32), mask_out=torch.zeros(2, 5, 1, dtype=i32),
              depth_out=torch.zeros(2, 5, dtype=i32))


@pytest.mark.parametrize("field,bad", [
    ("k_tree", torch.zeros(2, 4, 2, 64, dtype=bf)),      # N differs from q
    ("v_tree", torch.zeros(2, 5, 1, 64, dtype=bf)),      # Hkv differs from the cache
    ("mask", torch.zeros(2, 5, 2, dtype=i32)),           # too many words
    ("mask", torch.zeros(1, 5, 1, dtype=i32)),           # batch
    ("prefix_len", torch.zeros(3, dtype=i32)),
    ("prefix_len", torch.zeros(2, 1, dtype=i32)),
    ("v_cache", torch.zeros(2, 2, 80, 64, dtype=bf)),    # capacity differs from k_cache
    ("k_cache", torch.zeros(2, 3, 96, 64, dtype=bf)),    # Hq % Hkv != 0
    ("k_cache", torch.zeros(2, 2, 96, 32, dtype=bf)),    # head_dim differs from q
])
def test_attention_bad_shape_raises(field, bad):
    ops = attn_ops()
    ops[field] = bad
    with pytest.raises(ValueError):
        call_attn(ops)


@pytest.mark.parametrize("kw", [
    dict(out=torch.zeros(2, 5, 8, 32, dtype=bf)),
    dict(out=torch.zeros(2, 5, 8, 64, dtype=f32)),
    dict(out=torch.zeros(2, 5, 64, 8, dtype=bf).transpose(2, 3)),   # not contiguous
    dict(lse=torch.zeros(2, 5, 4, dtype=f32)),
    dict(lse=torch.zeros(2, 5, 8, dtype=bf)),
    dict(block_idx=torch.zeros(1, 3, dtype=i32), n_blocks=torch.zeros(2, dtype=i32)),
    dict(block_idx=torch.zeros(2, 3, dtype=i32), n_blocks=torch.zeros(1, dtype=i32)),
    dict(block_idx=torch.zeros(2, 3, dtype=i32)),                   # n_blocks missing
    dict(workspace=torch.zeros(4, 4, dtype=torch.uint8)),
    dict(workspace=torch.zeros(16, dtype=f32)),
    dict(dev_err=torch.zeros(0, dtype=i32)),
    dict(dev_err=torch.zeros(1, dtype=f32)),
])
def test_attention_bad_outputs_raise(kw):
    with pytest.raises(ValueError):
        call_attn(attn_ops(), **kw)


def test_attention_parent_form_shapes():
    ops = attn_ops()
    ops["mask"] = None
    for kw in (dict(parents=torch.zeros(2, 4, dtype=i32)),
               dict(parents=torch.zeros(2, 5, dtype=i32), mask_out=torch.zeros(2, 5, 2, dtype=i32)),
               dict(parents=torch.zeros(2, 5, dtype=i32), depth_out=torch.zeros(5, dtype=i32))):
        with pytest.raises(ValueError):
            call_attn(ops, **kw)


def test_cache_rows_must_be_contiguous():
    ops = attn_ops()
    big = torch.zeros(2, 2, 96, 128, dtype=bf)
    ops["k_cache"] = big[..., :64]            # rows strided
    ops["v_cache"] = big[..., 64:]
    with pytest.raises(ValueError):
        call_attn(ops)


def test_accept_checks():
    bsz, n, v = 2, 6, 50
    logits = torch.zeros(bsz, n, v, dtype=bf)
    parents = torch.zeros(bsz, n, dtype=i32)
    draft = torch.zeros(bsz, n, dtype=i32)
    outs = (torch.zeros(bsz, n, dtype=i32), torch.zeros(bsz, dtype=i32),
            torch.zeros(bsz, n, dtype=i32), torch.zeros(bsz, dtype=i32))
    B.validate_accept(logits, parents, draft, None, outs)
    B.validate_accept(logits, parents, draft, v, outs)
    B.validate_accept(logits[:, :, :40], parents, draft, 40, outs)    # strided rows are allowed
    bad_cases = [
        (logits, parents, torch.zeros(bsz, n - 1, dtype=i32), None, outs),   # draft shape
        (logits, parents, draft, v + 1, outs),                             # vocab past the row
        (logits, parents, draft, 0, outs),
        (torch.zeros(bsz, n + 1, v, dtype=bf), parents, draft, None, outs),  # N differs
        (logits.transpose(1, 2), parents, draft, None, None),              # vocab stride != 1
        (logits, parents, draft, None, outs[:3]),
        (logits, parents, draft, None, (outs[0], outs[1], torch.zeros(bsz, n + 1, dtype=i32),
                                        outs[3])),
        (logits, parents, draft, None, (outs[0], torch.zeros(bsz, dtype=torch.int64), outs[2],
                                        outs[3])),
        (logits, torch.zeros(bsz * n, dtype=i32), draft, None, None),       # parents not 2-D
    ]
    for args in bad_cases:
        with pytest.raises(ValueError):
            B.validate_accept(*args)
    # stochastic outputs: (accept_len, accept_path, bonus)
    B.validate_accept(logits, parents, draft, None, outs[1:], n_outputs=3)
    with pytest.raises(ValueError):
        B.validate_accept(logits, parents, draft, None, outs[:3], n_outputs=3)


def test_commit_checks():
    bsz, n, hkv, d, cap = 2, 7, 2, 64, 40
    kt = torch.zeros(bsz, n, hkv, d, dtype=bf)
    kc = torch.zeros(bsz, hkv, cap, d, dtype=bf)
    plen = torch.zeros(bsz, dtype=i32)
    path = torch.zeros(bsz, n, dtype=i32)
    B.validate_commit(kt, kt.clone(), kc, kc.clone(), plen, accept_path=path, accept_len=plen,
                      new_prefix_len=plen)
    bad = [
        dict(k_tree=torch.zeros(bsz, n, hkv + 1, d, dtype=bf)),
        dict(v_tree=torch.zeros(bsz, n - 1, hkv, d, dtype=bf)),
        dict(accept_path=torch.zeros(bsz, n + 1, dtype=i32)),
        dict(accept_len=torch.zeros(bsz + 1, dtype=i32)),
        dict(prefix_len=torch.zeros(bsz, dtype=torch.int64)),
        dict(new_prefix_len=torch.zeros(1, dtype=i32)),
        dict(v_cache=torch.zeros(bsz, hkv, cap + 1, d, dtype=bf)),
        dict(k_tree=torch.zeros(bsz, n, hkv, d // 2, dtype=bf)),
    ]
    for over in bad:
        args = dict(k_tree=kt, v_tree=kt.clone(), k_cache=kc, v_cache=kc.clone(), prefix_len=plen,
                    accept_path=path, accept_len=plen, new_prefix_len=plen)
        args.update(over)
        with pytest.raises((ValueError, TypeError)):
            B.validate_commit(args.pop("k_tree"), args.pop("v_tree"), args.pop("k_cache"),
                              args.pop("v_cache"), args.pop("prefix_len"), **args)
