"""Helpers shared by the GPU tests: moving seeded workloads to the device and
comparing with the oracle."""

import numpy as np
import torch

import oracle
from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W

ATOL, RTOL = 2e-2, 1e-2   # bf16 attention output contract (allclose form)


def dev_bf16(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def dev_i32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def bf16_host(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(t):
    return W.bf16_bits_to_f32(bf16_host(t)).astype(np.float64)


class DevWorkload:
    """Device copies of one workload's tensors (bit-identical to the host)."""

    def __init__(self, wl: W.Workload, device="cuda"):
        self.wl = wl
        self.q = dev_bf16(wl.q, device)
        self.k_tree = dev_bf16(wl.k_tree, device)
        self.v_tree = dev_bf16(wl.v_tree, device)
        self.k_cache = dev_bf16(wl.k_cache, device)
        self.v_cache = dev_bf16(wl.v_cache, device)
        self.prefix_len = dev_i32(wl.prefix_len, device)
        self.parents = dev_i32(wl.parents, device)
        self.draft = dev_i32(wl.draft_tokens, device)
        if wl.logits_dtype == "bf16":
            self.logits = dev_bf16(wl.logits, device)
        else:
            self.logits = torch.from_numpy(wl.logits).to(device)
        self.block_idx = None if wl.block_idx is None else dev_i32(wl.block_idx, device)
        self.n_blocks = None if wl.n_blocks is None else dev_i32(wl.n_blocks, device)

    def attention(self, mask, partial=False, **kw):
        wl = self.wl
        return binding.tree_attention(
            self.q, self.k_cache, self.v_cache, self.k_tree, self.v_tree, self.prefix_len, mask,
            max_prefix_len=wl.max_prefix_len,
            block_idx=self.block_idx if partial else None,
            n_blocks=self.n_blocks if partial else None,
            block_size=wl.block_size if partial else 0, **kw)


def oracle_attention(wl, partial=False, **kw):
    mask, _ = oracle.build_mask(wl.parents)
    return oracle.tree_attention(
        wl.q, wl.k_cache, wl.v_cache, wl.k_tree, wl.v_tree, wl.prefix_len, mask,
        block_idx=wl.block_idx if partial else None,
        n_blocks=wl.n_blocks if partial else None,
        block_size=wl.block_size if partial else None, **kw)


def check_attention_close(got_bf16, ref, label=""):
    got = bf16_to_f64(got_bf16)
    assert got.shape == ref.shape, label
    assert np.all(np.isfinite(got)), f"{label}: non-finite output (poisoned KV read?)"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (
        f"{label}: max err {err.max():.4g} at {worst} (ref {ref[worst]:.4g}, got {got[worst]:.4g})")
    # tripwire: error relative to the output scale
    rel = err.max() / max(np.abs(ref).max(), 1e-30)
    assert rel <= 1e-2, f"{label}: max_abs_err / max|ref| = {rel:.3g}"
    return err.max(), rel
