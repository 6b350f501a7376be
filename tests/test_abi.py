"""The built library loads and exports every function include/*.h declares
(no GPU needed: nothing is called that touches a device)."""

import ctypes
import glob
import os
import re

import pytest

from tree_verification_attention_tv_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"\b(tv_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_four_calls():
    names = declared_functions()
    for fn in ("tv_build_tree_mask", "tv_tree_attention", "tv_greedy_accept", "tv_commit_kv",
               "tv_tree_attention_workspace_size", "tv_greedy_accept_workspace_size",
               "tv_status_string", "tv_version"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libtreeverify.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(binding.library_path())
    missing = [fn for fn in declared_functions() if not hasattr(lib, fn)]
    assert not missing, f"not exported: {missing}"


def test_host_only_entry_points():
    assert binding.version() == 100
    assert binding.status_string(0) == "TV_OK"
    assert "NULL" in binding.status_string(1)
    assert binding.accept_workspace_size(1, 60, 128256) > 0
    assert binding.accept_workspace_size(1, 0, 128256) == 0
    assert binding.accept_workspace_size(1, 257, 128256) == 0


def test_null_and_shape_errors_enqueue_nothing():
    L = binding.lib()
    # null parents -> TV_ERR_NULL; zero nodes -> TV_ERR_SHAPE (no device work)
    assert L.tv_build_tree_mask(None, 1, 8, None, None, None, None) == 1
    assert L.tv_build_tree_mask(ctypes.c_void_p(16), 1, 0, ctypes.c_void_p(16), None, None,
                                None) == 2
    assert L.tv_build_tree_mask(ctypes.c_void_p(16), 1, 257, ctypes.c_void_p(16), None, None,
                                None) == 2
    d = binding.AttnDesc(batch=1, n_nodes=8, n_q_heads=4, n_kv_heads=1, head_dim=96,
                         cache_capacity=64, max_prefix_len=32)
    assert L.tv_tree_attention(ctypes.byref(d), None, None, 0, None, None) == 3
    d.head_dim, d.n_q_heads, d.n_kv_heads = 128, 6, 4
    assert L.tv_tree_attention(ctypes.byref(d), None, None, 0, None, None) == 2
    # commit with unsupported head_dim
    p = ctypes.c_void_p(256)
    assert L.tv_commit_kv(p, p, p, p, p, p, p, p, 0, 64, 1, 8, 1, 80, None, None) == 3
    # accept: row stride below vocab
    assert L.tv_greedy_accept(p, 0, 100, 50, p, p, 1, 8, p, p, p, p, p, 1 << 20, None,
                              None) == 2


def test_attention_descriptor_tree_placement_is_validated():
    # descriptor checks come before the pointer checks: a valid descriptor with
    # null pointers gives TV_ERR_NULL, an invalid placement TV_ERR_SHAPE
    L = binding.lib()
    d = binding.AttnDesc(batch=1, n_nodes=60, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         cache_capacity=1088, max_prefix_len=1000)
    for placement in (binding.TREE_AUTO, binding.TREE_OWN_WORKGROUP, binding.TREE_IN_LAST_SPLIT):
        d.tree_placement = placement
        assert L.tv_tree_attention(ctypes.byref(d), None, None, 0, None, None) == 1
    d.tree_placement = 3
    assert L.tv_tree_attention(ctypes.byref(d), None, None, 0, None, None) == 2
    d.tree_placement, d.kernel = 0, 3
    assert L.tv_tree_attention(ctypes.byref(d), None, None, 0, None, None) == 2
    for k in (binding.KERNEL_AUTO, binding.KERNEL_SPLIT16, binding.KERNEL_WIDE):
        d.kernel = k
        assert L.tv_tree_attention(ctypes.byref(d), None, None, 0, None, None) == 1


def test_header_declares_the_selection_calls():
    names = declared_functions()
    for fn in ("tv_block_summaries", "tv_select_blocks", "tv_select_blocks_workspace_size"):
        assert fn in names


def test_selection_host_checks_enqueue_nothing():
    L = binding.lib()
    p = ctypes.c_void_p(256)
    # summaries: null cache, unsupported head_dim, zero block size, bad stride
    assert L.tv_block_summaries(None, 0, 64, 1, 1, 128, 16, p, None, 64, p, None, None) == 1
    assert L.tv_block_summaries(p, 0, 64, 1, 1, 96, 16, p, None, 64, p, None, None) == 3
    assert L.tv_block_summaries(p, 0, 64, 1, 1, 128, 0, p, None, 64, p, None, None) == 2
    assert L.tv_block_summaries(p, 8, 64, 1, 1, 128, 16, p, None, 64, p, None, None) == 2
    assert L.tv_block_summaries(p, 0, 64, 0, 1, 128, 16, p, None, 64, p, None, None) == 0

    def desc(**kw):
        base = dict(batch=1, n_nodes=60, n_q_heads=32, n_kv_heads=8, head_dim=128,
                    cache_capacity=60096, max_prefix_len=60000, block_size=16, n_sink_blocks=2,
                    n_window_blocks=8, top_k=246, reduction=binding.REDUCE_MEAN,
                    max_blocks=256, reserved=0)
        base.update(kw)
        return binding.SelectDesc(**base)

    def call(d, ptr=None):
        return L.tv_select_blocks(ctypes.byref(d), ptr, ptr, ptr, ptr, ptr, None, ptr, 1 << 20,
                                  None, None)

    assert call(desc()) == 1                                   # valid, null pointers
    assert call(desc(max_blocks=255)) == 2                     # list cannot hold the selection
    assert call(desc(reduction=3)) == 2
    assert call(desc(head_dim=96)) == 3
    assert call(desc(block_size=0)) == 2
    assert call(desc(top_k=-1)) == 2
    assert call(desc(max_prefix_len=60097)) == 2
    assert call(desc(reserved=1)) == 2
    assert call(desc(n_q_heads=130, n_kv_heads=2, reduction=binding.REDUCE_MAX)) == 3
    assert call(desc(n_q_heads=130, n_kv_heads=2, reduction=binding.REDUCE_MEAN)) == 1
    assert L.tv_select_blocks(None, p, p, p, p, p, None, p, 1 << 20, None, None) == 1


def test_stochastic_accept_host_checks():
    L = binding.lib()
    names = declared_functions()
    assert "tv_stochastic_accept" in names and "tv_stochastic_accept_workspace_size" in names
    p = ctypes.c_void_p(256)
    assert binding.stochastic_accept_workspace_size(2, 60, 128256) > 0
    assert binding.stochastic_accept_workspace_size(1, 0, 128256) == 0
    args = lambda t: (p, 0, 100, 100, p, p, 1, 8, t, 1, 2, 3, p, p, p, p, 1 << 20, None, None)  # noqa
    assert L.tv_stochastic_accept(*args(0.0)) == 2
    assert L.tv_stochastic_accept(*args(-1.0)) == 2
    assert L.tv_stochastic_accept(*args(float("inf"))) == 2
    assert L.tv_stochastic_accept(*args(float("nan"))) == 2
    assert L.tv_stochastic_accept(None, 0, 100, 100, p, p, 1, 8, 1.0, 1, 2, 3, p, p, p, p,
                                  1 << 20, None, None) == 1
    assert L.tv_stochastic_accept(p, 0, 100, 50, p, p, 1, 8, 1.0, 1, 2, 3, p, p, p, p, 1 << 20,
                                  None, None) == 2


def test_attention_needs_exactly_one_of_mask_and_parents():
    L = binding.lib()
    d = binding.AttnDesc(batch=1, n_nodes=8, n_q_heads=4, n_kv_heads=1, head_dim=128,
                         cache_capacity=64, max_prefix_len=32)
    p = 256
    ptrs = binding.AttnPtrs(q=p, k_tree=p, v_tree=p, k_cache=p, v_cache=p, prefix_len=p,
                            mask=None, out=p, parents=None)
    assert L.tv_tree_attention(ctypes.byref(d), ctypes.byref(ptrs), ctypes.c_void_p(p), 1 << 20,
                               None, None) == 1
    ptrs.mask, ptrs.parents = p, p
    assert L.tv_tree_attention(ctypes.byref(d), ctypes.byref(ptrs), ctypes.c_void_p(p), 1 << 20,
                               None, None) == 2


def test_multi_layer_commit_host_checks():
    L = binding.lib()
    names = declared_functions()
    assert "tv_commit_kv_layers" in names and "tv_greedy_accept_commit_layers" in names
    p = ctypes.c_void_p(256)
    a, b = ctypes.c_void_p(4096), ctypes.c_void_p(8192)

    def commit(n_layers, ts, cs, prefix=a, new_prefix=b):
        return L.tv_commit_kv_layers(p, p, p, p, prefix, new_prefix, p, p, 0, 64, 2, 8, 1, 128,
                                     n_layers, ts, cs, None, None)
    assert commit(0, 1024, 8192) == 2                       # no layers
    assert commit(binding.MAX_LAYERS + 1, 1024, 8192) == 2  # too many
    assert commit(2, 1020, 8192) == 2                       # tree stride not whole vectors
    assert commit(2, 1024, 0) == 2                          # zero cache stride
    assert commit(2, 1024, 8192, a, a) == 3                 # new_prefix_len aliases prefix_len
    assert commit(2, 1024, 8192, a, ctypes.c_void_p(4100)) == 3  # partial overlap
    assert L.tv_commit_kv_layers(p, p, p, p, a, b, p, p, 0, 64, 1, 8, 1, 80, 2, 1024, 8192,
                                 None, None) == 3           # head_dim
    assert L.tv_commit_kv_layers(None, p, p, p, a, b, p, p, 0, 64, 1, 8, 1, 128, 2, 1024, 8192,
                                 None, None) == 1

    def accept_commit(n_layers, ts, cs, new_prefix=b):
        return L.tv_greedy_accept_commit_layers(
            p, 0, 100, 100, p, p, 1, 8, p, p, p, p, p, 1 << 20, p, p, a, new_prefix, p, p, 0, 64,
            1, 128, n_layers, ts, cs, None, None)
    assert accept_commit(0, 1024, 8192) == 2
    assert accept_commit(3, 1024, 8188) == 2
    assert accept_commit(3, 1024, 8192, a) == 3


def test_filtered_stochastic_accept_host_checks():
    L = binding.lib()
    assert "tv_stochastic_accept_filtered" in declared_functions()
    p = ctypes.c_void_p(256)

    def call(k, top_p, temp=1.0):
        return L.tv_stochastic_accept_filtered(p, 0, 100, 100, p, p, 1, 8, temp, k, top_p, 1, 2,
                                               3, p, p, p, p, 1 << 20, None, None)
    assert call(-1, 1.0) == 2
    assert call(0, 0.0) == 2
    assert call(0, 1.5) == 2
    assert call(0, float("nan")) == 2
    assert call(20, 0.95, temp=0.0) == 2


def test_binding_constants_match_the_header():
    text = open(os.path.join(ROOT, "include", "treeverify.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(TV_\w+)\s+(\d+)", text)}
    assert defs["TV_ATTN_WS_COUNTER_BYTES"] == binding.ATTN_WS_COUNTER_BYTES
    assert defs["TV_DERR_SYNC"] == binding.DERR_SYNC
    assert defs["TV_ATTN_NOALLOC_SCRATCH_BYTES"] == binding.ATTN_NOALLOC_SCRATCH_BYTES
    assert defs["TV_STREAM_READ_SINK_WORDS"] == binding.STREAM_READ_SINK_WORDS
    enums = dict(re.findall(r"(TV_ATTN_KERNEL_\w+)\s*=\s*(\d+)", text))
    assert [int(enums[k]) for k in ("TV_ATTN_KERNEL_AUTO", "TV_ATTN_KERNEL_SPLIT16", "TV_ATTN_KERNEL_WIDE")] == \
        [binding.KERNEL_AUTO, binding.KERNEL_SPLIT16, binding.KERNEL_WIDE]

