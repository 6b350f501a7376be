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
    d.tree_placement, d.reserved = 0, 1
    assert L.tv_tree_attention(ctypes.byref(d), None, None, 0, None, None) == 2
