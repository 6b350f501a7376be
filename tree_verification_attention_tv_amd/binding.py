"""ctypes binding of libtreeverify for torch tensors.

Argument marshalling only: every step runs in the HIP library.  torch
supplies device memory (outputs and workspaces are allocated with torch) and
the current stream.  If the library is missing or a tensor is not on a GPU
the call raises -- there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtreeverify.so")
_lock = threading.Lock()
_lib = None

TV_BF16, TV_F32 = 0, 1
DERR_BAD_PARENT, DERR_BAD_BLOCK, DERR_CAPACITY, DERR_BAD_PREFIX, DERR_BAD_PATH = 1, 2, 4, 8, 16
DERR_SYNC = 32  # a merge of split partials waited past its bound
MAX_NODES = 256
MAX_LAYERS = 4096


class TVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_nodes", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32), ("max_prefix_len", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("num_splits", ctypes.c_int32),
        ("cache_seq_stride", ctypes.c_int64),
        ("tree_placement", ctypes.c_int32), ("kernel", ctypes.c_int32),
    ]


class AttnPtrs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_tree", ctypes.c_void_p), ("v_tree", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("prefix_len", ctypes.c_void_p), ("mask", ctypes.c_void_p),
        ("block_idx", ctypes.c_void_p), ("n_blocks", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("parents", ctypes.c_void_p), ("mask_out", ctypes.c_void_p),
        ("depth_out", ctypes.c_void_p),
    ]


class SelectDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_nodes", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32), ("max_prefix_len", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("n_sink_blocks", ctypes.c_int32),
        ("n_window_blocks", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("reduction", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


REDUCE_MEAN, REDUCE_MAX, REDUCE_LAST = 0, 1, 2
REDUCTIONS = {"mean": REDUCE_MEAN, "max": REDUCE_MAX, "last": REDUCE_LAST}
MAX_SELECT_GROUP = 64
MAX_SELECT_BLOCKS = 32768


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libtreeverify.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is not built; run `python -m "
                    "tree_verification_attention_tv_amd.build` (hipcc, gfx950)")
            L = ctypes.CDLL(_LIB_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            L.tv_build_tree_mask.argtypes = [vp, i32, i32, vp, vp, vp, vp]
            L.tv_build_tree_mask.restype = i32
            L.tv_tree_attention_workspace_size.argtypes = [ctypes.POINTER(AttnDesc)]
            L.tv_tree_attention_workspace_size.restype = sz
            L.tv_tree_attention_num_splits.argtypes = [ctypes.POINTER(AttnDesc)]
            L.tv_tree_attention_num_splits.restype = i32
            L.tv_tree_attention.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnPtrs),
                                            vp, sz, vp, vp]
            L.tv_tree_attention_noalloc.argtypes = [ctypes.POINTER(AttnDesc),
                                                    ctypes.POINTER(AttnPtrs), vp, vp]
            L.tv_tree_attention_noalloc.restype = i32
            L.tv_stream_read.argtypes = [vp, sz, vp, vp]
            L.tv_stream_read.restype = i32
            L.tv_tree_attention.restype = i32
            L.tv_greedy_accept_workspace_size.argtypes = [i32, i32, i64]
            L.tv_greedy_accept_workspace_size.restype = sz
            L.tv_greedy_accept.argtypes = [vp, i32, i64, i64, vp, vp, i32, i32, vp, vp, vp, vp,
                                           vp, sz, vp, vp]
            L.tv_greedy_accept.restype = i32
            L.tv_commit_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                       i32, vp, vp]
            L.tv_commit_kv.restype = i32
            L.tv_commit_kv_layers.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32,
                                              i32, i32, i32, i64, i64, vp, vp]
            L.tv_commit_kv_layers.restype = i32
            L.tv_block_summaries.argtypes = [vp, i64, i32, i32, i32, i32, i32, vp, vp, i32, vp,
                                             vp, vp]
            L.tv_block_summaries.restype = i32
            L.tv_select_blocks_workspace_size.argtypes = [ctypes.POINTER(SelectDesc)]
            L.tv_select_blocks_workspace_size.restype = sz
            L.tv_select_blocks.argtypes = [ctypes.POINTER(SelectDesc), vp, vp, vp, vp, vp, vp, vp,
                                           sz, vp, vp]
            L.tv_select_blocks.restype = i32
            L.tv_specpv_needs_rectification.argtypes = [i32, i32]
            L.tv_specpv_needs_rectification.restype = i32
            L.tv_specpv_rectify_tree.argtypes = [vp, i32, i32, vp, vp, i32, vp, vp]
            L.tv_specpv_rectify_tree.restype = i32
            L.tv_greedy_accept_commit.argtypes = [vp, i32, i64, i64, vp, vp, i32, i32, vp, vp,
                                                  vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, i64,
                                                  i32, i32, i32, vp, vp]
            L.tv_greedy_accept_commit.restype = i32
            L.tv_greedy_accept_commit_layers.argtypes = [
                vp, i32, i64, i64, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp,
                i64, i32, i32, i32, i32, i64, i64, vp, vp]
            L.tv_greedy_accept_commit_layers.restype = i32
            L.tv_stochastic_accept_workspace_size.argtypes = [i32, i32, i64]
            L.tv_stochastic_accept_workspace_size.restype = sz
            L.tv_stochastic_accept.argtypes = [vp, i32, i64, i64, vp, vp, i32, i32,
                                               ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_uint64, vp, vp, vp, vp, sz, vp, vp]
            L.tv_stochastic_accept.restype = i32
            L.tv_stochastic_accept_filtered.argtypes = [
                vp, i32, i64, i64, vp, vp, i32, i32, ctypes.c_float, i32, ctypes.c_float,
                ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp, vp, sz, vp, vp]
            L.tv_stochastic_accept_filtered.restype = i32
            L.tv_status_string.argtypes = [i32]
            L.tv_status_string.restype = ctypes.c_char_p
            L.tv_version.argtypes = []
            L.tv_version.restype = i32
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tv_status_string(int(status)).decode()


def version() -> int:
    return int(lib().tv_version())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_gpu(name, t, dtype=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device}); there is no CPU path")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(name, t, shape):
    """Raise ValueError unless tensor ``t`` has exactly ``shape``."""
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, "
                         f"got {tuple(t.shape)}")


def _same_device(ref, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the other operands on {ref.device}")


def _int_vec(name, t, n, dtype=torch.int32):
    """A contiguous int32 vector of n elements (None passes)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _shape(name, t, (n,))


def _workspace_ok(workspace, ref):
    if workspace is None:
        return
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    _same_device(ref, workspace=workspace)


def _dev_err_ok(dev_err, ref):
    if dev_err is None:
        return
    if dev_err.dtype != torch.int32 or dev_err.numel() < 1:
        raise ValueError("dev_err must be an int32 tensor with at least one element")
    _same_device(ref, dev_err=dev_err)


def _cache_rows(name, t, ref_shape):
    """A [B][Hkv][cap][D] cache with contiguous rows within a sequence."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B][Hkv][cap][D]")
    if tuple(t.shape) != tuple(ref_shape):
        raise ValueError(f"{name} must have shape {tuple(ref_shape)}, got {tuple(t.shape)}")
    _, hkv, cap, d = t.shape
    if t.stride()[1:] != (cap * d, d, 1):
        raise ValueError(f"{name} must have contiguous rows per sequence ([B][Hkv][cap][D])")


def validate_attention(q, k_cache, v_cache, k_tree, v_tree, prefix_len, mask, *, block_idx=None,
                       n_blocks=None, out=None, lse=None, parents=None, mask_out=None,
                       depth_out=None, workspace=None, dev_err=None):
    """Shape, dtype, layout and device checks of tv_tree_attention's operands
    against q [B][N][Hq][D] and k_cache [B][Hkv][cap][D]; raises before any
    launch.  (Pure: needs no GPU.)"""
    if q.dim() != 4:
        raise ValueError("q must be [B][N][Hq][D]")
    bsz, n, hq, d = q.shape
    if k_cache.dim() != 4 or k_cache.shape[0] != bsz or k_cache.shape[3] != d:
        raise ValueError(f"k_cache must be [B={bsz}][Hkv][cap][D={d}], got {tuple(k_cache.shape)}")
    hkv = k_cache.shape[1]
    if hkv < 1 or hq % hkv:
        raise ValueError(f"n_q_heads {hq} is not a multiple of n_kv_heads {hkv}")
    _cache_rows("k_cache", k_cache, k_cache.shape)
    _cache_rows("v_cache", v_cache, k_cache.shape)
    if v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must have the same strides")
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
        _shape(name, t, (bsz, n, hkv, d))
    _int_vec("prefix_len", prefix_len, bsz)
    w = (n + 31) // 32
    if mask is not None:
        _shape("mask", mask, (bsz, n, w))
    if parents is not None:
        _shape("parents", parents, (bsz, n))
    if mask_out is not None:
        _shape("mask_out", mask_out, (bsz, n, w))
    if depth_out is not None:
        _shape("depth_out", depth_out, (bsz, n))
    if (block_idx is None) != (n_blocks is None):
        raise ValueError("give both block_idx and n_blocks, or neither")
    if block_idx is not None:
        if block_idx.dim() != 2 or block_idx.shape[0] != bsz or block_idx.shape[1] < 1:
            raise ValueError(f"block_idx must be [B={bsz}][max_blocks >= 1]")
        _int_vec("n_blocks", n_blocks, bsz)
    if out is not None:
        if out.dtype != q.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous bf16 tensor")
        _shape("out", out, q.shape)
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 tensor")
        _shape("lse", lse, (bsz, n, hq))
    _workspace_ok(workspace, q)
    _dev_err_ok(dev_err, q)
    _same_device(q, k_cache=k_cache, v_cache=v_cache, k_tree=k_tree, v_tree=v_tree,
                 prefix_len=prefix_len, mask=mask, block_idx=block_idx, n_blocks=n_blocks,
                 out=out, lse=lse, parents=parents, mask_out=mask_out, depth_out=depth_out)


def validate_accept(logits, parents, draft_tokens, vocab=None, outputs=None, n_outputs=4):
    """Checks of the acceptance calls' operands: logits [B][N][V] with unit
    vocab stride and one row stride, parents and draft_tokens [B][N], the
    vocab override within the row, and the output tensors' shapes."""
    if parents.dim() != 2:
        raise ValueError("parents must be [B][N]")
    bsz, n = parents.shape
    _shape("draft_tokens", draft_tokens, (bsz, n))
    if logits.dim() != 3 or tuple(logits.shape[:2]) != (bsz, n) or logits.stride(2) != 1 or \
            (bsz > 1 and logits.stride(0) != n * logits.stride(1)):
        raise ValueError("logits must be [B][N][V] with unit vocab stride and uniform row stride")
    if vocab is not None and not (1 <= int(vocab) <= logits.shape[2]):
        raise ValueError(f"vocab {vocab} must be in [1, {logits.shape[2]}] (the logits row)")
    if outputs is not None:
        if len(outputs) != n_outputs:
            raise ValueError(f"outputs must hold {n_outputs} tensors")
        shapes = ([(bsz, n), (bsz,), (bsz, n), (bsz,)] if n_outputs == 4
                  else [(bsz,), (bsz, n), (bsz,)])
        names = (["target_argmax", "accept_len", "accept_path", "bonus_token"] if n_outputs == 4
                 else ["accept_len", "accept_path", "bonus_token"])
        for name, t, shp in zip(names, outputs, shapes):
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 tensor")
            _shape(name, t, shp)
            _same_device(parents, **{name: t})
    _same_device(parents, logits=logits, draft_tokens=draft_tokens)


def validate_commit(k_tree, v_tree, k_cache, v_cache, prefix_len, *, accept_path=None,
                    accept_len=None, new_prefix_len=None, n_nodes=None):
    """Checks of the commit operands: tree K/V [B][N][Hkv][D] contiguous,
    caches [B][Hkv][cap][D] with contiguous rows, and [B] / [B][N] int32
    vectors."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B][Hkv][cap][D]")
    bsz, hkv, cap, d = k_cache.shape
    _cache_rows("k_cache", k_cache, k_cache.shape)
    _cache_rows("v_cache", v_cache, k_cache.shape)
    if v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must have the same strides")
    if k_tree.dim() != 4:
        raise ValueError("k_tree must be [B][N][Hkv][D]")
    n = k_tree.shape[1] if n_nodes is None else n_nodes
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
        _shape(name, t, (bsz, n, hkv, d))
    _int_vec("prefix_len", prefix_len, bsz)
    _int_vec("accept_len", accept_len, bsz)
    _int_vec("new_prefix_len", new_prefix_len, bsz)
    if accept_path is not None:
        _shape("accept_path", accept_path, (bsz, n))
    _same_device(k_cache, k_tree=k_tree, v_tree=v_tree, v_cache=v_cache, prefix_len=prefix_len,
                 accept_path=accept_path, accept_len=accept_len, new_prefix_len=new_prefix_len)


def _check(fn, status):
    if status != 0:
        raise TVError(fn, status)


def _err_ptr(dev_err):
    if dev_err is None:
        return None
    _on_gpu("dev_err", dev_err, torch.int32)
    return _ptr(dev_err)


# ---------------------------------------------------------------------------
# public calls
# ---------------------------------------------------------------------------

def build_tree_mask(parents: torch.Tensor, *, dev_err=None, with_depth=True):
    """parents int32 [B][N] -> (mask int32 [B][N][W] holding uint32 bit
    patterns, depth int32 [B][N] or None)."""
    _on_gpu("parents", parents, torch.int32)
    if parents.dim() != 2:
        raise ValueError("parents must be [B][N]")
    _dev_err_ok(dev_err, parents)
    bsz, n = parents.shape
    w = (n + 31) // 32
    mask = torch.empty((bsz, n, w), dtype=torch.int32, device=parents.device)
    depth = torch.empty((bsz, n), dtype=torch.int32, device=parents.device) if with_depth else None
    _check("tv_build_tree_mask", lib().tv_build_tree_mask(
        _ptr(parents), bsz, n, _ptr(mask), _ptr(depth), _err_ptr(dev_err), _stream(parents.device)))
    return mask, depth


TREE_AUTO, TREE_OWN_WORKGROUP, TREE_IN_LAST_SPLIT = 0, 1, 2
KERNEL_AUTO, KERNEL_SPLIT16, KERNEL_WIDE = 0, 1, 2
ATTN_WS_COUNTER_BYTES = 32768  # merge counters at the start of an attention workspace


def attn_desc(q, k_cache, *, max_prefix_len, block_size=0, max_blocks=0, scale=0.0,
              num_splits=0, tree_placement=TREE_AUTO, kernel=KERNEL_AUTO) -> AttnDesc:
    bsz, n, hq, d = q.shape
    _, hkv, cap, d2 = k_cache.shape
    if d2 != d:
        raise ValueError("head_dim of q and the cache differ")
    return AttnDesc(batch=bsz, n_nodes=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                    cache_capacity=cap, max_prefix_len=int(max_prefix_len),
                    block_size=int(block_size), max_blocks=int(max_blocks),
                    softmax_scale=float(scale), num_splits=int(num_splits),
                    tree_placement=int(tree_placement), kernel=int(kernel),
                    cache_seq_stride=int(k_cache.stride(0)))


def attention_workspace_size(desc: AttnDesc) -> int:
    return int(lib().tv_tree_attention_workspace_size(ctypes.byref(desc)))


def attention_workspace(desc: AttnDesc, device) -> torch.Tensor:
    """A workspace for tv_tree_attention calls of `desc`, with the merge
    counters at its start zeroed as the call requires.  Reuse it for later
    calls (of any descriptor that fits) that do not overlap in time."""
    return torch.zeros(attention_workspace_size(desc), dtype=torch.uint8, device=device)


def attention_num_splits(desc: AttnDesc) -> int:
    return int(lib().tv_tree_attention_num_splits(ctypes.byref(desc)))


def _attention_args(q, k_cache, v_cache, k_tree, v_tree, prefix_len, mask, max_prefix_len,
                    block_idx, n_blocks, block_size, scale, num_splits, tree_placement, kernel,
                    out, lse, workspace, dev_err, parents, mask_out, depth_out):
    """Checks shared by the attention calls -> (desc, ptrs)."""
    bf = torch.bfloat16
    _on_gpu("q", q, bf)
    _on_gpu("k_cache", k_cache, bf)
    _on_gpu("v_cache", v_cache, bf)
    _on_gpu("k_tree", k_tree, bf)
    _on_gpu("v_tree", v_tree, bf)
    _on_gpu("prefix_len", prefix_len, torch.int32)
    if (mask is None) == (parents is None):
        raise ValueError("give exactly one of mask and parents")
    if mask is not None:
        _on_gpu("mask", mask, torch.int32)
    else:
        _on_gpu("parents", parents, torch.int32)
        for name, t in (("mask_out", mask_out), ("depth_out", depth_out)):
            if t is not None:
                _on_gpu(name, t, torch.int32)
    partial = block_idx is not None
    if partial:
        _on_gpu("block_idx", block_idx, torch.int32)
        _on_gpu("n_blocks", n_blocks, torch.int32)
    validate_attention(q, k_cache, v_cache, k_tree, v_tree, prefix_len, mask,
                       block_idx=block_idx, n_blocks=n_blocks, out=out, lse=lse, parents=parents,
                       mask_out=mask_out, depth_out=depth_out, workspace=workspace,
                       dev_err=dev_err)
    desc = attn_desc(q, k_cache, max_prefix_len=max_prefix_len,
                     block_size=block_size if partial else 0,
                     max_blocks=block_idx.shape[1] if partial else 0,
                     scale=scale, num_splits=num_splits, tree_placement=tree_placement,
                     kernel=kernel)
    ptrs = AttnPtrs(q=q.data_ptr(), k_tree=k_tree.data_ptr(), v_tree=v_tree.data_ptr(),
                    k_cache=k_cache.data_ptr(), v_cache=v_cache.data_ptr(),
                    prefix_len=prefix_len.data_ptr(),
                    mask=mask.data_ptr() if mask is not None else None,
                    block_idx=block_idx.data_ptr() if partial else None,
                    n_blocks=n_blocks.data_ptr() if partial else None,
                    out=out.data_ptr(), lse=lse.data_ptr() if lse is not None else None,
                    parents=parents.data_ptr() if parents is not None else None,
                    mask_out=mask_out.data_ptr() if mask_out is not None else None,
                    depth_out=depth_out.data_ptr() if depth_out is not None else None)
    return desc, ptrs


def tree_attention(q, k_cache, v_cache, k_tree, v_tree, prefix_len, mask, *, max_prefix_len,
                   block_idx=None, n_blocks=None, block_size=0, scale=0.0, num_splits=0,
                   tree_placement=TREE_AUTO, kernel=KERNEL_AUTO,
                   want_lse=False, out=None, lse=None, workspace=None, dev_err=None,
                   parents=None, mask_out=None, depth_out=None):
    """bf16 tree-masked GQA attention.  Returns out (and lse if asked).
    With mask=None and ``parents`` given, the kernel builds the tree mask
    itself and writes it to ``mask_out`` / ``depth_out`` when given."""
    if out is None:
        _on_gpu("q", q, torch.bfloat16)
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    desc, ptrs = _attention_args(q, k_cache, v_cache, k_tree, v_tree, prefix_len, mask,
                                 max_prefix_len, block_idx, n_blocks, block_size, scale,
                                 num_splits, tree_placement, kernel, out, lse, workspace, dev_err,
                                 parents, mask_out, depth_out)
    ws_bytes = attention_workspace_size(desc)
    if ws_bytes == 0:
        raise TVError("tv_tree_attention_workspace_size", 2)
    if workspace is None or workspace.numel() < ws_bytes:
        # the leading merge counters must start at zero; calls keep them so
        workspace = attention_workspace(desc, q.device)
    _check("tv_tree_attention", lib().tv_tree_attention(
        ctypes.byref(desc), ctypes.byref(ptrs), _ptr(workspace), workspace.numel(),
        _err_ptr(dev_err), _stream(q.device)))
    return (out, lse) if want_lse else out


ATTN_NOALLOC_SCRATCH_BYTES = 33554432  # the library's per-device workspace of the no-alloc call


def tree_attention_noalloc(q, k_cache, v_cache, k_tree, v_tree, prefix_len, mask, *,
                           max_prefix_len, out, lse=None, block_idx=None, n_blocks=None,
                           block_size=0, scale=0.0, num_splits=0, tree_placement=TREE_AUTO,
                           kernel=KERNEL_AUTO, dev_err=None, parents=None, mask_out=None,
                           depth_out=None):
    """tv_tree_attention_noalloc: as tree_attention, with the workspace the
    library's own device array, for callers that cannot allocate.  The
    outputs are the caller's (``out``, and ``lse`` if wanted); nothing is
    allocated here or in the call.  Calls on one device must not overlap."""
    if out is None:
        raise ValueError("out is required (the no-alloc call allocates nothing)")
    desc, ptrs = _attention_args(q, k_cache, v_cache, k_tree, v_tree, prefix_len, mask,
                                 max_prefix_len, block_idx, n_blocks, block_size, scale,
                                 num_splits, tree_placement, kernel, out, lse, None, dev_err,
                                 parents, mask_out, depth_out)
    _check("tv_tree_attention_noalloc", lib().tv_tree_attention_noalloc(
        ctypes.byref(desc), ctypes.byref(ptrs), _err_ptr(dev_err), _stream(q.device)))
    return out


STREAM_READ_SINK_WORDS = 2048


def stream_read(src, sink=None):
    """tv_stream_read over the bytes of a contiguous device tensor (a
    measurement aid: the read bandwidth the device reaches).  Returns sink."""
    if not (isinstance(src, torch.Tensor) and src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(STREAM_READ_SINK_WORDS, dtype=torch.int32, device=src.device)
    _on_gpu("sink", sink, torch.int32)
    if sink.numel() < STREAM_READ_SINK_WORDS:
        raise ValueError(f"sink must hold {STREAM_READ_SINK_WORDS} words")
    nbytes = src.numel() * src.element_size()
    _check("tv_stream_read", lib().tv_stream_read(_ptr(src), nbytes - nbytes % 16, _ptr(sink),
                                                  _stream(src.device)))
    return sink


def accept_workspace_size(batch, n_nodes, vocab) -> int:
    return int(lib().tv_greedy_accept_workspace_size(int(batch), int(n_nodes), int(vocab)))


def greedy_accept(logits, parents, draft_tokens, *, vocab=None, workspace=None, dev_err=None,
                  outputs=None):
    """logits [B][N][V] (bf16 or fp32; rows may be strided) ->
    (target_argmax [B][N], accept_len [B], accept_path [B][N], bonus [B]), int32."""
    _on_gpu("logits", logits, (torch.bfloat16, torch.float32), contiguous=False)
    _on_gpu("parents", parents, torch.int32)
    _on_gpu("draft_tokens", draft_tokens, torch.int32)
    validate_accept(logits, parents, draft_tokens, vocab, outputs)
    _workspace_ok(workspace, parents)
    _dev_err_ok(dev_err, parents)
    bsz, n = parents.shape
    v = logits.shape[2] if vocab is None else int(vocab)
    dt = TV_BF16 if logits.dtype == torch.bfloat16 else TV_F32
    dev = parents.device
    if outputs is None:
        outputs = (torch.empty((bsz, n), dtype=torch.int32, device=dev),
                   torch.empty((bsz,), dtype=torch.int32, device=dev),
                   torch.empty((bsz, n), dtype=torch.int32, device=dev),
                   torch.empty((bsz,), dtype=torch.int32, device=dev))
    amax, alen, path, bonus = outputs
    ws_bytes = accept_workspace_size(bsz, n, v)
    if ws_bytes == 0:
        raise TVError("tv_greedy_accept_workspace_size", 2)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check("tv_greedy_accept", lib().tv_greedy_accept(
        _ptr(logits), dt, v, int(logits.stride(1)), _ptr(parents), _ptr(draft_tokens), bsz, n,
        _ptr(amax), _ptr(alen), _ptr(path), _ptr(bonus), _ptr(workspace), workspace.numel(),
        _err_ptr(dev_err), _stream(dev)))
    return amax, alen, path, bonus


def greedy_accept_commit(logits, parents, draft_tokens, k_tree, v_tree, prefix_len, k_cache,
                         v_cache, *, new_prefix_len=None, vocab=None, workspace=None,
                         dev_err=None, outputs=None):
    """tv_greedy_accept then tv_commit_kv of its path, in one call.  Returns
    (target_argmax, accept_len, accept_path, bonus, new_prefix_len)."""
    _on_gpu("logits", logits, (torch.bfloat16, torch.float32), contiguous=False)
    _on_gpu("parents", parents, torch.int32)
    _on_gpu("draft_tokens", draft_tokens, torch.int32)
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
        _on_gpu(name, t, torch.bfloat16)
    _on_gpu("k_cache", k_cache, torch.bfloat16, contiguous=False)
    _on_gpu("v_cache", v_cache, torch.bfloat16, contiguous=False)
    _on_gpu("prefix_len", prefix_len, torch.int32)
    validate_accept(logits, parents, draft_tokens, vocab, outputs)
    bsz, n = parents.shape
    validate_commit(k_tree, v_tree, k_cache, v_cache, prefix_len, new_prefix_len=new_prefix_len,
                    n_nodes=n)
    _workspace_ok(workspace, parents)
    _dev_err_ok(dev_err, parents)
    _same_device(parents, k_cache=k_cache)
    _, hkv, cap, d = k_cache.shape
    v = logits.shape[2] if vocab is None else int(vocab)
    dt = TV_BF16 if logits.dtype == torch.bfloat16 else TV_F32
    dev = parents.device
    if outputs is None:
        outputs = (torch.empty((bsz, n), dtype=torch.int32, device=dev),
                   torch.empty((bsz,), dtype=torch.int32, device=dev),
                   torch.empty((bsz, n), dtype=torch.int32, device=dev),
                   torch.empty((bsz,), dtype=torch.int32, device=dev))
    amax, alen, path, bonus = outputs
    if new_prefix_len is None:
        new_prefix_len = torch.empty_like(prefix_len)
    ws_bytes = accept_workspace_size(bsz, n, v)
    if ws_bytes == 0:
        raise TVError("tv_greedy_accept_workspace_size", 2)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check("tv_greedy_accept_commit", lib().tv_greedy_accept_commit(
        _ptr(logits), dt, v, int(logits.stride(1)), _ptr(parents), _ptr(draft_tokens), bsz, n,
        _ptr(amax), _ptr(alen), _ptr(path), _ptr(bonus), _ptr(workspace), workspace.numel(),
        _ptr(k_tree), _ptr(v_tree), _ptr(prefix_len), _ptr(new_prefix_len), _ptr(k_cache),
        _ptr(v_cache), int(k_cache.stride(0)), cap, hkv, d, _err_ptr(dev_err), _stream(dev)))
    return amax, alen, path, bonus, new_prefix_len


def _layer_views(k_tree, v_tree, k_cache, v_cache):
    """Checks the [L][B][N][Hkv][D] tree and [L][B][Hkv][cap][D] cache views of
    the multi-layer calls; returns (layers, tree stride, cache stride,
    cache sequence stride) in elements."""
    bf = torch.bfloat16
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _on_gpu(name, t, bf, contiguous=False)
        if t.dim() != 5:
            raise ValueError(f"{name} must have a leading layer dimension")
    nl, bsz, n, hkv, d = k_tree.shape
    if v_tree.shape != k_tree.shape or v_tree.stride() != k_tree.stride() or \
            k_tree.stride()[1:] != (n * hkv * d, hkv * d, d, 1):
        raise ValueError("k_tree/v_tree must be [L][B][N][Hkv][D], contiguous within a layer")
    if k_cache.shape[:2] != (nl, bsz) or k_cache.shape[2] != hkv or k_cache.shape[4] != d:
        raise ValueError("caches must be [L][B][Hkv][cap][D] matching the tree")
    cap = k_cache.shape[3]
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride() or \
            k_cache.stride()[2:] != (cap * d, d, 1):
        raise ValueError("caches must have contiguous rows per (layer, sequence)")
    _same_device(k_tree, v_tree=v_tree, k_cache=k_cache, v_cache=v_cache)
    return nl, int(k_tree.stride(0)), int(k_cache.stride(0)), int(k_cache.stride(1))


def commit_kv_layers(k_tree, v_tree, accept_path, accept_len, prefix_len, k_cache, v_cache, *,
                     new_prefix_len=None, dev_err=None):
    """tv_commit_kv_layers: the same accepted rows into every layer's cache,
    one launch.  k_tree/v_tree [L][B][N][Hkv][D], caches [L][B][Hkv][cap][D]
    (layer and sequence strides free).  Returns new_prefix_len (a fresh
    tensor unless one is given; with L > 1 it may not be prefix_len)."""
    nl, t_stride, c_stride, seq_stride = _layer_views(k_tree, v_tree, k_cache, v_cache)
    for name, t in (("accept_path", accept_path), ("accept_len", accept_len),
                    ("prefix_len", prefix_len)):
        _on_gpu(name, t, torch.int32)
    _, bsz, n, hkv, d = k_tree.shape
    cap = k_cache.shape[3]
    _int_vec("accept_len", accept_len, bsz)
    _int_vec("prefix_len", prefix_len, bsz)
    _int_vec("new_prefix_len", new_prefix_len, bsz)
    _shape("accept_path", accept_path, (bsz, n))
    _dev_err_ok(dev_err, k_tree)
    _same_device(k_tree, accept_path=accept_path, accept_len=accept_len, prefix_len=prefix_len,
                 new_prefix_len=new_prefix_len)
    if new_prefix_len is None:
        new_prefix_len = torch.empty_like(prefix_len)
    _check("tv_commit_kv_layers", lib().tv_commit_kv_layers(
        _ptr(k_tree), _ptr(v_tree), _ptr(accept_path), _ptr(accept_len), _ptr(prefix_len),
        _ptr(new_prefix_len), _ptr(k_cache), _ptr(v_cache), seq_stride, cap, bsz, n, hkv, d,
        nl, t_stride, c_stride, _err_ptr(dev_err), _stream(k_cache.device)))
    return new_prefix_len


def greedy_accept_commit_layers(logits, parents, draft_tokens, k_tree, v_tree, prefix_len,
                                k_cache, v_cache, *, new_prefix_len=None, vocab=None,
                                workspace=None, dev_err=None, outputs=None):
    """tv_greedy_accept_commit_layers: acceptance, then the accepted rows
    into every layer's cache, in one call.  Tree and cache views as
    commit_kv_layers.  Returns (target_argmax, accept_len, accept_path,
    bonus, new_prefix_len)."""
    nl, t_stride, c_stride, seq_stride = _layer_views(k_tree, v_tree, k_cache, v_cache)
    _on_gpu("logits", logits, (torch.bfloat16, torch.float32), contiguous=False)
    _on_gpu("parents", parents, torch.int32)
    _on_gpu("draft_tokens", draft_tokens, torch.int32)
    _on_gpu("prefix_len", prefix_len, torch.int32)
    validate_accept(logits, parents, draft_tokens, vocab, outputs)
    bsz, n = parents.shape
    if k_tree.shape[1:3] != (bsz, n):
        raise ValueError("k_tree must be [L][B][N][Hkv][D] for the parents' B and N")
    _int_vec("prefix_len", prefix_len, bsz)
    _int_vec("new_prefix_len", new_prefix_len, bsz)
    _workspace_ok(workspace, parents)
    _dev_err_ok(dev_err, parents)
    _same_device(parents, k_tree=k_tree, prefix_len=prefix_len, new_prefix_len=new_prefix_len)
    _, _, _, hkv, d = k_tree.shape
    cap = k_cache.shape[3]
    v = logits.shape[2] if vocab is None else int(vocab)
    dt = TV_BF16 if logits.dtype == torch.bfloat16 else TV_F32
    dev = parents.device
    if outputs is None:
        outputs = (torch.empty((bsz, n), dtype=torch.int32, device=dev),
                   torch.empty((bsz,), dtype=torch.int32, device=dev),
                   torch.empty((bsz, n), dtype=torch.int32, device=dev),
                   torch.empty((bsz,), dtype=torch.int32, device=dev))
    amax, alen, path, bonus = outputs
    if new_prefix_len is None:
        new_prefix_len = torch.empty_like(prefix_len)
    ws_bytes = accept_workspace_size(bsz, n, v)
    if ws_bytes == 0:
        raise TVError("tv_greedy_accept_workspace_size", 2)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check("tv_greedy_accept_commit_layers", lib().tv_greedy_accept_commit_layers(
        _ptr(logits), dt, v, int(logits.stride(1)), _ptr(parents), _ptr(draft_tokens), bsz, n,
        _ptr(amax), _ptr(alen), _ptr(path), _ptr(bonus), _ptr(workspace), workspace.numel(),
        _ptr(k_tree), _ptr(v_tree), _ptr(prefix_len), _ptr(new_prefix_len), _ptr(k_cache),
        _ptr(v_cache), seq_stride, cap, hkv, d, nl, t_stride, c_stride, _err_ptr(dev_err),
        _stream(dev)))
    return amax, alen, path, bonus, new_prefix_len


def stochastic_accept_workspace_size(batch, n_nodes, vocab) -> int:
    return int(lib().tv_stochastic_accept_workspace_size(int(batch), int(n_nodes), int(vocab)))


def stochastic_accept(logits, parents, draft_tokens, temperature, *, seed=(0, 0), step=0,
                      vocab=None, workspace=None, dev_err=None, outputs=None):
    """Speculative sampling along the tree at temperature > 0 ->
    (accept_len [B], accept_path [B][N], bonus [B]), int32."""
    return _stochastic(logits, parents, draft_tokens, temperature, None, seed, step, vocab,
                       workspace, dev_err, outputs)


def stochastic_accept_filtered(logits, parents, draft_tokens, temperature, *, top_k=0,
                               top_p=1.0, seed=(0, 0), step=0, vocab=None, workspace=None,
                               dev_err=None, outputs=None):
    """tv_stochastic_accept_filtered: speculative sampling along the tree
    from the top-k / top-p filtered distributions (top_k = 0: off; top_p =
    1: off) -> (accept_len, accept_path, bonus)."""
    return _stochastic(logits, parents, draft_tokens, temperature, (int(top_k), float(top_p)),
                       seed, step, vocab, workspace, dev_err, outputs)


def _stochastic(logits, parents, draft_tokens, temperature, filt, seed, step, vocab, workspace,
                dev_err, outputs):
    _on_gpu("logits", logits, (torch.bfloat16, torch.float32), contiguous=False)
    _on_gpu("parents", parents, torch.int32)
    _on_gpu("draft_tokens", draft_tokens, torch.int32)
    validate_accept(logits, parents, draft_tokens, vocab, outputs, n_outputs=3)
    _workspace_ok(workspace, parents)
    _dev_err_ok(dev_err, parents)
    # temperature (finite, > 0) is checked by the library: TVError otherwise
    bsz, n = parents.shape
    v = logits.shape[2] if vocab is None else int(vocab)
    dt = TV_BF16 if logits.dtype == torch.bfloat16 else TV_F32
    dev = parents.device
    if outputs is None:
        outputs = (torch.empty((bsz,), dtype=torch.int32, device=dev),
                   torch.empty((bsz, n), dtype=torch.int32, device=dev),
                   torch.empty((bsz,), dtype=torch.int32, device=dev))
    alen, path, bonus = outputs
    ws_bytes = stochastic_accept_workspace_size(bsz, n, v)
    if ws_bytes == 0:
        raise TVError("tv_stochastic_accept_workspace_size", 2)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    mask64 = (1 << 64) - 1
    seeds = (int(seed[0]) & mask64, int(seed[1]) & mask64, int(step) & mask64)
    if filt is None:
        _check("tv_stochastic_accept", lib().tv_stochastic_accept(
            _ptr(logits), dt, v, int(logits.stride(1)), _ptr(parents), _ptr(draft_tokens), bsz, n,
            float(temperature), *seeds, _ptr(alen), _ptr(path), _ptr(bonus), _ptr(workspace),
            workspace.numel(), _err_ptr(dev_err), _stream(dev)))
    else:
        _check("tv_stochastic_accept_filtered", lib().tv_stochastic_accept_filtered(
            _ptr(logits), dt, v, int(logits.stride(1)), _ptr(parents), _ptr(draft_tokens), bsz, n,
            float(temperature), filt[0], filt[1], *seeds, _ptr(alen), _ptr(path), _ptr(bonus),
            _ptr(workspace), workspace.numel(), _err_ptr(dev_err), _stream(dev)))
    return alen, path, bonus


def commit_kv(k_tree, v_tree, accept_path, accept_len, prefix_len, k_cache, v_cache, *,
              new_prefix_len=None, dev_err=None):
    """Append the accepted rows to the caches in place; returns new_prefix_len
    (a fresh tensor unless one is given -- it may be prefix_len itself)."""
    bf = torch.bfloat16
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
        _on_gpu(name, t, bf)
    _on_gpu("k_cache", k_cache, bf, contiguous=False)
    _on_gpu("v_cache", v_cache, bf, contiguous=False)
    for name, t in (("accept_path", accept_path), ("accept_len", accept_len),
                    ("prefix_len", prefix_len)):
        _on_gpu(name, t, torch.int32)
    validate_commit(k_tree, v_tree, k_cache, v_cache, prefix_len, accept_path=accept_path,
                    accept_len=accept_len, new_prefix_len=new_prefix_len)
    _dev_err_ok(dev_err, k_cache)
    bsz, hkv, cap, d = k_cache.shape
    n = k_tree.shape[1]
    if new_prefix_len is None:
        new_prefix_len = torch.empty_like(prefix_len)
    _check("tv_commit_kv", lib().tv_commit_kv(
        _ptr(k_tree), _ptr(v_tree), _ptr(accept_path), _ptr(accept_len), _ptr(prefix_len),
        _ptr(new_prefix_len), _ptr(k_cache), _ptr(v_cache), int(k_cache.stride(0)), cap, bsz,
        n, hkv, d, _err_ptr(dev_err), _stream(k_cache.device)))
    return new_prefix_len


def summaries_shape(k_cache, block_size):
    """[B][Hkv][ceil(cap / block_size)][2][D] for a [B][Hkv][cap][D] cache."""
    bsz, hkv, cap, d = k_cache.shape
    return (bsz, hkv, (cap + block_size - 1) // block_size, 2, d)


def block_summaries(k_cache, prefix_len, *, block_size, first_token=None, max_tokens=None,
                    summaries=None, dev_err=None):
    """Element-wise max/min key records of the blocks holding rows in
    [first_token, prefix_len) (all blocks of the prefix when first_token is
    None).  Writes into ``summaries`` (allocated if None) and returns it."""
    _on_gpu("k_cache", k_cache, torch.bfloat16, contiguous=False)
    _on_gpu("prefix_len", prefix_len, torch.int32)
    if first_token is not None:
        _on_gpu("first_token", first_token, torch.int32)
    bsz, hkv, cap, d = k_cache.shape
    if k_cache.stride()[1:] != (cap * d, d, 1):
        raise ValueError("k_cache must be [B][Hkv][cap][D] with contiguous rows per sequence")
    if int(block_size) < 1:
        raise ValueError("block_size must be >= 1")
    _int_vec("prefix_len", prefix_len, bsz)
    _int_vec("first_token", first_token, bsz)
    _dev_err_ok(dev_err, k_cache)
    _same_device(k_cache, prefix_len=prefix_len, first_token=first_token, summaries=summaries)
    shape = summaries_shape(k_cache, block_size)
    if summaries is None:
        summaries = torch.empty(shape, dtype=torch.bfloat16, device=k_cache.device)
    _on_gpu("summaries", summaries, torch.bfloat16)
    if tuple(summaries.shape) != shape:
        raise ValueError(f"summaries must have shape {shape}")
    if max_tokens is None:
        max_tokens = cap
    _check("tv_block_summaries", lib().tv_block_summaries(
        _ptr(k_cache), int(k_cache.stride(0)), cap, bsz, hkv, d, int(block_size),
        _ptr(prefix_len), _ptr(first_token), int(max_tokens), _ptr(summaries),
        _err_ptr(dev_err), _stream(k_cache.device)))
    return summaries


def select_desc(q, summaries, *, cache_capacity, max_prefix_len, block_size, n_sink, n_window,
                top_k, reduction="mean", max_blocks=None) -> SelectDesc:
    bsz, n, hq, d = q.shape
    hkv = summaries.shape[1]
    if max_blocks is None:
        max_blocks = n_sink + n_window + top_k
    return SelectDesc(batch=bsz, n_nodes=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                      cache_capacity=int(cache_capacity), max_prefix_len=int(max_prefix_len),
                      block_size=int(block_size), n_sink_blocks=int(n_sink),
                      n_window_blocks=int(n_window), top_k=int(top_k),
                      reduction=REDUCTIONS[reduction], max_blocks=int(max_blocks), reserved=0)


def select_workspace_size(desc: SelectDesc) -> int:
    return int(lib().tv_select_blocks_workspace_size(ctypes.byref(desc)))


def select_blocks(q, summaries, prefix_len, *, cache_capacity, max_prefix_len, block_size,
                  n_sink, n_window, top_k, reduction="mean", max_blocks=None, want_scores=False,
                  outputs=None, scores=None, workspace=None, dev_err=None):
    """Score every block against the tree's queries and select sink + top-k +
    window.  Returns (block_idx int32 [B][max_blocks], n_blocks int32 [B]) and
    the fp32 scores [B][nb] when asked."""
    _on_gpu("q", q, torch.bfloat16)
    _on_gpu("summaries", summaries, torch.bfloat16)
    _on_gpu("prefix_len", prefix_len, torch.int32)
    bsz, n, hq, d = q.shape
    nb_cap = (int(cache_capacity) + int(block_size) - 1) // int(block_size)
    if summaries.dim() != 5 or tuple(summaries.shape) != (bsz, summaries.shape[1], nb_cap, 2, d):
        raise ValueError("summaries do not match q, cache_capacity and block_size")
    _int_vec("prefix_len", prefix_len, bsz)
    _workspace_ok(workspace, q)
    _dev_err_ok(dev_err, q)
    _same_device(q, summaries=summaries, prefix_len=prefix_len)
    desc = select_desc(q, summaries, cache_capacity=cache_capacity,
                       max_prefix_len=max_prefix_len, block_size=block_size, n_sink=n_sink,
                       n_window=n_window, top_k=top_k, reduction=reduction,
                       max_blocks=max_blocks)
    dev = q.device
    if outputs is None:
        outputs = (torch.empty((bsz, desc.max_blocks), dtype=torch.int32, device=dev),
                   torch.empty((bsz,), dtype=torch.int32, device=dev))
    block_idx, n_blocks = outputs
    _on_gpu("block_idx", block_idx, torch.int32)
    _on_gpu("n_blocks", n_blocks, torch.int32)
    if tuple(block_idx.shape) != (bsz, desc.max_blocks) or not block_idx.is_contiguous():
        raise ValueError("block_idx must be a contiguous [B][max_blocks] tensor")
    _int_vec("n_blocks", n_blocks, bsz)
    _same_device(q, block_idx=block_idx, n_blocks=n_blocks)
    if want_scores and scores is None:
        scores = torch.empty((bsz, nb_cap), dtype=torch.float32, device=dev)
    if scores is not None:
        _on_gpu("scores", scores, torch.float32)
        _shape("scores", scores, (bsz, nb_cap))
        _same_device(q, scores=scores)
    ws_bytes = select_workspace_size(desc)
    if ws_bytes == 0:
        raise TVError("tv_select_blocks_workspace_size", 2)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check("tv_select_blocks", lib().tv_select_blocks(
        ctypes.byref(desc), _ptr(q), _ptr(summaries), _ptr(prefix_len), _ptr(block_idx),
        _ptr(n_blocks), _ptr(scores), _ptr(workspace), workspace.numel(), _err_ptr(dev_err),
        _stream(dev)))
    return (block_idx, n_blocks, scores) if want_scores else (block_idx, n_blocks)


# ---------------------------------------------------------------------------
# SpecPV buffer policy (host functions of the library)
# ---------------------------------------------------------------------------

def _host_i32(name, a):
    import numpy as np
    arr = np.ascontiguousarray(a, dtype=np.int32)
    if arr.ndim != 1:
        raise ValueError(f"{name} must be one-dimensional")
    return arr


def specpv_needs_rectification(n_partial: int, buffer_size: int) -> bool:
    r = int(lib().tv_specpv_needs_rectification(int(n_partial), int(buffer_size)))
    if r < 0:
        raise TVError("tv_specpv_needs_rectification", 2)
    return r == 1


def specpv_rectify_tree(buffer_tokens, root_token, parents, draft_tokens):
    """Host arrays -> (parents, tokens) int32 numpy arrays of the rectifying
    tree: the buffered tokens as a chain, the current root, the draft tree."""
    import numpy as np
    buf = _host_i32("buffer_tokens", buffer_tokens)
    par = _host_i32("parents", parents)
    dr = _host_i32("draft_tokens", draft_tokens)
    if dr.shape != par.shape:
        raise ValueError("parents and draft_tokens differ in length")
    n = buf.shape[0] + par.shape[0]
    par_out = np.empty(n, dtype=np.int32)
    tok_out = np.empty(n, dtype=np.int32)
    c = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    _check("tv_specpv_rectify_tree", lib().tv_specpv_rectify_tree(
        c(buf), buf.shape[0], int(root_token), c(par), c(dr), par.shape[0], c(par_out),
        c(tok_out)))
    return par_out, tok_out
