"""Host-side driver of SpecPV partial verification for one sequence.

"SpecPV: Improving Self-Speculative Decoding for Long-Context Generation via
Partial Verification": partial verification attends to a selected subset of
the KV (Sec. 3.2); the tokens it accepts are partially verified and wait in a
buffer; when the buffer would overflow, a full verification re-checks them,
prepended to the new candidates, and the partial cache is refreshed
(Sec. 3.3; App. C and App. D for the sizes).

The driver keeps the bookkeeping (prefix lengths, buffered tokens, the
current root) and sequences the library calls.  Every step of the
computation runs in the HIP library: selection, mask, attention, acceptance,
commit and the summary update; the buffer rule and the rectifying tree come
from the library's host functions.  The model that produces queries, tree
K/V and logits for a step's tree is the caller's.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding


class SpecPVSequence:
    """Verification state of one sequence (batch 1).

    Cache rows [0, p_full) hold fully verified K/V, rows [p_full, p) the
    partially verified tokens in ``buffer`` (oldest first), and ``root`` is
    the last emitted token, whose K/V is not in the cache yet.
    """

    def __init__(self, k_cache, v_cache, prefix_len: int, root_token: int, *, block_size=16,
                 n_sink=2, n_window=8, top_k=246, buffer_size=20, reduction="mean",
                 max_nodes=binding.MAX_NODES):
        if k_cache.shape[0] != 1:
            raise ValueError("one sequence per driver (batch 1)")
        self.k_cache, self.v_cache = k_cache, v_cache
        self.dev = k_cache.device
        self.cap = k_cache.shape[2]
        self.bs, self.n_sink, self.n_window, self.top_k = block_size, n_sink, n_window, top_k
        self.buffer_size, self.reduction = buffer_size, reduction
        self.max_nodes = max_nodes
        self.p_full = self.p = int(prefix_len)
        self.buffer: list[int] = []
        self.root = int(root_token)
        self.err = torch.zeros(1, dtype=torch.int32, device=self.dev)
        self.summ = torch.zeros(binding.summaries_shape(k_cache, block_size), dtype=torch.bfloat16,
                                device=self.dev)
        binding.block_summaries(k_cache, self._i32([self.p]), block_size=block_size,
                                max_tokens=self.p, summaries=self.summ, dev_err=self.err)
        self.sel = (torch.empty((1, n_sink + n_window + top_k), dtype=torch.int32,
                                device=self.dev),
                    torch.empty((1,), dtype=torch.int32, device=self.dev))
        self.last = None

    def _i32(self, vals):
        return torch.tensor(list(vals), dtype=torch.int32, device=self.dev)

    # -- policy ------------------------------------------------------------
    def next_is_full(self) -> bool:
        """Whether the next step must be a rectifying full verification."""
        return binding.specpv_needs_rectification(len(self.buffer), self.buffer_size)

    def step_tree(self, parents, draft_tokens):
        """(parents, tokens, n_chain) of the tree the next step verifies,
        for a draft tree whose node 0 is the current root."""
        parents = np.asarray(parents, dtype=np.int32)
        draft = np.asarray(draft_tokens, dtype=np.int32).copy()
        if self.next_is_full() and self.buffer:
            par, tok = binding.specpv_rectify_tree(self.buffer, self.root, parents, draft)
            return par, tok, len(self.buffer)
        draft[0] = self.root
        return parents, draft, 0

    # -- one verification step -----------------------------------------------
    def verify(self, q, k_tree, v_tree, logits, parents, tokens, n_chain):
        """Run one step over the tree from ``step_tree`` with the caller's
        queries, tree K/V and logits for its nodes.  Returns a dict with the
        step kind, accept_len, the accepted path, the bonus token and the
        tokens whose rows were committed."""
        n = int(parents.shape[0])
        if n > self.max_nodes:
            raise ValueError("tree larger than max_nodes")
        full = n_chain > 0 or self.next_is_full()
        parents_d = self._i32(parents).view(1, n)
        tokens_d = self._i32(tokens).view(1, n)
        start = self.p_full if full else self.p
        start_d = self._i32([start])
        mask, _ = binding.build_tree_mask(parents_d, dev_err=self.err, with_depth=False)
        if full:
            out = binding.tree_attention(q, self.k_cache, self.v_cache, k_tree, v_tree, start_d,
                                         mask, max_prefix_len=start, dev_err=self.err)
        else:
            binding.select_blocks(q, self.summ, start_d, cache_capacity=self.cap,
                                  max_prefix_len=start, block_size=self.bs, n_sink=self.n_sink,
                                  n_window=self.n_window, top_k=self.top_k,
                                  reduction=self.reduction, outputs=self.sel, dev_err=self.err)
            out = binding.tree_attention(q, self.k_cache, self.v_cache, k_tree, v_tree, start_d,
                                         mask, max_prefix_len=start, block_idx=self.sel[0],
                                         n_blocks=self.sel[1], block_size=self.bs,
                                         dev_err=self.err)
        amax, alen, path, bonus = binding.greedy_accept(logits, parents_d, tokens_d,
                                                        dev_err=self.err)
        new_p = binding.commit_kv(k_tree, v_tree, path, alen, start_d, self.k_cache, self.v_cache,
                                  dev_err=self.err)
        binding.block_summaries(self.k_cache, new_p, block_size=self.bs, first_token=start_d,
                                max_tokens=n, summaries=self.summ, dev_err=self.err)
        a = int(alen.item())
        if int(self.err.item()) != 0:
            raise RuntimeError(f"device error bits {int(self.err.item())}")
        path_h = path.cpu().numpy()[0, :a + 1]
        committed = [int(tokens[i]) for i in path_h]
        if full:
            self.p_full = self.p = start + a + 1
            self.buffer = []
        else:
            self.p = start + a + 1
            self.buffer.extend(committed)
        self.root = int(bonus.item())
        self.last = dict(kind="full" if full else "partial", accept_len=a, path=path_h,
                         bonus=self.root, committed=committed, out=out, target_argmax=amax,
                         selected=None if full else
                         self.sel[0][0, :int(self.sel[1].item())].cpu().numpy())
        return self.last
