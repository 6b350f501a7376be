"""A whole verify step captured in a HIP graph replays to the eager results.

The library only launches kernels (no memset, no allocation), so the four
calls can be captured.  The graph is replayed several times, with eager work
and synchronisation between the replays, and every replay is compared bit for
bit with an eager step on an identical copy of the inputs.
"""

import pytest
import torch

from tree_verification_attention_tv_amd import binding
from tree_verification_attention_tv_amd import workloads as W

from .gpu_util import DevWorkload

pytestmark = pytest.mark.gpu


class _Step:
    """Inputs (a private device copy) and preallocated outputs of one step."""

    def __init__(self, wl):
        self.dw = DevWorkload(wl)
        dw = self.dw
        b, n = wl.parents.shape
        dev = dw.q.device
        self.mask = torch.empty((b, n, (n + 31) // 32), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(dw.q)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.acc = tuple(torch.empty(s, dtype=torch.int32, device=dev)
                         for s in ((b, n), (b,), (b, n), (b,)))
        self.new_prefix = torch.empty_like(dw.prefix_len)
        desc = binding.attn_desc(dw.q, dw.k_cache, max_prefix_len=wl.max_prefix_len)
        self.ws_attn = binding.attention_workspace(desc, dev)
        self.ws_acc = torch.empty(binding.accept_workspace_size(b, n, wl.vocab), dtype=torch.uint8,
                                  device=dev)

    fused = False

    def run(self):
        dw, wl = self.dw, self.dw.wl
        b, n = wl.parents.shape
        if self.fused:   # the attention builds and writes the mask itself
            binding.tree_attention(dw.q, dw.k_cache, dw.v_cache, dw.k_tree, dw.v_tree,
                                   dw.prefix_len, None, max_prefix_len=wl.max_prefix_len,
                                   out=self.out, workspace=self.ws_attn, dev_err=self.err,
                                   parents=dw.parents, mask_out=self.mask)
        else:
            st = binding.lib().tv_build_tree_mask(binding._ptr(dw.parents), b, n,
                                                  binding._ptr(self.mask), None,
                                                  binding._ptr(self.err),
                                                  binding._stream(dw.q.device))
            assert st == 0
            binding.tree_attention(dw.q, dw.k_cache, dw.v_cache, dw.k_tree, dw.v_tree,
                                   dw.prefix_len, self.mask, max_prefix_len=wl.max_prefix_len,
                                   out=self.out, workspace=self.ws_attn, dev_err=self.err)
        if self.fused:   # acceptance and the commit of its path in one call
            binding.greedy_accept_commit(dw.logits, dw.parents, dw.draft, dw.k_tree, dw.v_tree,
                                         dw.prefix_len, dw.k_cache, dw.v_cache,
                                         new_prefix_len=self.new_prefix, workspace=self.ws_acc,
                                         dev_err=self.err, outputs=self.acc)
        else:
            binding.greedy_accept(dw.logits, dw.parents, dw.draft, workspace=self.ws_acc,
                                  dev_err=self.err, outputs=self.acc)
            binding.commit_kv(dw.k_tree, dw.v_tree, self.acc[2], self.acc[1], dw.prefix_len,
                              dw.k_cache, dw.v_cache, new_prefix_len=self.new_prefix,
                              dev_err=self.err)

    def results(self):
        return [self.mask, self.out.view(torch.int16), *self.acc, self.new_prefix,
                self.dw.k_cache.view(torch.int16), self.dw.v_cache.view(torch.int16), self.err]

    def scramble(self):
        # outputs overwritten with junk by eager kernels, outside the graph
        for t in (self.mask, self.out.view(torch.int16), *self.acc, self.new_prefix):
            t.fill_(-7)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["8b_layer", "batched"])
def test_step_graph_replays_match_eager(name, fused):
    print(f"[graph] {name} step capture and replay (mask and commit fused: {fused})",
          flush=True)
    wl = W.make_workload(name)
    eager, graphed = _Step(wl), _Step(wl)
    eager.fused = graphed.fused = fused
    eager.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in eager.results()]
    assert int(eager.err.item()) == 0

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    torch.cuda.synchronize()

    for rep in range(4):
        graphed.scramble()
        eager.run()              # eager library work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip(graphed.results(), ref)):
            assert torch.equal(got, want), f"replay {rep}: output {k} differs from the eager step"
    _replay_vs_oracle(graphed, wl)


def _replay_vs_oracle(step, wl):
    # the last replay's outputs against the oracle itself, not only the eager run
    import numpy as np

    import oracle

    from .gpu_util import bf16_host, check_attention_close, oracle_attention
    r_mask, _ = oracle.build_mask(wl.parents)
    assert np.array_equal(step.mask.cpu().numpy().view(np.uint32), r_mask)
    ref_o, _ = oracle_attention(wl)
    check_attention_close(step.out, ref_o, "graph replay")
    r_amax, r_alen, r_path, r_bonus = oracle.greedy_accept(wl.logits, wl.parents, wl.draft_tokens)
    for got, want in zip(step.acc, (r_amax, r_alen, r_path, r_bonus)):
        assert np.array_equal(got.cpu().numpy(), want)
    rk, rv, rp = oracle.commit_kv(wl.k_tree, wl.v_tree, r_path, r_alen, wl.prefix_len,
                                  wl.k_cache, wl.v_cache)
    assert np.array_equal(step.new_prefix.cpu().numpy(), rp)
    assert np.array_equal(bf16_host(step.dw.k_cache), rk)
    assert np.array_equal(bf16_host(step.dw.v_cache), rv)
    assert int(step.err.item()) == 0


def test_specpv_step_graph_replays_match_eager():
    """select -> mask -> partial attention over the selected blocks -> accept
    -> commit -> summary update, captured once and replayed."""
    print("[graph] SpecPV step capture and replay", flush=True)
    bs, n_sink, n_window, top_k = 16, 2, 4, 20
    wl = W.make_select_case(81, batch=2, n_nodes=24, hq=8, hkv=2, d=128,
                            prefix_lens=[1500, 977], block_size=bs, n_planted=4)

    class SpecStep(_Step):
        def __init__(self):
            super().__init__(wl)
            dw = self.dw
            # records past the prefix are never written: start them equal
            self.summ = torch.zeros(binding.summaries_shape(dw.k_cache, bs),
                                    dtype=torch.bfloat16, device="cuda")
            binding.block_summaries(dw.k_cache, dw.prefix_len, block_size=bs,
                                    summaries=self.summ)
            self.sel = (torch.empty((2, n_sink + n_window + top_k), dtype=torch.int32,
                                    device="cuda"),
                        torch.empty((2,), dtype=torch.int32, device="cuda"))
            self.ws_sel = torch.empty(binding.select_workspace_size(binding.select_desc(
                dw.q, self.summ, cache_capacity=wl.capacity, max_prefix_len=wl.max_prefix_len,
                block_size=bs, n_sink=n_sink, n_window=n_window, top_k=top_k)),
                dtype=torch.uint8, device="cuda")
            self.desc = binding.attn_desc(dw.q, dw.k_cache, max_prefix_len=wl.max_prefix_len,
                                          block_size=bs, max_blocks=n_sink + n_window + top_k)
            self.ws_attn = binding.attention_workspace(self.desc, "cuda")

        def run(self):
            dw = self.dw
            b, n = wl.parents.shape
            binding.select_blocks(dw.q, self.summ, dw.prefix_len, cache_capacity=wl.capacity,
                                  max_prefix_len=wl.max_prefix_len, block_size=bs,
                                  n_sink=n_sink, n_window=n_window, top_k=top_k,
                                  outputs=self.sel, workspace=self.ws_sel, dev_err=self.err)
            st = binding.lib().tv_build_tree_mask(binding._ptr(dw.parents), b, n,
                                                  binding._ptr(self.mask), None,
                                                  binding._ptr(self.err),
                                                  binding._stream(dw.q.device))
            assert st == 0
            binding.tree_attention(dw.q, dw.k_cache, dw.v_cache, dw.k_tree, dw.v_tree,
                                   dw.prefix_len, self.mask, max_prefix_len=wl.max_prefix_len,
                                   block_idx=self.sel[0], n_blocks=self.sel[1], block_size=bs,
                                   out=self.out, workspace=self.ws_attn, dev_err=self.err)
            binding.greedy_accept(dw.logits, dw.parents, dw.draft, workspace=self.ws_acc,
                                  dev_err=self.err, outputs=self.acc)
            binding.commit_kv(dw.k_tree, dw.v_tree, self.acc[2], self.acc[1], dw.prefix_len,
                              dw.k_cache, dw.v_cache, new_prefix_len=self.new_prefix,
                              dev_err=self.err)
            binding.block_summaries(dw.k_cache, self.new_prefix, block_size=bs,
                                    first_token=dw.prefix_len, max_tokens=n,
                                    summaries=self.summ, dev_err=self.err)

        def results(self):
            return super().results() + [*self.sel, self.summ.view(torch.int16)]

        def scramble(self):
            super().scramble()
            for t in self.sel:
                t.fill_(-7)

    eager, graphed = SpecStep(), SpecStep()
    eager.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in eager.results()]
    assert int(eager.err.item()) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    torch.cuda.synchronize()
    for rep in range(4):
        graphed.scramble()
        eager.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip(graphed.results(), ref)):
            assert torch.equal(got, want), f"replay {rep}: output {k} differs from the eager step"


def test_multi_layer_and_filtered_calls_replay_to_eager():
    """Three layers' attention, the layer-batched acceptance and commit, and
    a filtered sampling call, captured once and replayed."""
    print("[graph] multi-layer step and filtered sampling, capture and replay", flush=True)
    import numpy as np
    layers = 3
    wl = W.make_random_case(91, batch=2, n_nodes=30, hq=8, hkv=2, d=128, prefix_lens=[700, 333],
                            vocab=3000, p_match=0.7)
    rng = np.random.default_rng(91)

    def bf(a):
        return torch.from_numpy(W.f32_to_bf16_bits(a.astype(np.float32)).view(np.int16)).cuda() \
            .view(torch.bfloat16)

    class Layered:
        def __init__(self):
            self.dw = DevWorkload(wl)
            b, n = wl.parents.shape
            cap = wl.capacity
            self.q = bf(rng.standard_normal((layers,) + wl.q.shape) * 0.1)
            self.kt = bf(rng.standard_normal((layers, b, n, 2, 128)))
            self.vt = bf(rng.standard_normal((layers, b, n, 2, 128)))
            self.kc = bf(rng.standard_normal((layers, b, 2, cap, 128)))
            self.vc = bf(rng.standard_normal((layers, b, 2, cap, 128)))
            self.out = torch.empty_like(self.q)
            self.mask = torch.empty((b, n, 1), dtype=torch.int32, device="cuda")
            self.err = torch.zeros(1, dtype=torch.int32, device="cuda")
            self.acc = tuple(torch.empty(s, dtype=torch.int32, device="cuda")
                             for s in ((b, n), (b,), (b, n), (b,)))
            self.sto = tuple(torch.empty(s, dtype=torch.int32, device="cuda")
                             for s in ((b,), (b, n), (b,)))
            self.new_prefix = torch.empty_like(self.dw.prefix_len)
            desc = binding.attn_desc(self.q[0], self.kc[0], max_prefix_len=wl.max_prefix_len)
            self.ws_attn = binding.attention_workspace(desc, "cuda")
            self.ws_acc = torch.empty(binding.accept_workspace_size(b, n, wl.vocab),
                                      dtype=torch.uint8, device="cuda")
            self.ws_sto = torch.empty(binding.stochastic_accept_workspace_size(b, n, wl.vocab),
                                      dtype=torch.uint8, device="cuda")

        def run(self):
            dw = self.dw
            for l in range(layers):
                binding.tree_attention(self.q[l], self.kc[l], self.vc[l], self.kt[l], self.vt[l],
                                       dw.prefix_len, None, max_prefix_len=wl.max_prefix_len,
                                       out=self.out[l], workspace=self.ws_attn, dev_err=self.err,
                                       parents=dw.parents, mask_out=self.mask if l == 0 else None)
            binding.greedy_accept_commit_layers(dw.logits, dw.parents, dw.draft, self.kt, self.vt,
                                                dw.prefix_len, self.kc, self.vc,
                                                new_prefix_len=self.new_prefix,
                                                workspace=self.ws_acc, dev_err=self.err,
                                                outputs=self.acc)
            binding.stochastic_accept_filtered(dw.logits, dw.parents, dw.draft, 0.6, top_k=20,
                                               top_p=0.95, seed=(4, 5), step=1,
                                               workspace=self.ws_sto, dev_err=self.err,
                                               outputs=self.sto)

        def results(self):
            return [self.mask, self.out.view(torch.int16), *self.acc, *self.sto, self.new_prefix,
                    self.kc.view(torch.int16), self.vc.view(torch.int16), self.err]

        def scramble(self):
            for t in (self.mask, self.out.view(torch.int16), *self.acc, *self.sto,
                      self.new_prefix):
                t.fill_(-7)

    eager = Layered()
    rng = np.random.default_rng(91)   # identical inputs for the graphed copy
    graphed = Layered()
    eager.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in eager.results()]
    assert int(eager.err.item()) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    torch.cuda.synchronize()
    for rep in range(4):
        graphed.scramble()
        eager.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip(graphed.results(), ref)):
            assert torch.equal(got, want), f"replay {rep}: output {k} differs from the eager step"
