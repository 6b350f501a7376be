"""Benchmark of one tree-verify step on one MI355X.

A step is the whole hot path over one batch of synthetic input, back to back
on one stream: one layer of tree attention over the verified-prefix KV (its
tree workgroups build the tree mask from the parent array and write it out),
then greedy acceptance over the vocabulary with the KV commit of the
accepted path done by the same walk workgroups.  The standalone mask, accept
and commit calls are timed on their own in `call_us`.
Default workload: the 8B-layer shape (batch 1, 32 query / 8 KV heads of 128,
1000-token prefix, 60-node EAGLE-style tree, 128256-token bf16 logits).

Inputs are resident in HBM before the timed region.  To measure HBM rather
than cache bandwidth, the step rotates over enough independent copies of its
inputs that their total exceeds the 256 MB Infinity Cache.

Prints one JSON line (rank 0):
  value = microseconds per verify step (lower is better), the step replayed
  from a captured HIP graph (the same four calls; the eager time is reported
  beside it); KV GB/s; a roofline
  entry for the dominant call (HIP-event timing of its own launches on the
  stream they run on, algorithmic bytes, and the HBM traffic measured with
  rocprofv3 counters when those were taken on the current kernel source);
  the long-context (60K prefix) full and partial lines; a 32-layer step of
  the 8B shape (each layer's attention, then one layer-batched acceptance and
  commit, against per-layer commit launches); the fp64 CPU oracle timed on a
  bounded sample of the same workload.

Helper modes (used to produce the committed profile summaries):
  --copy-calibration      plain 256 MiB device copies, for scaling counters
  --pmc-summary F W CF CW rocprofv3 FETCH_SIZE / WRITE_SIZE directories (bench
                          run, copy run) -> traffic summary text on stdout
                          (with --workload: the workload those runs used)
  --trace-summary CSV CMD rocprofv3 kernel-stats CSV -> text summary on stdout
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure
STREAM_BYTES = 2 << 30          # buffer of the measured stream-read peak
MALL_BYTES = 256 * 1024 * 1024  # Infinity Cache
COPY_BYTES = 256 * 1024 * 1024  # calibration copy size
ATTN_SOURCES = [os.path.join(ROOT, "tree_verification_attention_tv_amd", "csrc", f)
                for f in ("tv_attention.hip", "tv_attn_wide.hip", "tv_attn_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_8b_layer_hbm_traffic.txt")
ATTN_KERNELS = ("attn_split_kernel", "attn_combine_kernel")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="8b_layer",
                    choices=["tiny", "8b_layer", "specblock_tree", "batched", "long_context"])
    ap.add_argument("--partial", action="store_true", help="partial-KV mode (long_context only)")
    ap.add_argument("--specpv", action="store_true",
                    help="long_context only: partial KV chosen each step by SpecPV block "
                         "selection (16-token blocks, 2 sink + 246 retrieved + 8 window blocks), "
                         "with the block summaries updated after the commit")
    ap.add_argument("--warm", action="store_true", help="no input rotation (cache-warm)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--kernel", default="auto", choices=["auto", "split16", "wide"],
                    help="attention schedule (auto: the planner's choice)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step with eager launches only (no HIP graph replay)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the long-context (60K prefix) full/partial lines")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device copies (for scaling HBM counters)")
    ap.add_argument("--pmc-summary", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE runs into a traffic text")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="condense rocprofv3 --pmc output directories (one per pass) into "
                         "per-kernel counters and MFMA / VALU / LDS ratios")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "COMMAND"),
                    help="condense a rocprofv3 kernel-stats CSV into a text summary")
    return ap.parse_args()


def source_hash() -> str:
    """Hash of the attention kernels' sources (both schedules and their
    shared header): a counter summary is current only for the same hash."""
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# measurement
# ---------------------------------------------------------------------------

class InputSet:
    """One device copy of every input and output of a step."""

    def __init__(self, wl, dev, torch, np):
        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

        self.q, self.k_tree, self.v_tree = bf(wl.q), bf(wl.k_tree), bf(wl.v_tree)
        self.k_cache, self.v_cache = bf(wl.k_cache), bf(wl.v_cache)
        self.prefix_len = i32(wl.prefix_len)
        self.parents, self.draft = i32(wl.parents), i32(wl.draft_tokens)
        self.logits = bf(wl.logits) if wl.logits_dtype == "bf16" else torch.from_numpy(wl.logits).to(dev)
        self.block_idx = None if wl.block_idx is None else i32(wl.block_idx)
        self.n_blocks = None if wl.n_blocks is None else i32(wl.n_blocks)
        b, n = wl.parents.shape
        self.mask = torch.empty((b, n, (n + 31) // 32), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        self.new_prefix = torch.empty_like(self.prefix_len)
        self.summ = self.sel_idx = self.sel_n = None

    def add_selection(self, binding, torch, bs, max_blocks):
        """Block summaries of the whole prefix (built here, untimed: they are
        kept from one step to the next) and the selected-list buffers."""
        b = self.prefix_len.shape[0]
        self.summ = binding.block_summaries(self.k_cache, self.prefix_len, block_size=bs)
        self.sel_idx = torch.empty((b, max_blocks), dtype=torch.int32, device=self.q.device)
        self.sel_n = torch.empty((b,), dtype=torch.int32, device=self.q.device)

    def nbytes(self):
        import torch
        return sum(t.numel() * t.element_size() for t in vars(self).values()
                   if isinstance(t, torch.Tensor))


class StepRunner:
    """The four library calls of one verify step, on torch's current stream."""

    def __init__(self, wl, partial, warm, num_splits, dev, specpv=False, kernel="auto"):
        import numpy as np
        import torch

        from tree_verification_attention_tv_amd import binding
        from tree_verification_attention_tv_amd import workloads as W

        self.specpv = specpv
        if specpv:
            partial = True
            wl = wl.without_blocks()
            wl.block_size = W.SPECPV_BLOCK_SIZE
            self.sel = dict(n_sink=W.SPECPV_SINK_BLOCKS, n_window=W.SPECPV_WINDOW_BLOCKS,
                            top_k=W.SPECPV_TOP_K)
            self.max_blocks = sum(self.sel.values())
        self.wl, self.partial, self.dev = wl, partial, dev
        self.binding = binding
        first = InputSet(wl, dev, torch, np)
        # at least three copies, and together 1.25x the Infinity Cache, so
        # that no call finds its inputs cached by the previous ones
        rot = 1 if warm else max(3, int(np.ceil(1.25 * MALL_BYTES / first.nbytes())))
        self.rot = min(rot, 64)
        self.sets = [first] + [InputSet(wl, dev, torch, np) for _ in range(self.rot - 1)]
        for i, st in enumerate(self.sets):
            st.gidx = i
            if specpv:
                st.add_selection(binding, torch, wl.block_size, self.max_blocks)
        self.graphs = []
        self.b, self.n = wl.parents.shape
        self.num_splits = num_splits
        self.kernel = {"auto": binding.KERNEL_AUTO, "split16": binding.KERNEL_SPLIT16,
                       "wide": binding.KERNEL_WIDE}[kernel]
        self.desc = binding.attn_desc(
            first.q, first.k_cache, max_prefix_len=wl.max_prefix_len,
            block_size=wl.block_size if partial else 0,
            max_blocks=(self.max_blocks if specpv else wl.max_blocks) if partial else 0,
            num_splits=num_splits, kernel=self.kernel)
        if specpv:
            self.sel_desc = binding.select_desc(
                first.q, first.summ, cache_capacity=wl.capacity,
                max_prefix_len=wl.max_prefix_len, block_size=wl.block_size, **self.sel)
            self.ws_sel = torch.empty(binding.select_workspace_size(self.sel_desc),
                                      dtype=torch.uint8, device=dev)
        self.ws_attn = binding.attention_workspace(self.desc, dev)
        self.ws_acc = torch.empty(binding.accept_workspace_size(self.b, self.n, wl.vocab),
                                  dtype=torch.uint8, device=dev)
        self.acc_out = (torch.empty((self.b, self.n), dtype=torch.int32, device=dev),
                        torch.empty((self.b,), dtype=torch.int32, device=dev),
                        torch.empty((self.b, self.n), dtype=torch.int32, device=dev),
                        torch.empty((self.b,), dtype=torch.int32, device=dev))
        self.ws_sto = torch.empty(binding.stochastic_accept_workspace_size(self.b, self.n, wl.vocab),
                                  dtype=torch.uint8, device=dev)
        self.sto_out = (torch.empty((self.b,), dtype=torch.int32, device=dev),
                        torch.empty((self.b, self.n), dtype=torch.int32, device=dev),
                        torch.empty((self.b,), dtype=torch.int32, device=dev))
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.per = 1                      # steps per captured graph
        self.one_per_graph_us = None      # step time with one step per graph
        self.one_per_graph_stats = None

    # -- the four calls ------------------------------------------------------
    def k_mask(self, s):
        bd = self.binding
        st = bd.lib().tv_build_tree_mask(bd._ptr(s.parents), self.b, self.n, bd._ptr(s.mask), None,
                                         bd._ptr(self.err), bd._stream(self.dev))
        if st:
            raise bd.TVError("tv_build_tree_mask", st)

    def k_select(self, s):
        self.binding.select_blocks(
            s.q, s.summ, s.prefix_len, cache_capacity=self.wl.capacity,
            max_prefix_len=self.wl.max_prefix_len, block_size=self.wl.block_size,
            outputs=(s.sel_idx, s.sel_n), workspace=self.ws_sel, dev_err=self.err, **self.sel)

    def k_summ_update(self, s):
        # the committed rows [prefix_len, new_prefix) enter the summaries
        self.binding.block_summaries(s.k_cache, s.new_prefix, block_size=self.wl.block_size,
                                     first_token=s.prefix_len, max_tokens=self.n,
                                     summaries=s.summ, dev_err=self.err)

    def k_summ_full(self, s):
        self.binding.block_summaries(s.k_cache, s.prefix_len, block_size=self.wl.block_size,
                                     max_tokens=self.wl.max_prefix_len, summaries=s.summ,
                                     dev_err=self.err)

    def k_attn(self, s):
        wl, p = self.wl, self.partial
        bidx, nblk = (s.sel_idx, s.sel_n) if self.specpv else (s.block_idx, s.n_blocks)
        # the tree mask (a1) is built by the attention's tree workgroups from
        # the parent array and written to s.mask
        self.binding.tree_attention(
            s.q, s.k_cache, s.v_cache, s.k_tree, s.v_tree, s.prefix_len, None,
            max_prefix_len=wl.max_prefix_len, block_idx=bidx if p else None,
            n_blocks=nblk if p else None, block_size=wl.block_size if p else 0,
            num_splits=self.num_splits, kernel=self.kernel, out=s.out, workspace=self.ws_attn,
            dev_err=self.err, parents=s.parents, mask_out=s.mask)

    def k_accept(self, s):
        self.binding.greedy_accept(s.logits, s.parents, s.draft, workspace=self.ws_acc,
                                   dev_err=self.err, outputs=self.acc_out)

    def k_accept_stochastic(self, s):
        # the same logits verified by sampling at T = 1 (counter-based uniforms)
        self.binding.stochastic_accept(s.logits, s.parents, s.draft, 1.0, seed=(1, 2), step=0,
                                       workspace=self.ws_sto, dev_err=self.err,
                                       outputs=self.sto_out)

    def k_accept_stochastic_filtered(self, s):
        # SpecPV App. D's sampling settings: T = 0.6, top-k 20, top-p 0.95
        self.binding.stochastic_accept_filtered(s.logits, s.parents, s.draft, 0.6, top_k=20,
                                                top_p=0.95, seed=(1, 2), step=0,
                                                workspace=self.ws_sto, dev_err=self.err,
                                                outputs=self.sto_out)

    def k_accept_stochastic_top_p(self, s):
        # SpecPV App. E's: T = 0.7, top-k off, top-p 0.9
        self.binding.stochastic_accept_filtered(s.logits, s.parents, s.draft, 0.7, top_k=0,
                                                top_p=0.9, seed=(1, 2), step=0,
                                                workspace=self.ws_sto, dev_err=self.err,
                                                outputs=self.sto_out)

    def k_accept_commit(self, s):
        # acceptance, and the commit of its path by the same walk workgroups
        self.binding.greedy_accept_commit(s.logits, s.parents, s.draft, s.k_tree, s.v_tree,
                                          s.prefix_len, s.k_cache, s.v_cache,
                                          new_prefix_len=s.new_prefix, workspace=self.ws_acc,
                                          dev_err=self.err, outputs=self.acc_out)

    def k_commit(self, s):
        self.binding.commit_kv(s.k_tree, s.v_tree, self.acc_out[2], self.acc_out[1], s.prefix_len,
                               s.k_cache, s.v_cache, new_prefix_len=s.new_prefix,
                               dev_err=self.err)

    def step(self, s):
        if self.specpv:
            self.k_select(s)
        self.k_attn(s)
        self.k_accept_commit(s)
        if self.specpv:
            self.k_summ_update(s)

    def capture(self, per=1):
        """HIP graphs of `per` whole steps each (the same calls and buffers
        as eager steps; no allocation or memset inside): graph g holds the
        steps on input sets g*per .. g*per + per - 1 (modulo the rotation),
        so consecutive steps never share an input set."""
        import torch
        torch.cuda.synchronize()
        self.graphs = []
        self.per = per
        for g in range(max(1, -(-self.rot // per))):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for j in range(per):
                    self.step(self.sets[(g * per + j) % self.rot])
            self.graphs.append(gr)
        torch.cuda.synchronize()

    def replay_steps(self, steps):
        """Replays covering `steps` steps (a multiple of the steps per graph)."""
        for k in range(steps // self.per):
            self.graphs[k % len(self.graphs)].replay()

    def timed_replays(self, steps):
        """Average GPU microseconds per step over `steps` steps of graph
        replays, from HIP events between the replays on the library's
        stream; the per-step times of each replay (its time over its steps)
        go to self.last_samples."""
        import torch
        n = steps // self.per
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for k in range(n):
            self.graphs[k % len(self.graphs)].replay()
            ev[k + 1].record(self.stream)
        torch.cuda.synchronize()
        self.last_samples = [ev[k].elapsed_time(ev[k + 1]) * 1e3 / self.per for k in range(n)]
        return ev[0].elapsed_time(ev[n]) * 1e3 / (n * self.per)

    # -- timing ----------------------------------------------------------------
    def timed(self, fn, iters):
        """Average microseconds of `fn` over `iters` back-to-back calls, from
        HIP events recorded on the stream the library launches on; the
        per-call times (an event between consecutive calls) go to
        self.last_samples."""
        import torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for k in range(iters):
            fn(self.sets[k % self.rot])
            ev[k + 1].record(self.stream)
        torch.cuda.synchronize()
        self.last_samples = [ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(iters)]
        return ev[0].elapsed_time(ev[iters]) * 1e3 / iters

    def timed_graph(self, fn, per_graph=20, reps=10):
        """Average microseconds of one call of `fn` on the GPU: `per_graph`
        calls over the rotated input copies captured in one HIP graph, whose
        replays are timed with HIP events on the library's stream.  No host
        launch overhead enters; the dispatch gaps between the graph's kernels
        do.  Per-call times of each replay go to self.last_samples."""
        import torch
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for k in range(per_graph):
                fn(self.sets[k % self.rot])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(self.stream)
        for k in range(reps):
            g.replay()
            ev[k + 1].record(self.stream)
        torch.cuda.synchronize()
        del g
        self.last_samples = [ev[k].elapsed_time(ev[k + 1]) * 1e3 / per_graph for k in range(reps)]
        return ev[0].elapsed_time(ev[reps]) * 1e3 / (reps * per_graph)

    def check_errors(self):
        if int(self.err.item()) != 0:
            print(f"device error bits {int(self.err.item())}", file=sys.stderr)
            sys.exit(1)

    def selection_bytes(self):
        """Algorithmic bytes of one selection call (summary records of every
        block of the prefix, the queries, per-KV-head partial scores written
        and read back, the list) and of one full summary build (the prefix
        keys read once, the records written)."""
        wl = self.wl
        b, n = self.b, self.n
        hq, hkv, d, bs = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.block_size
        nv = [(int(p) + bs - 1) // bs for p in wl.prefix_len]
        rec = hkv * 2 * d * 2
        sel = sum(nv) * rec + b * n * hq * d * 2 + 2 * sum(nv) * hkv * 4 + b * self.max_blocks * 4
        full = sum(int(p) for p in wl.prefix_len) * hkv * d * 2 + sum(nv) * rec
        return sel, full, nv if b > 1 else nv[0]

    def bytes(self):
        """Algorithmic bytes: visible prefix tokens, KV bytes, bytes of the
        attention call (KV, Q, O, mask) and of the acceptance (logits)."""
        wl = self.wl
        b, n = self.b, self.n
        hq, hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
        if self.partial:
            prefix_tokens = []
            if self.specpv:
                st = self.sets[0]
                lists = [st.sel_idx[s, :int(st.sel_n[s])].cpu().numpy() for s in range(b)]
            else:
                lists = [wl.block_idx[s, :int(wl.n_blocks[s])] for s in range(b)]
            for s in range(b):
                vis = 0
                for x in lists[s]:
                    lo = int(x) * wl.block_size
                    vis += max(0, min(wl.block_size, int(wl.prefix_len[s]) - lo))
                prefix_tokens.append(vis)
        else:
            prefix_tokens = [int(p) for p in wl.prefix_len]
        kv = (sum(prefix_tokens) + b * n) * hkv * d * 2 * 2   # K and V, bf16
        qo = 2 * b * n * hq * d * 2                            # Q read, O written
        mask = b * n * ((n + 31) // 32) * 4
        return prefix_tokens, kv, kv + qo + mask, wl.logits.nbytes


def measure(wl, partial, steps, warmup, warm, num_splits, dev, graph=True, specpv=False,
            kernel="auto"):
    """Returns (runner, step_us, wall_us, eager_step_us, calls).  step_us is
    the graph-replayed step when `graph` (several consecutive steps per
    graph; runner.one_per_graph_us holds the one-step-per-graph figure),
    else the eager one."""
    import torch
    r = StepRunner(wl, partial, warm, num_splits, dev, specpv=specpv, kernel=kernel)
    for k in range(warmup):
        r.step(r.sets[k % r.rot])
    torch.cuda.synchronize()
    r.check_errors()
    t0 = time.perf_counter()
    eager_us = r.timed(r.step, steps)
    wall_us = (time.perf_counter() - t0) * 1e6 / steps
    step_us = eager_us
    r.step_stats = spread(r.last_samples)
    if graph:
        # One step per graph first: each replay then also pays the start of
        # a graph (measured on MI355X: ~12 us at the 8B layer, more than a
        # dependent kernel's dispatch gap), a cost a serving loop shares
        # over everything it captures with the verify step.  Then the
        # reported figure: `per` consecutive steps per graph.
        r.capture(1)
        r.replay_steps(warmup)
        r.one_per_graph_us = r.timed_replays(steps)
        r.one_per_graph_stats = spread(r.last_samples)
        per = steps_per_graph(steps)
        r.capture(per)
        r.replay_steps(-(-warmup // per) * per)
        t0 = time.perf_counter()
        step_us = r.timed_replays(steps)
        wall_us = (time.perf_counter() - t0) * 1e6 / steps
        r.step_stats = spread(r.last_samples)
    # per-call GPU time from graph replays (eager back-to-back calls would
    # also measure the host's launch rate)
    tm0 = r.timed_graph if graph else (lambda fn, **kw: r.timed(fn, max(steps, 50)))
    r.call_stats = {}

    def tm(fn, name, **kw):
        v = tm0(fn, **kw)
        r.call_stats[name] = spread(r.last_samples)
        return v
    calls = {"mask": tm(r.k_mask, "mask"), "attention": tm(r.k_attn, "attention"),
             "accept": tm(r.k_accept, "accept"), "commit": tm(r.k_commit, "commit"),
             "accept_commit": tm(r.k_accept_commit, "accept_commit")}
    if not specpv and not partial:
        calls["accept_stochastic"] = tm(r.k_accept_stochastic, "accept_stochastic")
        calls["accept_stochastic_filtered"] = tm(r.k_accept_stochastic_filtered,
                                                 "accept_stochastic_filtered")
        calls["accept_stochastic_top_p"] = tm(r.k_accept_stochastic_top_p,
                                              "accept_stochastic_top_p")
    if specpv:
        calls["select"] = tm(r.k_select, "select")
        calls["summaries_update"] = tm(r.k_summ_update, "summaries_update")
        calls["summaries_full"] = tm(r.k_summ_full, "summaries_full", per_graph=5)
    r.check_errors()
    return r, step_us, wall_us, eager_us, calls


def steps_per_graph(steps, most=8):
    """Steps captured per HIP graph: the largest divisor of `steps` up to
    `most`, so that the timed replays cover exactly `steps` steps."""
    return max(d for d in range(1, min(most, steps) + 1) if steps % d == 0)


def spread(samples):
    """p10 / p50 / p90 of per-call microseconds."""
    import numpy as np
    q = np.percentile(np.asarray(samples, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(q[0]), 3), "p50": round(float(q[1]), 3),
            "p90": round(float(q[2]), 3)}


def attention_flops(wl, partial):
    """Algorithmic MFMA work of one attention call: per (sequence, node,
    query head) row and visible key, d multiply-adds for q.k and d for p.v
    (4 d flops); visible keys = the prefix (or its selected blocks) plus the
    node's ancestors and itself."""
    import numpy as np
    b, n = wl.parents.shape
    depth = np.zeros((b, n), dtype=np.int64)   # parents precede their children
    for i in range(1, n):
        depth[:, i] = depth[np.arange(b), wl.parents[:, i]] + 1
    total = 0
    for s in range(b):
        if partial:
            vis = 0
            for x in wl.block_idx[s, :int(wl.n_blocks[s])]:
                lo = int(x) * wl.block_size
                vis += max(0, min(wl.block_size, int(wl.prefix_len[s]) - lo))
        else:
            vis = int(wl.prefix_len[s])
        total += int(np.sum(vis + depth[s] + 1))
    return 4 * wl.head_dim * wl.n_q_heads * total


def secondary_line(name, partial, steps, dev, stream_gbps=None):
    import torch

    from tree_verification_attention_tv_amd import workloads as W
    wl = W.make_workload(name)
    r, step_us, _, eager_us, calls = measure(wl, partial, steps, 5, False, 0, dev)
    prefix_tokens, kv, attn_bytes, logit_bytes = r.bytes()
    gbps = attn_bytes / (calls["attention"] * 1e-6) / 1e9
    flops = attention_flops(wl, partial)
    tflops = flops / (calls["attention"] * 1e-6) / 1e12
    out = {
        "mode": "partial" if partial else "full",
        "batch": r.b, "n_nodes": r.n,
        "step_us": round(step_us, 3),
        "steps_per_graph": r.per,
        "step_us_one_per_graph": round(r.one_per_graph_us, 3),
        "step_us_spread": r.step_stats,
        "eager_step_us": round(eager_us, 3),
        "attention_us": round(calls["attention"], 3),
        "kv_bytes": kv,
        "attention_bytes": attn_bytes,
        "kv_gbps": round(kv / (calls["attention"] * 1e-6) / 1e9, 1),
        "attention_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "hbm_frac_of_measured_read": round(gbps / stream_gbps, 4) if stream_gbps else None,
        "attention_flops": flops,
        "attention_tflops": round(tflops, 1),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "accept_gbps": round(logit_bytes / (calls["accept"] * 1e-6) / 1e9, 1),
        "accept_hbm_frac": round(logit_bytes / (calls["accept"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "prefix_tokens": prefix_tokens if r.b <= 4 else [min(prefix_tokens), max(prefix_tokens)],
        "num_splits": r.binding.attention_num_splits(r.desc),
        "cache_rotation": r.rot,
        "call_us": {k: round(v, 3) for k, v in calls.items()},
        "call_us_spread": r.call_stats,
    }
    del r
    torch.cuda.empty_cache()
    return out


def specpv_line(steps, dev):
    """The long-context step with SpecPV selection: select -> mask -> partial
    attention over the selected blocks -> accept -> commit -> summary update."""
    import torch

    from tree_verification_attention_tv_amd import workloads as W
    wl = W.make_workload("long_context")
    r, step_us, _, eager_us, calls = measure(wl, True, steps, 5, False, 0, dev, specpv=True)
    prefix_tokens, kv, attn_bytes, _ = r.bytes()
    sel_bytes, sum_bytes, nv = r.selection_bytes()
    out = {
        "mode": "specpv_select",
        "step_us": round(step_us, 3),
        "steps_per_graph": r.per,
        "step_us_one_per_graph": round(r.one_per_graph_us, 3),
        "eager_step_us": round(eager_us, 3),
        "attention_us": round(calls["attention"], 3),
        "prefix_tokens": prefix_tokens,
        "blocks": nv,
        "select_bytes": sel_bytes,
        "select_gbps": round(sel_bytes / (calls["select"] * 1e-6) / 1e9, 1),
        "select_hbm_frac": round(sel_bytes / (calls["select"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "summaries_full_bytes": sum_bytes,
        "summaries_full_gbps": round(sum_bytes / (calls["summaries_full"] * 1e-6) / 1e9, 1),
        "summaries_full_hbm_frac": round(
            sum_bytes / (calls["summaries_full"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "attention_gbps": round(attn_bytes / (calls["attention"] * 1e-6) / 1e9, 1),
        "cache_rotation": r.rot,
        "call_us": {k: round(v, 3) for k, v in calls.items()},
    }
    del r
    torch.cuda.empty_cache()
    return out


def rectify_line(steps, dev):
    """SpecPV's rectifying full verification at the long-context shape: the
    tree is 21 buffered tokens (one more than the 20-token buffer) as a
    chain, the current root and the 60-node draft tree, verified with full
    attention over the 60000-token prefix."""
    import numpy as np
    import torch

    from tree_verification_attention_tv_amd import binding
    from tree_verification_attention_tv_amd import workloads as W
    base = W.make_workload("long_context")
    rng = np.random.Generator(np.random.PCG64(2024))
    chain = rng.integers(0, base.vocab, size=21)
    par, _ = binding.specpv_rectify_tree(chain, int(base.draft_tokens[0, 0]), base.parents[0],
                                         base.draft_tokens[0])
    wl = W.long_context_with_tree(par, "long_context_rectify")
    r, step_us, _, eager_us, calls = measure(wl, False, steps, 5, False, 0, dev)
    _, kv, attn_bytes, _ = r.bytes()
    out = {
        "mode": "specpv_rectify",
        "n_nodes": int(par.shape[0]),
        "step_us": round(step_us, 3),
        "steps_per_graph": r.per,
        "step_us_one_per_graph": round(r.one_per_graph_us, 3),
        "eager_step_us": round(eager_us, 3),
        "attention_us": round(calls["attention"], 3),
        "kv_gbps": round(kv / (calls["attention"] * 1e-6) / 1e9, 1),
        "hbm_frac": round(attn_bytes / (calls["attention"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "cache_rotation": r.rot,
        "call_us": {k: round(v, 3) for k, v in calls.items()},
    }
    del r
    torch.cuda.empty_cache()
    return out


def multi_layer_line(steps, dev, layers=32):
    """A verify step over all attention layers of the 8B shape (32 layers):
    each layer's tree attention over its own KV cache, then acceptance and
    the commit of the accepted rows into every layer's cache.  Fused: the
    layer-batched acceptance-and-commit call (one walk-and-copy launch for
    all layers).  Separate: acceptance, then one commit launch per layer.
    Both are captured in HIP graphs over two copies of the inputs (more than
    the Infinity Cache holds) and replayed."""
    import torch

    from tree_verification_attention_tv_amd import binding
    from tree_verification_attention_tv_amd import workloads as W
    wl = W.make_workload("8b_layer")
    b, n, hq, hkv, d = wl.batch, wl.n_nodes, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    cap = wl.capacity
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    bf = torch.bfloat16

    def rnd(*shape, scale=1.0):
        return (torch.randn(shape, generator=g, device=dev) * scale).to(bf)

    class LayerSet:
        def __init__(self):
            self.q = rnd(layers, b, n, hq, d, scale=d ** -0.5)
            self.k_tree = rnd(layers, b, n, hkv, d)
            self.v_tree = rnd(layers, b, n, hkv, d)
            self.k_cache = rnd(layers, b, hkv, cap, d)
            self.v_cache = rnd(layers, b, hkv, cap, d)
            self.out = torch.empty_like(self.q)
            self.logits = torch.from_numpy(wl.logits.view("int16")).to(dev).view(bf)
            self.parents = torch.from_numpy(wl.parents).to(dev)
            self.draft = torch.from_numpy(wl.draft_tokens).to(dev)
            self.prefix = torch.from_numpy(wl.prefix_len).to(dev)
            self.new_prefix = torch.empty_like(self.prefix)
            self.mask = torch.empty((b, n, (n + 31) // 32), dtype=torch.int32, device=dev)

    sets = [LayerSet(), LayerSet()]
    desc = binding.attn_desc(sets[0].q[0], sets[0].k_cache[0], max_prefix_len=wl.max_prefix_len)
    ws_attn = binding.attention_workspace(desc, dev)
    ws_acc = torch.empty(binding.accept_workspace_size(b, n, wl.vocab), dtype=torch.uint8,
                         device=dev)
    acc_out = (torch.empty((b, n), dtype=torch.int32, device=dev),
               torch.empty((b,), dtype=torch.int32, device=dev),
               torch.empty((b, n), dtype=torch.int32, device=dev),
               torch.empty((b,), dtype=torch.int32, device=dev))
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def attention(st):
        for l in range(layers):
            binding.tree_attention(
                st.q[l], st.k_cache[l], st.v_cache[l], st.k_tree[l], st.v_tree[l], st.prefix,
                None, max_prefix_len=wl.max_prefix_len, out=st.out[l], workspace=ws_attn,
                dev_err=err, parents=st.parents, mask_out=st.mask if l == 0 else None)

    def fused(st):
        attention(st)
        binding.greedy_accept_commit_layers(st.logits, st.parents, st.draft, st.k_tree,
                                            st.v_tree, st.prefix, st.k_cache, st.v_cache,
                                            new_prefix_len=st.new_prefix, workspace=ws_acc,
                                            dev_err=err, outputs=acc_out)

    def separate(st):
        attention(st)
        binding.greedy_accept(st.logits, st.parents, st.draft, workspace=ws_acc, dev_err=err,
                              outputs=acc_out)
        for l in range(layers):
            binding.commit_kv(st.k_tree[l], st.v_tree[l], acc_out[2], acc_out[1], st.prefix,
                              st.k_cache[l], st.v_cache[l], new_prefix_len=st.new_prefix,
                              dev_err=err)

    def graph_us(fn):
        graphs = []
        torch.cuda.synchronize()
        for st in sets:
            fn(st)   # warm-up outside the capture
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn(st)
            graphs.append(gr)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for k in range(4):
            graphs[k % 2].replay()
        torch.cuda.synchronize()
        a.record(stream)
        for k in range(steps):
            graphs[k % 2].replay()
        z.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(z) * 1e3 / steps

    fused_us = graph_us(fused)
    separate_us = graph_us(separate)
    attn_us = graph_us(attention)
    if int(err.item()) != 0:
        print(f"device error bits {int(err.item())} (multi-layer step)", file=sys.stderr)
        sys.exit(1)
    out = {
        "mode": "multi_layer",
        "layers": layers,
        "step_us": round(fused_us, 3),
        "step_us_per_layer_commits": round(separate_us, 3),
        "attention_us": round(attn_us, 3),
        "attention_us_per_layer": round(attn_us / layers, 3),
        "accept_commit_us": round(fused_us - attn_us, 3),
        "accept_and_commits_us": round(separate_us - attn_us, 3),
        "launches_per_step": {"fused": 2 * layers + 2, "separate": 3 * layers + 2},
        "cache_rotation": len(sets),
    }
    del sets
    torch.cuda.empty_cache()
    return out


def read_traffic():
    """HBM bytes per attention call from the committed counter summary, or
    None when it is missing or was taken on another kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for {args.gpus}); "
              "multi-GPU sharding is described in the design notes but not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from tree_verification_attention_tv_amd import binding
    from tree_verification_attention_tv_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    binding.lib()   # fail loudly if the HIP library is missing

    if args.copy_calibration:
        copy_calibration(torch, dev)
        return

    stream_gbps = stream_read_gbps(torch, binding, dev)
    wl = W.make_workload(args.workload)
    specpv = args.specpv and args.workload == "long_context"
    partial = specpv or (args.partial and wl.block_idx is not None)
    r, step_us, wall_us, eager_us, calls = measure(wl, partial, args.steps, args.warmup,
                                                   args.warm, args.num_splits, dev,
                                                   graph=not args.no_graph, specpv=specpv,
                                                   kernel=args.kernel)
    prefix_tokens, kv_bytes, attn_bytes, logit_bytes = r.bytes()
    b, n = r.b, r.n
    dominant = max(("attention", "accept"), key=lambda c: calls[c])
    dom_bytes = attn_bytes if dominant == "attention" else logit_bytes
    achieved = dom_bytes / (calls[dominant] * 1e-6) / 1e9
    traffic = read_traffic() if (dominant == "attention" and args.workload == "8b_layer"
                                 and not partial and not args.warm
                                 and args.num_splits == 0) else None

    result = {
        "metric": "tree-verify step µs and KV GB/s (% of MI355X HBM peak), 8B shape, 1 GPU",
        "value": round(step_us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 6),
        "step_us_spread": r.step_stats,
        "wall_ms_per_step": round(wall_us / 1e3, 6),
        "steps_per_graph": r.per,
        "step_launch": (f"hip_graph_replay, {r.per} consecutive steps per graph"
                        if not args.no_graph else "eager"),
        "step_us_one_per_graph": (round(r.one_per_graph_us, 3)
                                  if r.one_per_graph_us is not None else None),
        "step_us_one_per_graph_spread": r.one_per_graph_stats,
        "eager_step_us": round(eager_us, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no dataset or weights)",
        "config": {
            "workload": args.workload + ("_specpv" if specpv else "_partial" if partial else ""),
            "batch": b, "n_nodes": n, "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
            "head_dim": wl.head_dim,
            "prefix_len": prefix_tokens if b <= 4 else [min(prefix_tokens), max(prefix_tokens)],
            "vocab": wl.vocab, "cache_rotation": r.rot,
            "num_splits": binding.attention_num_splits(r.desc),
        },
        "kv_gbps": round(kv_bytes / (calls["attention"] * 1e-6) / 1e9, 1),
        "kv_hbm_frac": round(kv_bytes / (calls["attention"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "call_us": {k: round(v, 3) for k, v in calls.items()},
        "call_us_spread": r.call_stats,
        "stream_read_gbps": round(stream_gbps, 1),
        "accept_gbps": {k: round(logit_bytes / (calls[k] * 1e-6) / 1e9, 1)
                        for k in ("accept", "accept_stochastic", "accept_stochastic_filtered",
                                  "accept_stochastic_top_p") if k in calls},
        "roofline": {
            "kernel": ("tv_tree_attention (attn_split_kernel + attn_combine_kernel)"
                       if dominant == "attention" else
                       "tv_greedy_accept (vocab_argmax_kernel + path_walk_kernel)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes": dom_bytes,
            "measured_read_peak": round(stream_gbps, 1),
            "frac_of_measured_read": round(achieved / stream_gbps, 4),
        },
        "secondary": None,
        "cpu_baseline": None,
    }
    first, acc_out = r.sets[0], r.acc_out
    if not args.no_secondary and args.workload != "long_context":
        del r
        torch.cuda.empty_cache()
        result["secondary"] = {
            "tiny": secondary_line("tiny", False, 100, dev, stream_gbps),
            "specblock_tree": secondary_line("specblock_tree", False, 100, dev, stream_gbps),
            "batched": secondary_line("batched", False, 100, dev, stream_gbps),
            "long_context_full": secondary_line("long_context", False, 40, dev, stream_gbps),
            "long_context_partial": secondary_line("long_context", True, 100, dev, stream_gbps),
            "long_context_specpv": specpv_line(100, dev),
            "long_context_specpv_rectify": rectify_line(40, dev),
            "multi_layer_8b": multi_layer_line(50, dev),
        }
    if not args.no_cpu_baseline and not specpv:
        result["cpu_baseline"] = cpu_baseline(wl, partial, first, acc_out, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def stream_read_gbps(torch, binding, dev, reps=10):
    """Read bandwidth this device reaches: tv_stream_read over a 2 GiB
    buffer (8x the Infinity Cache), timed with HIP events."""
    x = torch.ones(STREAM_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(binding.STREAM_READ_SINK_WORDS, dtype=torch.int32, device=dev)
    for _ in range(3):
        binding.stream_read(x, sink)
    stream = torch.cuda.current_stream(dev)
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        binding.stream_read(x, sink)
    z.record(stream)
    torch.cuda.synchronize()
    gbps = STREAM_BYTES * reps / (a.elapsed_time(z) * 1e-3) / 1e9
    del x
    torch.cuda.empty_cache()
    return gbps


def cpu_baseline(wl, partial, dev_set, acc_out, seconds):
    """The fp64 oracle (unmodified) on the same workload, repeated for about
    `seconds` of host time; also checks the GPU results of input set 0."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1

    def one_step():
        mask, _ = oracle.build_mask(wl.parents)
        o, _ = oracle.tree_attention(
            wl.q, wl.k_cache, wl.v_cache, wl.k_tree, wl.v_tree, wl.prefix_len, mask,
            block_idx=wl.block_idx if partial else None, n_blocks=wl.n_blocks if partial else None,
            block_size=wl.block_size if partial else None)
        amax, alen, path, bonus = oracle.greedy_accept(wl.logits, wl.parents, wl.draft_tokens)
        oracle.commit_kv(wl.k_tree, wl.v_tree, path, alen, wl.prefix_len, wl.k_cache, wl.v_cache)
        return mask, o, amax, alen, path, bonus

    t0 = time.perf_counter()
    reps = 0
    res = None
    while True:
        res = one_step()
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    mask, o, amax, alen, path, bonus = res
    got_o = dev_set.out.view(torch.int16).cpu().numpy().view(np.uint16)
    got_o = ((got_o.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    parity = bool(
        np.array_equal(dev_set.mask.cpu().numpy().view(np.uint32), mask)
        and np.all(np.abs(got_o - o) <= 2e-2 + 1e-2 * np.abs(o))
        and np.array_equal(acc_out[1].cpu().numpy(), alen))
    return {
        "value": round(el / reps * 1e6, 1),
        "unit": "us/step",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps} full steps of the same workload (mask, attention, accept, commit), "
                  f"{el:.1f} s",
        "sample_parity": parity,
    }


# ---------------------------------------------------------------------------
# helper modes for the committed profile summaries
# ---------------------------------------------------------------------------

def copy_calibration(torch, dev):
    """Plain device copies of a known size: the counters' reading for them
    scales FETCH_SIZE / WRITE_SIZE to bytes."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}), flush=True)


def short_name(full, keep_template=False):
    """Kernel name without return type, anonymous namespace and arguments."""
    s = full.replace("(anonymous namespace)::", "")
    if s.startswith("void "):
        s = s[5:]
    s = s.split("(")[0]
    return s if keep_template else s.split("<")[0].split("::")[-1]


def _counter_per_dispatch(directory, counter, match):
    """Per kernel (short name): the counter summed over its instances within
    a dispatch, averaged over dispatches."""
    per = {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter or match not in row["Kernel_Name"]:
                    continue
                key = short_name(row["Kernel_Name"])
                d = per.setdefault(key, {})
                d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items() if v}


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload="8b_layer"):
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", "attn_")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE", "attn_")
    cf = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "")
    cw = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "")
    # the copy kernel is the largest reading of the calibration run
    cf_k = max(cf.values()) if cf else 0.0
    cw_k = max(cw.values()) if cw else 0.0
    f_scale = COPY_BYTES / cf_k if cf_k else float("nan")
    w_scale = COPY_BYTES / cw_k if cw_k else float("nan")
    tot_f = sum(fetch.get(k, 0.0) for k in ATTN_KERNELS)
    tot_w = sum(write.get(k, 0.0) for k in ATTN_KERNELS)
    hbm = int(round(tot_f * f_scale + tot_w * w_scale))
    what = {"8b_layer": "8B-layer workload (bench.py default",
            "specblock_tree": "SpecBlock-tree workload, 96 nodes (bench.py --workload specblock_tree",
            "batched": "16-sequence batch (bench.py --workload batched",
            "long_context": "60K-prefix workload, full KV (bench.py --workload long_context"}
    lines = [
        f"HBM traffic of one tv_tree_attention call, {what.get(workload, workload + ' (')},",
        "inputs rotated over copies so that they miss the Infinity Cache).",
        "Counter readings are scaled by what the same counter reads for a plain",
        f"device copy of {COPY_BYTES} bytes (bench.py --copy-calibration).",
        f"source_sha256_16: {source_hash()}",
        f"hbm_bytes_per_call: {hbm}",
        f"fetch_bytes_per_call: {int(round(tot_f * f_scale))}",
        f"write_bytes_per_call: {int(round(tot_w * w_scale))}",
        f"fetch_scale_bytes_per_unit: {f_scale:.2f}",
        f"write_scale_bytes_per_unit: {w_scale:.2f}",
        "  per dispatch (counter units, average over dispatches):",
    ]
    for k in ATTN_KERNELS:
        lines.append(f"    {k:22s} FETCH_SIZE {fetch.get(k, 0.0):12.1f}  "
                     f"WRITE_SIZE {write.get(k, 0.0):12.1f}")
    lines.append(f"    copy of {COPY_BYTES} B  FETCH_SIZE {cf_k:12.1f}  WRITE_SIZE {cw_k:12.1f}")
    print("\n".join(lines))


def counter_summary(dirs, match="attn_", cus=256, simds_per_cu=4, shader_engines=32):
    """Per kernel (template arguments kept), each counter summed over its
    instances within a dispatch and averaged over dispatches, from
    rocprofv3 --pmc output directories (one per pass); then ratios read off
    them.  Units, as read on MI355X: SQ_VALU_MFMA_BUSY_CYCLES and
    SQ_VALU_MFMA_COEXEC_CYCLES are cycles summed over SIMDs;
    SQ_BUSY_CYCLES is cycles summed over the 32 shader engines (so /32 is
    the dispatch's length in cycles); SQ_BUSY_CU_CYCLES is cycles summed
    over CUs; SQ_ACTIVE_INST_*, SQ_WAIT_INST_ANY and SQ_WAVE_CYCLES are
    quad-cycles summed over waves."""
    # per (pass, kernel, counter): the dispatch sums, averaged; a counter
    # read in several passes is averaged over them
    per = {}
    # per kernel: (SQ_BUSY_CYCLES / shader engines, dispatch ns) of each
    # dispatch, from the same pass (its own start and end timestamps)
    clock = {}
    for d in dirs:
        one = {}
        span = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if match not in row["Kernel_Name"]:
                        continue
                    k = short_name(row["Kernel_Name"], keep_template=True)
                    c = one.setdefault(k, {}).setdefault(row["Counter_Name"], {})
                    c[row["Dispatch_Id"]] = c.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
                    if "Start_Timestamp" in row:
                        span[(k, row["Dispatch_Id"])] = (int(row["End_Timestamp"])
                                                         - int(row["Start_Timestamp"]))
        for k, cs in one.items():
            for n, v in cs.items():
                if v:
                    per.setdefault(k, {}).setdefault(n, []).append(sum(v.values()) / len(v))
            for disp, cyc in cs.get("SQ_BUSY_CYCLES", {}).items():
                ns = span.get((k, disp), 0)
                if ns > 0:
                    clock.setdefault(k, []).append((cyc / shader_engines, ns))
    print(f"source_sha256_16: {source_hash()}")
    print("counter averages per dispatch; ratios below each kernel")
    simds = cus * simds_per_cu
    for k, cs in sorted(per.items()):
        avg = {n: sum(v) / len(v) for n, v in cs.items()}
        print(f"\n{k}")
        for n in sorted(avg):
            print(f"  {n:32s} {avg[n]:16.1f}")
        cyc = avg.get("SQ_BUSY_CYCLES", 0.0) / shader_engines
        mfma = avg.get("SQ_VALU_MFMA_BUSY_CYCLES")
        if cyc:
            print(f"  dispatch_cycles                  {cyc:16.1f}")
        if clock.get(k):
            # shader clock while the dispatch ran: its busy cycles over its
            # own duration (median over dispatches)
            ghz = sorted(c / ns for c, ns in clock[k])[len(clock[k]) // 2]
            print(f"  shader_clock_ghz (median)        {ghz:16.3f}")
        if mfma is not None and cyc:
            print(f"  mfma_busy_frac (of SIMD cycles)  {mfma / (simds * cyc):16.4f}")
        if mfma is not None and avg.get("SQ_BUSY_CU_CYCLES"):
            print(f"  mfma_busy_frac (CU-busy cycles)  "
                  f"{mfma / (simds_per_cu * avg['SQ_BUSY_CU_CYCLES']):16.4f}")
        if mfma and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
            print(f"  valu_coexec_of_mfma_busy         {avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / mfma:16.4f}")
        waves_cyc = 4 * avg.get("SQ_WAVE_CYCLES", 0.0)
        for n, lab in (("SQ_ACTIVE_INST_VALU", "valu_active_of_wave_cycles"),
                       ("SQ_ACTIVE_INST_LDS", "lds_active_of_wave_cycles"),
                       ("SQ_WAIT_INST_ANY", "issue_wait_of_wave_cycles")):
            if waves_cyc and n in avg:
                print(f"  {lab:32s} {4 * avg[n] / waves_cyc:16.4f}")
        mops = avg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        if mops is not None:
            print(f"  mfma_bf16_flops                  {mops * 512:16.4e}")
        if avg.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in avg:
            print(f"  lds_bank_conflict_cycles_frac    "
                  f"{avg['SQ_LDS_BANK_CONFLICT'] / (4 * avg['SQ_ACTIVE_INST_LDS']):16.4f}")


def trace_summary(stats_csv, command):
    with open(stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    print(f"rocprofv3 kernel-trace stats\ncommand: {command}\n")
    print(f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}")
    for r in rows:
        name = short_name(r["Name"], keep_template=True)
        print(f"{name[:60]:60s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:9.2f} "
              f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
              f"{float(r['Percentage']):6.2f}")


if __name__ == "__main__":
    main()
