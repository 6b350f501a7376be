"""Benchmark of one tree-verify step on one MI355X.

A step is the whole hot path over one batch of synthetic input, back to back
on one stream: build the tree mask, one layer of tree attention over the
verified-prefix KV, greedy acceptance over the vocabulary, KV commit.
Default workload: the 8B-layer shape (batch 1, 32 query / 8 KV heads of 128,
1000-token prefix, 60-node EAGLE-style tree, 128256-token bf16 logits).

Inputs are resident in HBM before the timed region.  To measure HBM rather
than cache bandwidth, the step rotates over enough independent copies of its
inputs that their total exceeds the 256 MB Infinity Cache.

Prints one JSON line (rank 0):
  value = microseconds per verify step (lower is better); also KV GB/s,
  a roofline entry for the dominant kernel (HIP-event timing of its own
  launches) and the fp64 CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MALL_BYTES = 256 * 1024 * 1024  # Infinity Cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="8b_layer",
                    choices=["tiny", "8b_layer", "specblock_tree", "batched", "long_context"])
    ap.add_argument("--partial", action="store_true", help="partial-KV mode (long_context only)")
    ap.add_argument("--warm", action="store_true", help="no input rotation (cache-warm)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--num-splits", type=int, default=0)
    return ap.parse_args()


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

    def nbytes(self):
        import torch
        return sum(t.numel() * t.element_size() for t in vars(self).values()
                   if isinstance(t, torch.Tensor))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for {args.gpus}); "
              "multi-GPU sharding is described in the design notes but not built.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from tree_verification_attention_tv_amd import binding
    from tree_verification_attention_tv_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    binding.lib()   # fail loudly if the HIP library is missing

    wl = W.make_workload(args.workload)
    partial = args.partial and wl.block_idx is not None
    b, n = wl.parents.shape
    hq, hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.head_dim

    # ---- rotation so that the working set exceeds the Infinity Cache ------
    first = InputSet(wl, dev, torch, np)
    per_set = first.nbytes()
    rot = 1 if args.warm else max(2, int(np.ceil(1.25 * MALL_BYTES / per_set)))
    rot = min(rot, 64)
    sets = [first] + [InputSet(wl, dev, torch, np) for _ in range(rot - 1)]

    desc = binding.attn_desc(first.q, first.k_cache, max_prefix_len=wl.max_prefix_len,
                             block_size=wl.block_size if partial else 0,
                             max_blocks=wl.max_blocks if partial else 0,
                             num_splits=args.num_splits)
    ws_attn = torch.empty(binding.attention_workspace_size(desc), dtype=torch.uint8, device=dev)
    ws_acc = torch.empty(binding.accept_workspace_size(b, n, wl.vocab), dtype=torch.uint8,
                         device=dev)
    acc_out = (torch.empty((b, n), dtype=torch.int32, device=dev),
               torch.empty((b,), dtype=torch.int32, device=dev),
               torch.empty((b, n), dtype=torch.int32, device=dev),
               torch.empty((b,), dtype=torch.int32, device=dev))
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def k_mask(s):
        st = binding.lib().tv_build_tree_mask(binding._ptr(s.parents), b, n, binding._ptr(s.mask),
                                              None, binding._ptr(err), binding._stream(dev))
        if st:
            raise binding.TVError("tv_build_tree_mask", st)

    def k_attn(s):
        binding.tree_attention(s.q, s.k_cache, s.v_cache, s.k_tree, s.v_tree, s.prefix_len,
                               s.mask, max_prefix_len=wl.max_prefix_len,
                               block_idx=s.block_idx if partial else None,
                               n_blocks=s.n_blocks if partial else None,
                               block_size=wl.block_size if partial else 0,
                               num_splits=args.num_splits, out=s.out, workspace=ws_attn,
                               dev_err=err)

    def k_accept(s):
        binding.greedy_accept(s.logits, s.parents, s.draft, workspace=ws_acc, dev_err=err,
                              outputs=acc_out)

    def k_commit(s):
        binding.commit_kv(s.k_tree, s.v_tree, acc_out[2], acc_out[1], s.prefix_len,
                          s.k_cache, s.v_cache, new_prefix_len=s.new_prefix, dev_err=err)

    def step(s):
        k_mask(s)
        k_attn(s)
        k_accept(s)
        k_commit(s)

    for k in range(args.warmup):
        step(sets[k % rot])
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        print(f"device error bits {int(err.item())}", file=sys.stderr)
        sys.exit(1)

    # ---- timed region: K whole steps -----------------------------------
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(args.steps):
        step(sets[k % rot])
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_us = e0.elapsed_time(e1) * 1e3 / args.steps
    wall_ms_per_step = (t1 - t0) * 1e3 / args.steps

    # ---- per-call timing (same rotation), for the roofline ------------------
    def time_call(fn, iters):
        for k in range(3):
            fn(sets[k % rot])
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k in range(iters):
            fn(sets[k % rot])
        z.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(z) * 1e3 / iters

    iters = max(args.steps, 50)
    t_mask = time_call(k_mask, iters)
    t_attn = time_call(k_attn, iters)
    t_accept = time_call(k_accept, iters)
    t_commit = time_call(k_commit, iters)

    # algorithmic bytes
    if partial:
        vis = sum(min(wl.block_size, int(wl.prefix_len[0]) - int(x) * wl.block_size)
                  for x in wl.block_idx[0, :int(wl.n_blocks[0])])
        prefix_tokens = [vis]
    else:
        prefix_tokens = [int(p) for p in wl.prefix_len]
    kv_bytes = (sum(prefix_tokens) + b * n) * hkv * d * 2 * 2
    qo_bytes = 2 * b * n * hq * d * 2
    mask_bytes = b * n * ((n + 31) // 32) * 4
    attn_bytes = kv_bytes + qo_bytes + mask_bytes
    logit_bytes = wl.logits.nbytes
    calls = {"mask": t_mask, "attention": t_attn, "accept": t_accept, "commit": t_commit}
    dominant = max(("attention", "accept"), key=lambda c: calls[c])
    dom_bytes = attn_bytes if dominant == "attention" else logit_bytes
    achieved = dom_bytes / (calls[dominant] * 1e-6) / 1e9

    result = {
        "metric": "tree-verify step µs and KV GB/s (% of MI355X HBM peak), 8B shape, 1 GPU",
        "value": round(step_us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 6),
        "wall_ms_per_step": round(wall_ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no dataset or weights)",
        "config": {
            "workload": args.workload + ("_partial" if partial else ""),
            "batch": b, "n_nodes": n, "n_q_heads": hq, "n_kv_heads": hkv, "head_dim": d,
            "prefix_len": prefix_tokens if b <= 4 else [min(prefix_tokens), max(prefix_tokens)],
            "vocab": wl.vocab, "cache_rotation": rot,
            "num_splits": binding.attention_num_splits(desc),
        },
        "kv_gbps": round(kv_bytes / (t_attn * 1e-6) / 1e9, 1),
        "kv_hbm_frac": round(kv_bytes / (t_attn * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "call_us": {k: round(v, 3) for k, v in calls.items()},
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "algorithmic_bytes": dom_bytes,
        },
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, partial, first, acc_out, args.cpu_seconds)
    print(json.dumps(result), flush=True)


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
        if time.perf_counter() - t0 >= seconds or reps >= 100:
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


if __name__ == "__main__":
    main()
