#!/usr/bin/env python3
"""Benchmark of the paged extend-attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input: for every batch
of the workload, build the step metadata (host planner + its copy to the
device), append the chunk's K/V into the pages, run the extend attention
(plus the split combine when the plan has split rows). The default workload
is a 4097-token prompt prefilled to completion under a 512-token chunk budget
(9 chunks; 16 query / 4 KV heads, head_dim 128, 64-token pages, bf16).

Prints ONE JSON line. `value` is extend-attention TFLOP/s over the step
(algorithmic FLOPs: 4*D*Hq per visible (query, key) pair); `tokens_per_s`
counts query tokens. `roofline` is for the attention kernel, timed with
events around each launch on the launch stream; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)

METRIC = "extend-attn TFLOP/s + % bf16 MFMA peak (4097-tok prompt, 512 chunk), tokens/s"
KERNEL_SRC = os.path.join(ROOT, "paged_chunked_prefill_amd", "csrc", "extend_attn.hip")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20       # bytes read and written per copy_calibration launch
MFMA_PEAK_BF16 = 2500.0      # TFLOP/s, MI355X dense bf16
MFMA_PEAK_FP32 = 157.3       # TFLOP/s, MI355X fp32 matrix (vector figure as stated for the chip)
HBM_PEAK = 8000.0            # GB/s
FUSE_MAX_SLOT_BLOCKS = 128   # paged_extend_attn_append fuses the append up to this plan.slot_blocks


# ---------------------------------------------------------------------------
# workloads: a list of batches run in order against one cache
# ---------------------------------------------------------------------------

class HipEvents:
    """Timing events recorded straight through the HIP runtime (one ctypes call
    per record): the per-launch brackets of the timed steps then add about a
    microsecond of host time each instead of a torch.cuda.Event round trip, so
    that they do not stretch a host-bound step."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)
        self.record = self.hip.hipEventRecord

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def workload(name):
    import workloads as wl
    if name.startswith("prompt"):
        # promptN_chunkB
        n, b = name[len("prompt"):].split("_chunk")
        w = wl.config3(int(n))
        chunks = wl.chunk_partition(int(n), int(b))
        desc = (f"{n}-token prompt prefilled in {len(chunks)} chunks of <= {b} tokens; 16 query / 4 KV heads, "
                f"head_dim 128, page_size 64, bf16")
        return w, wl.chunked_steps(w, chunks), False, desc
    if name.startswith("budget"):
        # budgetB_decodeN: the 4097-token prompt in chunks of B - N tokens, each step also N decode rows
        bb, nd = name[len("budget"):].split("_decode")
        w, steps = wl.budget_steps(4097, int(bb), int(nd))
        desc = (f"4097-token prompt prefilled under a {bb}-token step budget shared with {nd} decoding requests "
                f"(cached 1024..8192): {len(steps)} steps of {nd} one-token rows + a {int(bb) - int(nd)}-token "
                f"chunk; 16 query / 4 KV heads, head_dim 128, page_size 64, bf16")
        # the decode rows' cached prefixes are written first (up to their last step's position)
        return w, steps, True, desc
    if name == "ragged4":
        w = wl.config2()
        return w, [w], True, "ragged batch P={0,100,513,1025} L={1,64,128,512}; 32/8 heads, D=128, ps=16, bf16"
    if name == "window8":
        w = wl.config4()
        return w, [w], True, "8 x (6000 cached + 1000 new), window 4096; 32/8 heads, D=128, ps=16, bf16"
    if name == "mixed":
        w = wl.config5()
        return w, [w], True, ("64 one-token rows (KV 2048..32768, 8 splits) + 2 x (16384 + 2048) prefill rows; "
                              "64/8 heads, D=128, ps=16, bf16")
    if name == "decode64":
        w = wl.config5(decode_only=True)
        return w, [w], True, "64 one-token rows (KV 2048..32768, 8 splits); 64/8 heads, D=128, ps=16, bf16"
    if name == "prefill2":
        w = wl.config5(prefill_only=True)
        return w, [w], True, "2 x (16384 cached + 2048 new); 64/8 heads, D=128, ps=16, bf16"
    raise SystemExit(f"unknown workload {name}")


def visible_pairs(P, L, window):
    import numpy as np
    tot = 0
    for p, l in zip(P, L):
        pos = np.arange(int(p), int(p) + int(l), dtype=np.int64)
        vis = pos + 1
        if window > 0:
            vis = np.minimum(vis, window)
        tot += int(vis.sum())
    return tot


def kv_span_tokens(P, L, window):
    tot = 0
    for p, l in zip(P, L):
        lo = 0 if window <= 0 else max(0, int(p) - window + 1)
        tot += int(p) + int(l) - lo
    return tot


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prompt4097_chunk512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the whole step replayed from one captured HIP graph (every batch's append + "
                         "attention in order, metadata built once), reported as graph_replay")
    ap.add_argument("--cpu-sample-rows", type=int, default=0, help="rows for the CPU oracle sample (0: auto)")
    ap.add_argument("--mask", choices=["none", "rows", "heads"], default="none",
                    help="run paged_extend_attn_masked with an all-keep mask of [B, 1, max_q_len, Ks] (rows) or "
                         "[B, Hq, max_q_len, Ks] (heads): same visible pairs, so the TFLOP/s show the mask's cost")
    ap.add_argument("--append", choices=["separate", "fused"], default="fused",
                    help="fused (default): paged_extend_attn_append, whose bf16 attention launch also writes the "
                         "chunk's K/V into the pool when the plan's slot_blocks <= 128 (else it runs the append "
                         "kernel first); separate: pkv_append then paged_extend_attn")
    ap.add_argument("--layers", type=int, default=1,
                    help="attention layers per batch: the batch's plan is built (and copied) once and every "
                         "layer runs its own append + attention on its own K/V pools, queries and outputs")
    ap.add_argument("--rope", action="store_true",
                    help="the step rotates q and k at their absolute positions with pkv_rope_append (in place "
                         "of pkv_append) before the attention; reports that kernel's HBM rate")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 --kernel-trace --stats output directory")
    ap.add_argument("--stats-json", metavar="PATH", help="with --summarize-stats: also write the attention "
                    "kernel's average duration and the combine's time per call as JSON (profiles/stats_<workload>.json)")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="rocprofv3 --pmc output directory (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES, "
                         "SQ_INSTS_VALU, SQ_INSTS_MFMA, GRBM_GUI_ACTIVE) of --workload: print the attention kernel's "
                         "executed MFMA work per launch against the algorithmic FLOPs, and its MFMA busy fraction")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE of --workload; the same "
                         "two of copy_calibration): print the attention kernel's HBM traffic per launch as JSON")
    args = ap.parse_args()
    if args.summarize_stats:
        return summarize_stats(args)
    if args.summarize_traffic:
        return summarize_traffic(args)
    if args.summarize_mfma:
        return summarize_mfma(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: runs on one GPU only (paged extend attention on one MI355X; no multi-GPU path); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_chunked_prefill_amd as pkv
    from gpu_harness import DeviceCache, shape_of, to_dev, upload_q

    torch.cuda.set_device(0)
    if args.workload == "copy_calibration":
        return copy_calibration(args)
    if args.workload == "gemm_calibration":
        return gemm_calibration(args)
    if not pkv.device_supported(0):
        raise SystemExit("device 0 is not gfx950")
    lib = pkv.lib()
    w, batches, prefill_prefix, desc = workload(args.workload)
    shape = shape_of(w)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    t_setup = time.time()
    cache = DeviceCache(w, dev)
    if prefill_prefix:
        cache.fill_prefix(w)
    nsteps = args.warmup + args.steps
    if args.layers < 1:
        raise SystemExit("--layers must be >= 1")
    # pools of layers 1.. (--layers): copies of the cache's pools as they stand after the prefix was written
    layer_pools = [(cache.k_pool.clone(), cache.v_pool.clone()) for _ in range(1, args.layers)]

    # rotary table (cos, sin) of every position the workload reaches, for --rope
    import workloads as wl
    max_pos = max(int((np.asarray(bw.prefix_lens) + np.asarray(bw.chunk_lens)).max()) for bw in batches)
    rope_table = torch.from_numpy(wl.rope_table(max_pos + 1, w.head_dim)).to(dev) if args.rope else None
    esize = 2 if w.dtype == "bf16" else 4
    # the rotary append and the masked attention keep their own calls
    fuse_mode = args.append == "fused" and not args.rope and args.mask == "none"
    # per batch: device inputs, output, metadata buffers, pre-marshalled ctypes arguments
    B = []
    for bw in batches:
        P = np.ascontiguousarray(bw.prefix_lens, np.int32)
        L = np.ascontiguousarray(bw.chunk_lens, np.int32)
        splits = bw.decode_splits
        meta_bytes, ws_bytes = pkv.extend_metadata_size(P, L, shape, bw.window, splits)
        kn, vn = cache._gather_new_kv(bw)
        q = upload_q(bw, dev)
        out = torch.empty_like(q)
        meta_dev = torch.empty(meta_bytes, dtype=torch.uint8, device=dev)
        hosts = [torch.empty(meta_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(nsteps)]
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        plan = pkv.PkvPlan()
        b = dict(P=P, L=L, kn=kn, vn=vn, q=q, out=out, meta_dev=meta_dev, hosts=hosts, ws=ws, plan=plan,
                 total_q=int(L.sum()), flops=4 * w.head_dim * w.num_q_heads * visible_pairs(P, L, bw.window),
                 bytes=2 * (2 * int(L.sum()) * w.num_q_heads * w.head_dim +
                            2 * w.num_kv_heads * w.head_dim * kv_span_tokens(P, L, bw.window)))
        vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        b["meta_args"] = [(len(L), P.ctypes.data_as(ctypes.c_void_p), L.ctypes.data_as(ctypes.c_void_p),
                           ctypes.byref(shape), bw.window, splits, vp(h), meta_bytes, vp(meta_dev), meta_bytes,
                           ctypes.byref(plan), sh) for h in hosts]
        def calls_for(q, out, k_pool, v_pool):
            """(append fn, its args, attention fn, its args, rotated-q buffer) of one layer's batch call."""
            append_fn = append_args = q_rot = None
            if args.rope:
                # q is rotated into q_rot, which the attention reads; per token the kernel moves q, K and V
                # in and out once and reads one table row
                q_rot = torch.empty_like(q)
                append_fn = lib.pkv_rope_append
                append_args = (vp(q), vp(q_rot), vp(kn), vp(vn), vp(rope_table), rope_table.shape[0],
                               vp(k_pool), vp(v_pool), vp(cache.page_table), cache.page_table.shape[1],
                               None, ctypes.byref(plan), ctypes.byref(shape), sh)
            else:
                append_fn = lib.pkv_append
                append_args = (vp(kn), vp(vn), vp(k_pool), vp(v_pool), vp(cache.page_table),
                               cache.page_table.shape[1], None, ctypes.byref(plan), ctypes.byref(shape), sh)
            q_attn = q_rot if args.rope else q
            if args.mask == "none":
                attn_fn = lib.paged_extend_attn
                attn_args = (vp(q_attn), vp(k_pool), vp(v_pool), vp(cache.page_table),
                             cache.page_table.shape[1], None, None, None, None, bw.window, 0.0, ctypes.byref(plan),
                             ctypes.byref(shape), vp(out), vp(ws), ws.numel(), sh)
            else:
                attn_fn = lib.paged_extend_attn_masked
                attn_args = (vp(q_attn), vp(k_pool), vp(v_pool), vp(cache.page_table),
                             cache.page_table.shape[1], None, None, None, None, bw.window, 0.0, vp(b["mask"]), mh,
                             int(L.max()), ks, ctypes.byref(plan), ctypes.byref(shape), vp(out), vp(ws), ws.numel(),
                             sh)
            if fuse_mode:
                append_fn = append_args = None
                attn_fn = lib.paged_extend_attn_append
                attn_args = (vp(q), vp(kn), vp(vn), vp(k_pool), vp(v_pool), vp(cache.page_table),
                             cache.page_table.shape[1], None, bw.window, 0.0, ctypes.byref(plan),
                             ctypes.byref(shape), vp(out), vp(ws), ws.numel(), sh)
            return append_fn, append_args, attn_fn, attn_args, q_rot

        if args.mask != "none":
            ks = (int((P + L).max()) + 3) // 4 * 4
            mh = w.num_q_heads if args.mask == "heads" else 1
            b["mask"] = torch.ones((len(L), mh, int(L.max()), ks), dtype=torch.uint8, device=dev)
        # layer 0 uses the cache's pools, q and out; each further layer (--layers) its own copies of
        # them (the pools as they stand after the prefix was written), all under the batch's one plan
        b["layers"] = [calls_for(q, out, cache.k_pool, cache.v_pool)]
        b["keep"] = []   # layer tensors, alive as long as their pointers are in use
        for li in range(1, args.layers):
            kp_l, vp_l = layer_pools[li - 1]
            q_l, out_l = q.clone(), torch.empty_like(out)
            b["keep"] += [q_l, out_l]
            b["layers"].append(calls_for(q_l, out_l, kp_l, vp_l))
        b["keep_rot"] = [c[4] for c in b["layers"]]
        tq = int(L.sum())
        b["append_bytes"] = (tq * (2 * esize * w.head_dim * (w.num_q_heads + 2 * w.num_kv_heads) + 4 * w.head_dim)
                             if args.rope else tq * 4 * esize * w.head_dim * w.num_kv_heads)
        B.append(b)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    hev = HipEvents(2 * nsteps * len(B) * args.layers)   # (step s, batch i, layer l): 2((s*len(B)+i)*layers+l), +1
    evs, rec = hev.ev, hev.record
    build = lib.build_extend_metadata

    def step(s, bracket):
        for i, b in enumerate(B):
            if build(*b["meta_args"][s]):
                raise RuntimeError(lib.pkv_last_error().decode())
            for li, (append_fn, append_args, attn_fn, attn_args, _) in enumerate(b["layers"]):
                if append_fn is not None and append_fn(*append_args):
                    raise RuntimeError(lib.pkv_last_error().decode())
                k = 2 * ((s * len(B) + i) * args.layers + li)
                if bracket:
                    rec(evs[k], sh)
                if attn_fn(*attn_args):
                    raise RuntimeError(lib.pkv_last_error().decode())
                if bracket:
                    rec(evs[k + 1], sh)

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, nsteps):
        step(s, False)
    t_enq = time.perf_counter() - t0      # host time to plan and enqueue the K steps
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    # Launch durations: the same K steps again (same plans, appends and attention
    # calls), each attention call bracketed by HIP events on its stream. The timed
    # steps above carry no events: on these launch-bound steps every event marker
    # between two kernels costs GPU time (the headline step measures about 25 %
    # longer with them).
    for s in range(args.warmup, nsteps):
        step(s, True)
    torch.cuda.synchronize()

    # per batch: its attention calls over every layer
    attn_ms = [sum(hev.elapsed_ms(2 * ((s * len(B) + i) * args.layers + li), 2 * ((s * len(B) + i) * args.layers + li) + 1)
                   for s in range(args.warmup, nsteps) for li in range(args.layers)) / args.steps
               for i in range(len(B))]
    hev.close()
    # the appends (or rotary appends) of a step, timed in a pass of their own after the timed steps so that
    # their events do not add to the step (rewriting the same slots and q rows: idempotent)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        for b in B:
            for append_fn, append_args, _, _, _ in b["layers"]:
                if append_fn is not None and append_fn(*append_args):
                    raise RuntimeError(lib.pkv_last_error().decode())
    e1.record(stream)
    torch.cuda.synchronize()
    append_ms = e0.elapsed_time(e1) / args.steps
    append_bytes = sum(b["append_bytes"] for b in B) * args.layers
    flops = sum(b["flops"] for b in B) * args.layers
    hbm_bytes = sum(b["bytes"] for b in B) * args.layers
    tokens = sum(b["total_q"] for b in B)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    attn_total_ms = sum(attn_ms)
    attn_tflops = flops / (attn_total_ms * 1e-3) / 1e12
    attn_gbs = hbm_bytes / (attn_total_ms * 1e-3) / 1e9
    n_launch = len(B) * args.layers
    # launches whose append ran inside the attention kernel (paged_extend_attn_append's choice)
    n_fused = args.layers * sum(1 for b in B if fuse_mode and w.dtype == "bf16" and b["plan"].total_q > 0 and
                                b["plan"].slot_blocks <= FUSE_MAX_SLOT_BLOCKS)
    decode_bound = args.workload == "decode64"
    roofline = {
        "kernel": f"extend_attn_{w.dtype}<{w.head_dim}>" + (
                  f" (append fused in {n_fused} of {n_launch} launches)" if n_fused else "") +
                  (" + combine_splits" if any(
            b["plan"].n_split_rows for b in B) else ""),
        "bound": "hbm" if decode_bound else "mfma",
        "achieved": round(attn_gbs if decode_bound else attn_tflops, 3),
        "peak": HBM_PEAK if decode_bound else (MFMA_PEAK_BF16 if w.dtype == "bf16" else MFMA_PEAK_FP32),
        "unit": "GB/s" if decode_bound else "TFLOP/s",
        "frac": None, "traffic": None,
        "avg_launch_us": round(1e3 * attn_total_ms / n_launch, 3),
        "launch_timing": "HIP events around every attention call of a second pass over the same K steps",
        "launches_per_step": n_launch,
        "algorithmic_per_launch": round((hbm_bytes if decode_bound else flops) / n_launch),
    }
    roofline["frac"] = round(roofline["achieved"] / roofline["peak"], 4)
    tr = load_traffic(args.workload)
    if tr is not None:
        # HBM bytes per attention kernel launch from the FETCH_SIZE / WRITE_SIZE counters, scaled by the
        # same counters on a copy of known size; the split combine's bytes are not in it
        # a launch with the append fused in also reads the chunk's K/V rows and writes them into the pool
        alg = hbm_bytes + (append_bytes if n_fused == n_launch else 0)
        roofline["traffic"] = tr["traffic_bytes_per_launch"]
        roofline["traffic_vs_algorithmic_bytes"] = round(tr["traffic_bytes_per_launch"] / (alg / n_launch), 3)
        roofline["traffic_source"] = f"profiles/traffic_{args.workload}.json"

    st = load_profile("stats", args.workload)
    if st is not None:
        # the same figure from the rocprofv3 kernel statistics of this command: the attention kernel
        # alone, and with the split combine's time per call (the event interval also holds the gap
        # between the two launches)
        per = roofline["algorithmic_per_launch"]            # FLOPs (bytes for the one-token rows)
        scale = 1e9 if decode_bound else 1e12                # -> GB/s or TFLOP/s, the peak's unit
        k_us, c_us = st["extend_attn_avg_us"], st["combine_us_per_attention_call"]

        def frac(us):
            return round(per / (us * 1e-6) / scale / roofline["peak"], 4)

        roofline["profile"] = {"extend_attn_avg_us": k_us, "combine_us_per_call": c_us,
                               "frac_kernel": frac(k_us), "frac_kernel_and_combine": frac(k_us + c_us),
                               "source": f"profiles/stats_{args.workload}.json"}
    roofline["frac_source"] = ("HIP events around each attention call: the attention kernel, the split combine "
                               "after it when the plan has split rows, and the gap between them")

    graph_replay = None
    if args.graph:
        graph_replay = time_graph_replay(args, B, lib, flops, tokens)

    # check the last step's outputs are finite (no canary NaN reached the result)
    for b in B:
        if torch.isnan(b["out"].float()).any():
            raise RuntimeError("NaN in attention output")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, batches, args.cpu_sample_rows)

    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0,1) q/k/v, shuffled page tables)",
        "config": {"workload": desc, "name": args.workload, "rotary_append": bool(args.rope),
                   "explicit_mask": args.mask, "append": "fused" if fuse_mode else "separate",
                   "layers": args.layers,
                   "split_partials": ("bf16 unnormalised output, fp32 (max, sum)" if w.dtype == "bf16"
                                      else "fp32 unnormalised output, fp32 (max, sum)"),
                   "batches_per_step": len(B),
                   "query_tokens_per_step": tokens, "flops_per_step": flops},
        "tokens_per_s": round(tokens / (ms_per_step * 1e-3), 1),
        "host_enqueue_ms_per_step": round(1e3 * t_enq / args.steps, 4),
        "mfma_peak_frac": round(tflops / MFMA_PEAK_BF16, 4),
        "attn_only": {"ms_per_step": round(attn_total_ms, 4), "tflops": round(attn_tflops, 3),
                      "mfma_peak_frac": round(attn_tflops / MFMA_PEAK_BF16, 4),
                      "hbm_gbs_algorithmic": round(attn_gbs, 1), "per_launch_ms": [round(x / args.layers, 4) for x in attn_ms]},
        "roofline": roofline, "cpu_baseline": cpu, "setup_s": round(setup_s, 2),
    }
    rope_cpu = None
    if args.rope and not args.no_cpu_baseline:
        rope_cpu = cpu_rope_baseline(batches, w, rope_table.cpu().numpy())
    line["append"] = {"kernel": "pkv_rope_append (rotary q, k + append)" if args.rope else
                      (f"paged_extend_attn_append: inside the attention launch in {n_fused} of {n_launch} "
                       "calls, the append kernel first in the others" if fuse_mode else "pkv_append"),
                      "ms_per_step": round(append_ms, 4), "bytes_per_step": append_bytes,
                      "gbs_algorithmic": round(append_bytes / (append_ms * 1e-3) / 1e9, 1) if append_ms > 0.01 else None,
                      "hbm_frac": round(append_bytes / (append_ms * 1e-3) / 1e9 / HBM_PEAK, 4) if append_ms > 0.01 else None}
    if rope_cpu is not None:
        line["append"]["cpu_baseline"] = rope_cpu
    if graph_replay is not None:
        line["graph_replay"] = graph_replay
    print(json.dumps(line), flush=True)


def time_graph_replay(args, B, lib, flops, tokens):
    """The whole step captured once into one HIP graph and replayed: every batch
    in order, each with its append and attention (and split combine), on a
    stream of its own. Each batch's plan is built once before capture (the
    host planner and the metadata copy stay outside the replay, as when a
    step's plan serves every layer). Reports the replayed step's rate next to
    the eager step's."""
    import torch
    s = torch.cuda.Stream()
    sh = ctypes.c_void_p(s.cuda_stream)
    calls = []
    for b in B:
        if lib.build_extend_metadata(*b["meta_args"][0]):
            raise RuntimeError(lib.pkv_last_error().decode())
        for append_fn, append_args, attn_fn, attn_args, _ in b["layers"]:
            ap = append_args[:-1] + (sh,) if append_args is not None else None
            calls.append((append_fn, ap, attn_fn, attn_args[:-1] + (sh,)))
    torch.cuda.synchronize()

    def step():
        for app_fn, ap, attn_fn, at in calls:
            if (app_fn is not None and app_fn(*ap)) or attn_fn(*at):
                raise RuntimeError(lib.pkv_last_error().decode())

    with torch.cuda.stream(s):       # one eager pass on the capture stream first
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
            "tokens_per_s": round(tokens / (ms * 1e-3), 1), "graphs_per_step": 1, "batches_per_graph": len(calls),
            "note": "the whole step (every batch's append + attention + combine, in order) replayed from one "
                    "captured graph; the host planner and metadata copies run once, outside the timed region"}


def kernel_hash():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_profile(kind, name):
    """profiles/<kind>_<workload>.json, if it was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"{kind}_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    return tr if tr.get("kernel_source_sha256_16") == kernel_hash() else None


def load_traffic(name):
    """Counter traffic recorded for this workload, if it was taken on the current kernel source."""
    return load_profile("traffic", name)


def _counter_means(directory, match):
    """Counter values summed over the instances of each dispatch whose kernel name contains `match`,
    then averaged over those dispatches (rocprofv3 csv: run_counter_collection.csv)."""
    import collections
    import csv
    per = collections.defaultdict(float)
    dur = {}
    with open(os.path.join(directory, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if match in r["Kernel_Name"]:
                key, v = (r["Dispatch_Id"], r["Counter_Name"]), float(r["Counter_Value"])
                # GRBM counters count GPU-wide cycles: the instances are copies, take the largest
                per[key] = max(per[key], v) if r["Counter_Name"].startswith("GRBM_") else per[key] + v
                dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = collections.defaultdict(list)
    for (_, c), v in per.items():
        out[c].append(v)
    means = {c: sum(v) / len(v) for c, v in out.items()}
    means["duration_ns"] = sum(dur.values()) / max(1, len(dur))
    return means, len({d for d, _ in per})


def summarize_traffic(args):
    f_dir, w_dir, cf_dir, cw_dir = args.summarize_traffic
    fetch, n = _counter_means(f_dir, "extend_attn")
    write, _ = _counter_means(w_dir, "extend_attn")
    cal_f, _ = _counter_means(cf_dir, "copyBuffer")
    cal_w, _ = _counter_means(cw_dir, "copyBuffer")
    fs = (COPY_BYTES / 1024) / cal_f["FETCH_SIZE"]    # counters are in KiB
    ws = (COPY_BYTES / 1024) / cal_w["WRITE_SIZE"]
    out = {"workload": args.workload, "kernel": "extend_attn", "kernel_source_sha256_16": kernel_hash(),
           "dispatches": n, "fetch_kib_per_launch": round(fetch["FETCH_SIZE"], 1),
           "write_kib_per_launch": round(write["WRITE_SIZE"], 1),
           "copy_fetch_kib": round(cal_f["FETCH_SIZE"], 1), "copy_write_kib": round(cal_w["WRITE_SIZE"], 1),
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "traffic_bytes_per_launch": round((fetch["FETCH_SIZE"] * fs + write["WRITE_SIZE"] * ws) * 1024)}
    print(json.dumps(out, indent=1))


def summarize_mfma(args):
    """Executed MFMA work of the attention kernel per launch (rocprofv3 counters,
    summed over the kernel's instances and averaged over its dispatches)
    against the workload's algorithmic FLOPs (4 D Hq per visible pair), the
    MFMA busy fraction (busy cycles per SIMD over one XCD's active cycles) and
    the clock the kernel ran at (active cycles over the dispatch's duration)."""
    import numpy as np
    c, n = _counter_means(args.summarize_mfma, "extend_attn")
    w, batches, _, desc = workload(args.workload)
    alg = [4 * w.head_dim * w.num_q_heads * visible_pairs(np.asarray(b.prefix_lens), np.asarray(b.chunk_lens), b.window)
           for b in batches]
    alg_per_launch = sum(alg) / len(alg)
    simds = 256 * 4
    executed = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    # GRBM_GUI_ACTIVE here sums the busy cycles of the 8 XCDs (a fill kernel of 176 us reads
    # 3.44e6 = 8 x 2.44 GHz x 176 us), so one XCD's cycles, the clock the kernel ran at, are an eighth
    xcd_cycles = c["GRBM_GUI_ACTIVE"] / 8
    out = {"workload": args.workload, "kernel": "extend_attn", "kernel_source_sha256_16": kernel_hash(),
           "dispatches": n, "launches_per_step": len(alg),
           "mfma_flops_executed_per_launch": round(executed),
           "mfma_flops_algorithmic_per_launch": round(alg_per_launch),
           "executed_over_algorithmic": round(executed / alg_per_launch, 4),
           "mfma_busy_frac": round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * simds), 4),
           "kernel_us_per_launch": round(c["duration_ns"] / 1e3, 3),
           "clock_ghz": round(xcd_cycles / c["duration_ns"], 3),
           "mfma_tflops_executed": round(executed / c["duration_ns"] / 1e3, 1),
           "gui_active_cycles_per_launch": round(c["GRBM_GUI_ACTIVE"]),
           "valu_insts_per_launch": round(c.get("SQ_INSTS_VALU", 0)),
           "mfma_insts_per_launch": round(c.get("SQ_INSTS_MFMA", 0))}
    print(json.dumps(out, indent=1))


def summarize_stats(args):
    """Markdown table of a rocprofv3 --kernel-trace --stats run; with
    --stats-json, also the attention kernel's average duration and the split
    combine's time per attention call as JSON (read back by the bench's
    roofline while the kernel source hash matches)."""
    import csv
    with open(os.path.join(args.summarize_stats, "run_kernel_stats.csv")) as f:
        rows = list(csv.DictReader(f))
    print("| kernel | calls | total us | avg us | min us | max us | % of GPU time |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        print(f"| `{name[:70]}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
              f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.1f} |")
    if args.stats_json:
        attn = [r for r in rows if "extend_attn" in r["Name"]]
        comb = [r for r in rows if "combine_splits" in r["Name"]]
        calls = sum(int(r["Calls"]) for r in attn)
        attn_ns = sum(float(r["TotalDurationNs"]) for r in attn)
        comb_ns = sum(float(r["TotalDurationNs"]) for r in comb)
        out = {"workload": args.workload, "kernel_source_sha256_16": kernel_hash(), "attention_calls": calls,
               "extend_attn_avg_us": round(attn_ns / calls / 1e3, 3),
               "combine_us_per_attention_call": round(comb_ns / calls / 1e3, 3),
               "combine_calls": sum(int(r["Calls"]) for r in comb)}
        with open(args.stats_json, "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")


def copy_calibration(args):
    """A plain device copy of a known size (256 MiB read + 256 MiB written per
    launch), to scale the FETCH_SIZE / WRITE_SIZE counters of the kernels."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup + args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "copy_calibration", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": args.warmup + args.steps}), flush=True)


def gemm_calibration(args):
    """What the device's own dense bf16 contraction sustains: torch.matmul
    (hipBLASLt) on square bf16 matrices of 4096, 8192 and 16384, timed with
    events over --steps launches after --warmup. A reference point for the
    attention kernel's fraction of the 2.5 PFLOP/s peak, not a bench line."""
    import torch
    rows = []
    for n in (4096, 8192, 16384):
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(max(args.warmup, 1)):
            c = a @ b
        steps = max(1, args.steps if n < 16384 else args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
        rows.append({"n": n, "ms": round(ms, 4), "tflops": round(tf, 1), "peak_frac": round(tf / MFMA_PEAK_BF16, 4)})
        del a, b, c
    print(json.dumps({"workload": "gemm_calibration", "op": "torch.matmul bf16 (hipBLASLt), square n x n x n",
                      "results": rows}), flush=True)


def cpu_rope_baseline(batches, w, table_np):
    """The CPU oracle's rotary append (oracle/rope.py, as it is) on the step's
    first batch: q and k rows rotated at their positions and written with v
    into the slots of a compact pool; GB/s on the kernel's algorithmic bytes."""
    import numpy as np

    import oracle
    import workloads as wl

    bw = batches[0]
    P, L = np.asarray(bw.prefix_lens, np.int64), np.asarray(bw.chunk_lens, np.int64)
    tq = int(L.sum())
    rng = np.random.default_rng(0)
    mk = lambda *s: wl.to_storage(rng.standard_normal(s).astype(np.float32), w.dtype)  # noqa: E731
    q, k, v = mk(tq, w.num_q_heads, w.head_dim), mk(tq, w.num_kv_heads, w.head_dim), mk(tq, w.num_kv_heads, w.head_dim)
    ps = w.page_size
    npg = [int((p + l + ps - 1) // ps) for p, l in zip(P, L)]
    pt = np.full((len(L), max(npg)), 0, np.int32)
    off = 0
    for b, c in enumerate(npg):
        pt[b, :c] = np.arange(off, off + c)
        off += c
    pool = np.zeros((off, ps, w.num_kv_heads, w.head_dim), wl.storage_np_dtype(w.dtype))
    t0 = time.perf_counter()
    oracle.rope_append(q, k, v, table_np, pool, pool.copy(), pt, P, L, w.dtype)
    dt = time.perf_counter() - t0
    esize = 2 if w.dtype == "bf16" else 4
    nbytes = tq * (2 * esize * w.head_dim * (w.num_q_heads + 2 * w.num_kv_heads) + 4 * w.head_dim)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3), "sample": f"the step's first batch ({tq} tokens), fp64 NumPy rotary oracle"}


def cpu_baseline(w, batches, sample_rows):
    """The CPU oracle, as it is, on a bounded sample of the same workload:
    whole-prompt rows for the long-prompt case (the oracle's result for a row
    does not depend on the chunking), sampled rows otherwise."""
    import numpy as np

    import oracle
    from pkv_testlib import oracle_pools
    import workloads as wl

    cores, blas = blas_info()
    last = batches[-1]
    if len(batches) > 1 and last.batch == 1:    # chunked prompt: the whole prompt as one full prefill
        full = last.with_lengths([0], [int(last.kv_lens[0])])
        pool_w = full
    else:
        full = last
        pool_w = last
    rows_total = int(full.chunk_lens.sum())
    # at most 4 requests (spread over the batch), at most `sample_rows` rows among them
    live = [b for b in range(full.batch) if int(full.chunk_lens[b]) > 0]
    reqs = sorted(set(live[int(i)] for i in np.linspace(0, len(live) - 1, min(4, len(live)))))
    sub = full.subset(reqs)
    sub_qo, _ = oracle.extend_metadata(sub.prefix_lens, sub.chunk_lens)
    n = min(int(sub.chunk_lens.sum()), sample_rows or 4097)
    sub_rows = [int(r) for r in np.unique(np.linspace(0, int(sub.chunk_lens.sum()) - 1, n).astype(np.int64))]
    # compact pool for the sampled requests
    npg = [(int(n_) + sub.page_size - 1) // sub.page_size for n_ in sub.kv_lens]
    pt = np.full((sub.batch, max(npg)), -1, np.int32)
    off = 0
    for b, c in enumerate(npg):
        pt[b, :c] = np.arange(off, off + c)
        off += c
    import dataclasses
    sub = dataclasses.replace(sub, page_table=pt, num_pages=off)
    kp, vp = oracle_pools(sub)
    q = wl.values(sub.q_all(), sub.dtype)
    kf, vf = wl.values(kp, sub.dtype), wl.values(vp, sub.dtype)
    t0 = time.perf_counter()
    oracle.extend_attention(q, kf, vf, sub.page_table, sub.prefix_lens, sub.chunk_lens, window=sub.window,
                            rows=sub_rows)
    dt = time.perf_counter() - t0
    flops = 0
    for r in sub_rows:
        b = int(np.searchsorted(sub_qo, r, side="right") - 1)
        pos = int(sub.prefix_lens[b]) + r - int(sub_qo[b])
        vis = pos + 1 if sub.window <= 0 else min(pos + 1, sub.window)
        flops += 4 * sub.head_dim * sub.num_q_heads * vis
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3), "tokens_per_s": round(len(sub_rows) / dt, 2), "blas": blas,
            "sample": f"{len(sub_rows)} of {rows_total} query rows (all heads), fp32 NumPy oracle"}


def blas_info():
    """(threads the BLAS runs with, its vendor / version / threading as one string)."""
    import numpy  # noqa: F401  (loads the BLAS that threadpoolctl then reports)
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # noqa: BLE001
        libs = []
    if not libs:
        return len(os.sched_getaffinity(0)), "unknown"
    b = libs[0]
    desc = (f"{b.get('internal_api', '?')} {b.get('version', '?')} ({b.get('threading_layer', '?')}, "
            f"{b.get('num_threads', '?')} threads, {b.get('architecture', '?')} kernels)")
    return int(b.get("num_threads", 1)), desc


if __name__ == "__main__":
    main()
