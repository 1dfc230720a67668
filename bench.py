#!/usr/bin/env python3
"""Benchmark of one block-sparse global-attention layer on one MI355X.

Workload: the VGGT-shaped global layer at 32 frames of 518x518 (37x37 patches
+ 5 special tokens per frame = 43,968 tokens), 16 heads, d_h = 64, bf16,
b = 128, rho = 0.75, tau = 0.9, with the planted-correspondence generator and
10 % sink keys (synthetic; inputs resident in HBM before timing).

One step = the whole hot path through the C ABI (the kernels bsga_layer
runs), on two streams: bsga_predict_mask -> bsga_select on the launch stream,
bsga_pack_kv -> bsga_special_rows_packed beside them on a side stream, then
bsga_patch_rows_packed once the mask and the packed K/V are ready.  The layer
time is measured over steps without any event inside them; a second pass of
the same steps with HIP events around each call, on its stream, gives the
per-call times, among them the patch-row call's (block-sparse attention over
the kept blocks plus the special keys, with the rows of the last, partial
round of workgroups split into key-range pieces, and the merge of those
pieces).

Prints ONE JSON line.  `value` is the layer's effective TFLOP/s:
4 * 64 * (computed score entries) / layer time, counting kept patch-patch
entries with exact block sizes plus every special-token entry.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HEAD_DIM = 64
# algorithmic flops of the backward per computed (query, key) entry: the five
# products S = QK^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q, dQ += dS K,
# 2 * d_h each (recomputation and hi + lo splits not counted)
BWD_FLOP_PER_ENTRY = 10 * HEAD_DIM


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="layer shape index 1..5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense comparison and the tau=0 diagnostic")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (torch.neg into a second "
                         "buffer) 5 times and exit: the reference reading for HBM counters")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "attn_patch_rows_32f_hbm_traffic.txt")
KERNEL_SOURCES = ("attention.hip", "tile_common.hpp", "bsga_internal.hpp")


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_sparse_global_bsga_amd",
                        "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch of the patch-row kernel from the committed counter
    summary, or None when that summary was taken on different kernel sources
    or on another workload."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    fields[key.strip()] = val.strip()
        if fields.get("kernel_source_sha256") != kernel_source_digest():
            return None
        if fields.get("workload") != workload:
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda:0").to(torch.bfloat16)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 2, "bytes_written": n * 2,
                      "launches": 5}), flush=True)


def computed_entries(row_ptr, col_idx, n_patch, block, heads, n_special):
    """Kept patch-patch score entries (exact block sizes) and special entries."""
    B = -(-n_patch // block)
    size = np.full(B, block, dtype=np.int64)
    size[-1] = n_patch - block * (B - 1)
    rp = row_ptr.astype(np.int64)
    rows = len(rp) - 1
    colsz = size[col_idx[:rp[-1]]]
    row_of = np.repeat(np.arange(rows), np.diff(rp))
    per_row = np.bincount(row_of, weights=colsz, minlength=rows).astype(np.int64)
    qsize = np.tile(size, heads)
    pp = int(np.sum(qsize * per_row))
    n = n_patch + n_special
    sp = heads * (n_special * n + n_patch * n_special)
    return pp, sp


def cpu_baseline(x, seconds, layer_entries):
    """The oracle as it stands, on a bounded sample of the same layer: the
    mask of head 0 (pooling, scores, softmax, selection over all its rows)
    plus the attention of as many query blocks of head 0 as fit in about
    `seconds` (patch queries over kept blocks and special keys).  Also an
    extrapolated time for the whole layer: the head's mask time times the
    heads, plus the sample's time per computed entry times the layer's
    computed entries (`layer_entries`, every head, special rows included)."""
    from threadpoolctl import threadpool_info
    from block_sparse_global_bsga_amd import synth
    from oracle import bsga_oracle as O
    cfg = x.cfg
    spec, patch = O.token_roles(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
    q, k, v = (synth.bf16_bits_to_f64(t[0]) for t in (x.q, x.k, x.v))
    t0 = time.perf_counter()
    _, _, _, p = O.predict_head(q[patch], k[patch], cfg.block)
    B = p.shape[0]
    rho0 = float(x.rho_per_head[0]) if x.rho_per_head is not None else cfg.rho
    kk = O.keep_count(B, rho0)
    kept = [O.select_row(p[i].astype(np.float32), kk, cfg.tau)[0] for i in range(B)]
    t_mask = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    order = rng.permutation(B)
    size = np.array([O.block_members(cfg.n_patch, cfg.block, j).shape[0] for j in range(B)])
    entries, done = 0, 0
    t1 = time.perf_counter()
    while done < B and (done < 4 or time.perf_counter() - t0 < seconds):
        i = int(order[done])
        O.layer_head(q, k, v, cfg.frames, cfg.patches_per_frame, cfg.special_per_frame,
                     cfg.block, kept, query_blocks=[i], special_queries=False)
        entries += int(size[i]) * (int(size[kept[i]].sum()) + cfg.n_special)
        done += 1
    t_attn = time.perf_counter() - t1
    dt = t_mask + t_attn
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    layer_ms = (cfg.heads * t_mask + t_attn / entries * layer_entries) * 1e3
    return {"value": 4 * HEAD_DIM * entries / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"numpy float64 oracle, head 0 of the same layer: full mask prediction "
                      f"and selection ({B} rows, {t_mask:.2f} s) plus attention of {done} of {B} "
                      f"query blocks (patch queries over kept blocks + special keys, "
                      f"{t_attn:.1f} s); effective FLOP/s on the attention entries computed",
            "ms_per_layer_extrapolated": round(layer_ms, 1),
            "extrapolation": f"extrapolated, not measured: {cfg.heads} heads x the head-0 mask "
                             f"time + the sample's time per computed entry x the layer's "
                             f"{layer_entries} computed entries (all heads, special rows "
                             f"included)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the per-head "
              "sharding across GPUs is described in the design notes but not built.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch
    from block_sparse_global_bsga_amd import bsga, synth

    cfg = synth.CONFIGS[args.config]
    x = synth.generate(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape = bsga.LayerShape(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame,
                            cfg.heads, cfg.block)
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    q, k, v = up(x.q), up(x.k), up(x.v)
    B = bsga.num_blocks(shape)
    probs = torch.empty((cfg.heads, B, B), dtype=torch.float32, device=dev)
    row_ptr = torch.empty(cfg.heads * B + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(bsga.csr_capacity(shape), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((cfg.heads, cfg.tokens), dtype=torch.float32, device=dev)
    ws_pred = bsga.workspace(shape, bsga.OP_PREDICT_MASK, dev)
    ws_sel = bsga.workspace(shape, bsga.OP_SELECT, dev)
    ws_spec = bsga.workspace(shape, bsga.OP_SPECIAL_DENSE_PACKED, dev)
    ws_patch = bsga.workspace(shape, bsga.OP_PATCH_ROWS_PACKED, dev)
    kv = torch.empty(bsga.packed_kv_bytes(shape) + 256, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    side = torch.cuda.Stream(device=dev)  # default priority, like every stream here
    stages = ("predict_mask", "select", "pack_kv", "special_rows", "patch_rows")
    on_side = ("pack_kv", "special_rows")
    fork_ev, packed_ev, side_ev = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()

    def step(rho, tau, ev=None):
        """One layer.  The mask (predict_mask, select) is built on the launch
        stream while a side stream packs K/V and computes the special rows,
        which need only Q and the packed K/V; the patch rows wait for both
        the mask and the packed K/V, and the step ends when both streams are
        done.  ev: per stage a (start, end) pair of timing events, recorded on
        the stream the stage runs on."""
        def rec(name, i):
            if ev is not None:
                ev[name][i].record(side if name in on_side else stream)
        fork_ev.record(stream)
        side.wait_event(fork_ev)
        with torch.cuda.stream(side):
            rec("pack_kv", 0)
            bsga.pack_kv(shape, k, v, kv=kv)
            rec("pack_kv", 1)
            packed_ev.record(side)
            rec("special_rows", 0)
            bsga.special_rows_packed(shape, q, kv, o, lse, ws=ws_spec)
            rec("special_rows", 1)
            side_ev.record(side)
        rec("predict_mask", 0)
        bsga.predict_mask(shape, q, k, probs=probs, ws=ws_pred)
        rec("predict_mask", 1)
        rec("select", 0)
        bsga.select(shape, probs, rho, tau, x.rho_per_head, row_ptr=row_ptr, col_idx=col_idx,
                    ws=ws_sel)
        rec("select", 1)
        stream.wait_event(packed_ev)
        rec("patch_rows", 0)
        bsga.patch_rows_packed(shape, q, kv, row_ptr, col_idx, o, lse, ws=ws_patch)
        rec("patch_rows", 1)
        stream.wait_event(side_ev)

    def timed(fn, steps, warmup, with_stage_events=False):
        """Average ms per step over `steps` timed steps, plus (optionally) the
        average ms of each stage from HIP events recorded on the stream the
        stage was launched on."""
        for _ in range(warmup):
            fn(None)
        torch.cuda.synchronize()
        mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        evs = [{name: (mk(), mk()) for name in stages} for _ in range(steps)] \
            if with_stage_events else [None] * steps
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            fn(evs[i])
        stop.record(stream)
        torch.cuda.synchronize()
        total = start.elapsed_time(stop) / steps
        per = None
        if with_stage_events:
            per = {name: sum(e[name][0].elapsed_time(e[name][1]) for e in evs) / steps
                   for name in stages}
        return total, per

    def timed_marks(fn, steps, warmup, marks):
        """Average ms per step and per interval between `marks` events."""
        for _ in range(warmup):
            fn(None)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)] for _ in range(steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            fn(evs[i])
        stop.record(stream)
        torch.cuda.synchronize()
        parts = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j in range(marks - 1)]
        return start.elapsed_time(stop) / steps, parts

    print(f"# warmup {args.warmup} + {args.steps} timed layer steps, {cfg.name}", file=sys.stderr,
          flush=True)
    # the layer time comes from steps without stage events (each event is a
    # marker packet that idles its stream for a few microseconds); the
    # per-stage times, the patch-row kernel's included, from a second pass
    # of the same steps with them
    ms, _ = timed(lambda ev: step(cfg.rho, cfg.tau, ev), args.steps, args.warmup)
    _, stage_ms = timed(lambda ev: step(cfg.rho, cfg.tau, ev), args.steps, 2, True)
    kern_ms = stage_ms["patch_rows"]
    rp = row_ptr.cpu().numpy()
    ci = col_idx[:int(rp[-1])].cpu().numpy()
    pp, sp = computed_entries(rp, ci, cfg.n_patch, cfg.block, cfg.heads, cfg.n_special)
    n = cfg.tokens
    tok_bytes = cfg.heads * HEAD_DIM * 2  # one token row of every head, bf16
    density = (pp + sp) / (cfg.heads * n * n)
    layer_tflops = 4 * HEAD_DIM * (pp + sp) / (ms * 1e-3) / 1e12
    # the patch-row kernel computes the kept patch-patch entries plus N_p x N_s
    # special-key entries per head
    kern_entries = pp + cfg.heads * cfg.n_patch * cfg.n_special
    kern_tflops = 4 * HEAD_DIM * kern_entries / (kern_ms * 1e-3) / 1e12
    print(f"# layer {ms:.3f} ms, sparse kernel {kern_ms:.3f} ms ({kern_tflops:.0f} TFLOP/s), "
          f"density {density:.4f}", file=sys.stderr, flush=True)

    extras = {}
    if not args.no_extras:
        def dense_step(_ev):
            bsga.pack_kv(shape, k, v, kv=kv)
            bsga.dense_attn_packed(shape, q, kv, o, lse)
        dense_ms, _ = timed(dense_step, max(3, args.steps // 2), 2)
        bufs = bsga.LayerBuffers(shape, dev)
        layer_call_ms, _ = timed(lambda _ev: bsga.layer(shape, q, k, v, cfg.rho, cfg.tau,
                                                        x.rho_per_head, bufs=bufs),
                                 args.steps, 2)
        # the two-stream step must reproduce bsga_layer (one stream) byte for byte
        step(cfg.rho, cfg.tau)
        torch.cuda.synchronize()
        same_as_layer = bool(torch.equal(o.view(torch.int16), bufs.o.view(torch.int16))
                             and torch.equal(lse, bufs.lse)
                             and torch.equal(row_ptr, bufs.row_ptr))
        if not same_as_layer:
            print("# WARNING: two-stream step differs from bsga_layer", file=sys.stderr,
                  flush=True)
        ms0, st0 = timed(lambda ev: step(cfg.rho, 0.0, ev), max(3, args.steps // 2), 2, True)
        kern0 = st0["patch_rows"]
        rp0 = row_ptr.cpu().numpy()
        pp0, sp0 = computed_entries(rp0, col_idx[:int(rp0[-1])].cpu().numpy(), cfg.n_patch,
                                    cfg.block, cfg.heads, cfg.n_special)
        print(f"# dense {dense_ms:.3f} ms; bsga_layer call {layer_call_ms:.3f} ms; "
              f"tau=0: {ms0:.3f} ms", file=sys.stderr, flush=True)
        # per-step latency, median of single steps: warm caches, and with 512 MB
        # written between steps so that neither L2 nor MALL (256 MB) still
        # holds the layer's K/V
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def step_latencies(flushed, reps):
            out = []
            for i in range(reps):
                if flushed:
                    flush.fill_(i & 255)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step(cfg.rho, cfg.tau)
                e1.record(stream)
                torch.cuda.synchronize()
                out.append(e0.elapsed_time(e1))
            return float(np.median(out))

        lat_reps = max(5, args.steps)
        warm_median = step_latencies(False, lat_reps)
        flushed_median = step_latencies(True, lat_reps)
        del flush
        print(f"# single-step median: warm {warm_median:.3f} ms, flushed {flushed_median:.3f} ms",
              file=sys.stderr, flush=True)
        # query-probe Top-K lists (1 % of the patch keys) and the attention over them
        topk = max(1, cfg.n_patch // 100)
        ws_probe = bsga.workspace(shape, bsga.OP_PROBE_SELECT, dev)

        def probe_step(ev):
            mark = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
            mark(0)
            bsga.probe_select(shape, q, k, topk, row_ptr=row_ptr, col_idx=col_idx, ws=ws_probe)
            mark(1)
            bsga.pack_kv(shape, k, v, kv=kv)
            bsga.patch_rows_packed(shape, q, kv, row_ptr, col_idx, o, lse, ws=ws_patch)
            bsga.special_rows_packed(shape, q, kv, o, lse, ws=ws_spec)
            mark(2)

        probe_ms, probe_parts = timed_marks(probe_step, max(3, args.steps // 2), 2, 3)
        rpp = row_ptr.cpu().numpy()
        ppp, spp = computed_entries(rpp, col_idx[:int(rpp[-1])].cpu().numpy(), cfg.n_patch,
                                    cfg.block, cfg.heads, cfg.n_special)
        probe_bytes = tok_bytes * (n + cfg.n_patch) + cfg.heads * cfg.n_patch * 4
        # sparse-vs-dense NMSE per head type, with and without the dense special path
        o_dense, _ = bsga.dense_attn(shape, q, k, v)
        ws_nmse = bsga.workspace(shape, bsga.OP_NMSE, dev)
        nm_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        layer_std = bsga.layer(shape, q, k, v, cfg.rho, cfg.tau, x.rho_per_head, bufs=bufs)
        nm_ev[0].record(stream)
        nm_std = bsga.nmse(shape, o_dense, layer_std.o, ws=ws_nmse)
        nm_ev[1].record(stream)
        pooled = bsga.pooled_specials_shape(shape)
        layer_pool = bsga.layer(pooled, q, k, v, cfg.rho, cfg.tau, x.rho_per_head)
        nm_pool = bsga.nmse(shape, o_dense, layer_pool.o, ws=ws_nmse)
        torch.cuda.synchronize()
        nmse_ms = nm_ev[0].elapsed_time(nm_ev[1])
        by_type = {}
        for name, vals in (("standard", nm_std), ("pooled_specials", nm_pool)):
            vals = vals.cpu().numpy()
            by_type[name] = {t: float(np.mean([vals[h] for h in range(cfg.heads)
                                              if x.head_types[h] == t]))
                             for t in sorted(set(x.head_types))}
        del layer_pool
        # backward of the layer's attention for the standard layer's mask
        d_o = up(synth.fp32_to_bf16_bits(np.random.default_rng(5).standard_normal(
            (cfg.heads, n, HEAD_DIM), dtype=np.float32)))
        ws_bwd = bsga.workspace(shape, bsga.OP_BACKWARD, dev)
        grads = [torch.empty((cfg.heads, n, HEAD_DIM), dtype=torch.float32, device=dev)
                 for _ in range(3)]
        bwd_ms, _ = timed(lambda _ev: bsga.attn_backward(
            shape, q, k, v, layer_std.o, layer_std.lse, d_o, layer_std.row_ptr,
            layer_std.col_idx, dq=grads[0], dk=grads[1], dv=grads[2], ws=ws_bwd),
            max(3, args.steps // 2), 2)
        rpb = layer_std.row_ptr.cpu().numpy()
        ppb, spb = computed_entries(rpb, layer_std.col_idx[:int(rpb[-1])].cpu().numpy(),
                                    cfg.n_patch, cfg.block, cfg.heads, cfg.n_special)
        bwd_tflops = BWD_FLOP_PER_ENTRY * (ppb + spb) / (bwd_ms * 1e-3) / 1e12
        print(f"# backward {bwd_ms:.3f} ms ({bwd_tflops:.0f} TFLOP/s)", file=sys.stderr,
              flush=True)
        # training mode: the forward writes float32 rows (P V with P as a
        # float16 pair hi + lo), and the backward takes D = dO . O from them
        bufs_t = bsga.LayerBuffers(shape, dev)
        o32 = torch.empty((cfg.heads, n, HEAD_DIM), dtype=torch.float32, device=dev)
        train_ms, _ = timed(lambda _ev: bsga.layer_train(shape, q, k, v, cfg.rho, cfg.tau,
                                                         x.rho_per_head, bufs=bufs_t, o32=o32),
                            max(3, args.steps // 2), 2)
        bwd32_ms, _ = timed(lambda _ev: bsga.attn_backward(
            shape, q, k, v, o32, bufs_t.lse, d_o, bufs_t.row_ptr, bufs_t.col_idx,
            dq=grads[0], dk=grads[1], dv=grads[2], ws=ws_bwd), max(3, args.steps // 2), 2)
        bwd32_tflops = BWD_FLOP_PER_ENTRY * (ppb + spb) / (bwd32_ms * 1e-3) / 1e12
        print(f"# training: layer {train_ms:.3f} ms + backward from o32 {bwd32_ms:.3f} ms",
              file=sys.stderr, flush=True)
        del grads, ws_bwd, d_o, bufs_t, o32
        extras = {
            "probe_topk": {"topk": topk, "select_ms": round(probe_parts[0], 4),
                           "select_GB/s": round(probe_bytes / (probe_parts[0] * 1e-3) / 1e9, 1),
                           "attention_ms": round(probe_parts[1], 4),
                           "density": round((ppp + spp) / (cfg.heads * n * n), 4)},
            "nmse_vs_dense_by_head_type": by_type,
            "nmse_kernel": {"ms": round(nmse_ms, 4),
                            "GB/s": round(2 * tok_bytes * n / (nmse_ms * 1e-3) / 1e9, 1)},
            "backward": {"ms": round(bwd_ms, 4),
                         "flop_per_entry": BWD_FLOP_PER_ENTRY,
                         "TFLOP/s": round(bwd_tflops, 1),
                         "frac_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4)},
            "training": {"note": "bsga_layer_train (float32 rows, P V with P as an fp16 "
                                 "pair hi + lo) then bsga_attn_backward_o32 (D = dO . O from "
                                 "them); compare bsga_layer + bsga_attn_backward",
                         "layer_train_ms": round(train_ms, 4),
                         "backward_o32_ms": round(bwd32_ms, 4),
                         "backward_o32_TFLOP/s": round(bwd32_tflops, 1),
                         "backward_o32_frac_peak": round(bwd32_tflops / PEAK_BF16_TFLOPS, 4),
                         "forward_plus_backward_ms": round(train_ms + bwd32_ms, 4),
                         "inference_forward_plus_backward_ms": round(layer_call_ms + bwd_ms, 4)},
            "step_latency_median_ms": {"warm": round(warm_median, 4),
                                       "flushed_512MB": round(flushed_median, 4),
                                       "steps": lat_reps},
            "dense_ms": round(dense_ms, 4),
            "speedup_vs_dense": round(dense_ms / ms, 3),
            "bsga_layer_call_ms": round(layer_call_ms, 4),
            "step_equals_bsga_layer": same_as_layer,
            "diag_tau0": {"note": "diagnostic, not a config: tau=0 so the top-k budget binds",
                          "ms": round(ms0, 4),
                          "density": round((pp0 + sp0) / (cfg.heads * n * n), 4),
                          "speedup_vs_dense": round(dense_ms / ms0, 3),
                          "sparse_kernel_tflops": round(
                              4 * HEAD_DIM * (pp0 + cfg.heads * cfg.n_patch * cfg.n_special)
                              / (kern0 * 1e-3) / 1e12, 1)},
        }

    # algorithmic HBM bytes of the bandwidth-bound stages (bf16 = 2 bytes)
    nnz = int(rp[-1])
    stage_bytes = {
        "predict_mask": 2 * cfg.n_patch * tok_bytes + cfg.heads * B * B * 4,
        "select": cfg.heads * B * B * 4 + (cfg.heads * B + 1 + nnz) * 4,
        "pack_kv": 4 * n * tok_bytes,
    }
    stages_out = {}
    for name, t in stage_ms.items():
        e = {"ms": round(t, 4)}
        if name in stage_bytes:
            e["algorithmic_bytes"] = stage_bytes[name]
            e["GB/s"] = round(stage_bytes[name] / (t * 1e-3) / 1e9, 1)
        stages_out[name] = e
    stages_out["special_rows"]["TFLOP/s"] = round(
        4 * HEAD_DIM * cfg.heads * cfg.n_special * n / (stage_ms["special_rows"] * 1e-3) / 1e12, 1)
    stages_out["patch_rows"]["TFLOP/s"] = round(kern_tflops, 1)

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(x, args.cpu_seconds, pp + sp)

    out = {
        "metric": "ms/global-attn layer + effective TFLOP/s (frac bf16 peak), 32 frames rho=0.75",
        "value": round(layer_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.frames} frames x ({cfg.patches_per_frame} patch "
                               f"+ {cfg.special_per_frame} special) = {n} tokens, {cfg.heads} heads, "
                               f"d_h 64, b {cfg.block}, rho {cfg.rho}, tau {cfg.tau}",
                   "tokens": n, "heads": cfg.heads, "block": cfg.block, "rho": cfg.rho,
                   "tau": cfg.tau, "parallelism": "none (1 GPU)"},
        "layer_frac_peak": round(layer_tflops / PEAK_BF16_TFLOPS, 4),
        "density": round(density, 4),
        "roofline": {"bound": "mfma",
                     "kernel": ("attn_kernel<128, 128, kSparseTail> + tail_merge_kernel "
                                "(bsga_patch_rows_packed)" if cfg.block == 128 else
                                "pair_csr_kernel + attn_kernel<128, 128, PAIR> over aligned "
                                "pairs of 64-blocks (bsga_patch_rows_packed)"),
                     "achieved": round(kern_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
                     "kernel_ms": round(kern_ms, 4), "traffic": recorded_traffic(cfg.name)},
        "stages": stages_out,
        "cpu_baseline": cpu,
        **extras,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
