#!/usr/bin/env python3
"""INT2-KV decode attention on one MI355X: microseconds per step and achieved
HBM GB/s at 100K context, batch 32 (default) and batch 1.

A step is one pass of the whole hot path over one decode token per sequence:
for every layer, the fused write kernel appends the new token (demoting the
oldest recent-window token into rotated INT2 history), then decode attention
runs over the mixed-precision pool (query pre-rotation, split-K INT2 history
scan, BF16 sink/recent segment, log-sum-exp merge with R_V^T).

All inputs are seeded synthetic data (bit_rotated_kv_int2_amd.synth) already
resident in HBM when timing starts.  Per-layer caches are distinct, so every
layer streams from HBM rather than the 256 MB last-level cache.

The timed steps replay one HIP graph of the step (the host-side launch
overhead would otherwise show at batch 1); the same steps launched one call
at a time are timed too (``ms_per_step_eager``).

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: the benchmark
measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT2-KV decode attention µs/step + achieved HBM GB/s at 100K ctx, batch 1/32"
HBM_PEAK_GBPS = 8000.0
D = 128
HIST_BYTES_PER_TOKEN_HEAD = 72      # 64 B codes (K+V) + 8 B metadata codes (K+V, 16 bits per group)

# HBM traffic of the scan kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# recorded with a hash of the kernel sources it was measured on; reported
# only while those sources are unchanged.
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "decode_scan_kernel_traffic.json")
TRAFFIC_SOURCES = ("bit_rotated_kv_int2_amd/csrc/oscar_decode_kernels.hip", "bit_rotated_kv_int2_amd/csrc/oscar_internal.h",
                   "bit_rotated_kv_int2_amd/csrc/oscar_wave.h", "include/oscar.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """Scaled HBM bytes per scan launch for this workload, or None when the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch", {}).get(workload)
WIN_BYTES_PER_TOKEN_HEAD = 512      # bf16 K + V


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# workload construction (plumbing: device memory via torch, compute via liboscar)
# ---------------------------------------------------------------------------

def gpu_kv(torch, synth, wl, layer, seq, L):
    """Seeded bf16 K/V bits [L, Hkv, d] (int16) of one sequence, on the GPU."""
    return synth.gpu_sequence_kv(wl, layer, seq, L, "cuda")


def calibrate_layer(O, synth, wl, layer, params, n_cal):
    q, k, v = synth.calibration_set(wl, layer, n_cal=n_cal)
    f = synth.bf16_bits_to_f32
    UK, UV, tK, tV = O.calibrate_rotation(params, f(q), f(k), f(v))
    return O.RotationTensors.from_numpy(UK, UV, tK, tV, "cuda")


class Workbench:
    def __init__(self, wl, n_layers, extra_tokens, n_cal, bf16_budget_gb, variant=0):
        import torch
        from bit_rotated_kv_int2_amd import oscar as O
        from bit_rotated_kv_int2_amd import synth
        self.torch, self.O, self.synth = torch, O, synth
        self.wl = wl
        self.params = O.make_params(wl.n_kv, wl.n_q)
        self.lengths = synth.sequence_lengths(wl)
        self.bt, self.total_pages = synth.block_table(wl, self.lengths, extra_tokens)
        self.n_layers = n_layers
        self.layers = []
        t0 = time.time()
        for layer in range(n_layers):
            rot = calibrate_layer(O, synth, wl, layer, self.params, n_cal)
            pool = O.KVPool(self.params, wl.batch, self.total_pages, self.bt, zero_pages=False)
            for b in range(wl.batch):
                k, v = gpu_kv(torch, synth, wl, layer, b, int(self.lengths[b]))
                O.quantize_append(self.params, rot, pool, k[None], v[None], seq=b)
                del k, v
            torch.cuda.synchronize()
            assert int(pool.error_flags.item()) == 0
            self.layers.append((rot, pool))
            if layer % 6 == 5 or layer == n_layers - 1:
                log(f"{wl.name}: built INT2 layer {layer + 1}/{n_layers} ({time.time() - t0:.1f}s)")
        self.variant = variant
        self.ws = O.alloc_workspace(O.decode_workspace_size(self.params, wl.batch, self.bt.shape[1], variant))
        self.out = torch.zeros((wl.batch, wl.n_q, D), dtype=torch.float32, device="cuda")
        # BF16 baseline caches holding the same token contents (as many layers as the budget allows)
        per_layer = float(np.sum(self.lengths)) * wl.n_kv * WIN_BYTES_PER_TOKEN_HEAD
        self.n_bf16 = int(max(1, min(n_layers, bf16_budget_gb * 1e9 // max(per_layer, 1))))
        self.bf16 = []
        pages16 = [(int(L) + 63) // 64 for L in self.lengths]
        mp16 = max(pages16)
        bt16 = np.full((wl.batch, mp16), -1, np.int32)
        perm = synth.rng(wl, 0, synth.STREAM_PERM, 16).permutation(sum(pages16)).astype(np.int32)
        nxt = 0
        for b, n in enumerate(pages16):
            bt16[b, :n] = perm[nxt:nxt + n]
            nxt += n
        self.bt16 = bt16
        for layer in range(self.n_bf16):
            cache = O.Bf16Cache(self.params, wl.batch, sum(pages16), bt16)
            for b in range(wl.batch):
                L = int(self.lengths[b])
                k, v = gpu_kv(torch, synth, wl, layer, b, L)
                n = pages16[b]
                pad = n * 64 - L
                for src, dst in ((k, cache.k_pages), (v, cache.v_pages)):
                    if pad:
                        src = torch.cat([src, torch.zeros((pad, wl.n_kv, D), dtype=src.dtype, device="cuda")])
                    blk = src.view(n, 64, wl.n_kv, D).permute(0, 2, 1, 3)
                    idx = torch.from_numpy(bt16[b, :n].astype(np.int64)).cuda()
                    dst.index_copy_(0, idx, blk.contiguous())
                del k, v
            cache.seq_lens.copy_(torch.from_numpy(self.lengths.astype(np.int32)))
            self.bf16.append(cache)
        torch.cuda.synchronize()
        self.ws16 = O.alloc_workspace(max(O.bf16_workspace_size(self.params, bb, mp16)
                                          for bb in range(1, wl.batch + 1)))
        log(f"{wl.name}: built {self.n_bf16} BF16 baseline layers ({time.time() - t0:.1f}s total)")

    # --- byte accounting -----------------------------------------------------
    def hist_bytes(self, lengths):
        n_hist = np.maximum(0, lengths.astype(np.int64) - self.wl.sink - self.wl.recent)
        return int(np.sum(n_hist)) * self.wl.n_kv * HIST_BYTES_PER_TOKEN_HEAD

    def scan_bytes(self, lengths):
        """Algorithmic HBM bytes of one scan-kernel launch: INT2 history pages,
        BF16 sink and recent windows, and the fp32 output."""
        wl = self.wl
        win = np.minimum(lengths.astype(np.int64), wl.sink + wl.recent)
        return (self.hist_bytes(lengths) + int(np.sum(win)) * wl.n_kv * WIN_BYTES_PER_TOKEN_HEAD
                + wl.batch * wl.n_q * D * 4)

    def layer_step_bytes(self, lengths):
        """Algorithmic HBM bytes of one layer of one step (append + decode)."""
        wl = self.wl
        win = np.minimum(lengths.astype(np.int64), wl.sink + wl.recent)
        b = self.hist_bytes(lengths) + int(np.sum(win)) * wl.n_kv * WIN_BYTES_PER_TOKEN_HEAD
        b += wl.batch * wl.n_q * D * (2 + 4)                      # q in, out
        b += 2 * wl.n_kv * D * D * 4                              # U_K, U_V
        b += wl.batch * wl.n_kv * 2 * (256 + 256 + 256 + 40)      # append: new in, ring in/out, codes+meta out
        return b


def graph_extra_tokens(steps):
    """Tokens per sequence the graph-replayed steps append (one warm replay
    plus the timed ones)."""
    return steps + 1


def run_workload(wb, steps, warmup, decode_reps, bf16_fit=None):
    torch, O = wb.torch, wb.O
    wl = wb.wl
    nl = wb.n_layers
    total = warmup + steps
    # per-layer per-step new tokens and queries
    g = torch.Generator(device="cuda")
    g.manual_seed(1234 + wl.wid)
    knew = [torch.randn((total, wl.batch, 1, wl.n_kv, D), generator=g, device="cuda").to(torch.bfloat16)
            .view(torch.int16).contiguous() for _ in range(nl)]
    vnew = [torch.randn((total, wl.batch, 1, wl.n_kv, D), generator=g, device="cuda").to(torch.bfloat16)
            .view(torch.int16).contiguous() for _ in range(nl)]
    qs = [torch.randn((total, wl.batch, wl.n_q, D), generator=g, device="cuda").to(torch.bfloat16)
          .view(torch.int16).contiguous() for _ in range(nl)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps * nl)]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    base = wb.lengths.astype(np.int64)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    wall0 = 0.0
    for s in range(total):
        if s == warmup:
            torch.cuda.synchronize()
            wall0 = time.perf_counter()
            t_start.record()
        for l, (rot, pool) in enumerate(wb.layers):
            O.quantize_append(wb.params, rot, pool, knew[l][s], vnew[l][s])
            # the decode is one kernel launch (MFMA variants) on torch's current
            # stream, so events recorded on that stream around it time the kernel
            if s >= warmup:
                ev[(s - warmup) * nl + l][0].record()
            O.decode_attention(wb.params, rot, pool, qs[l][s], wb.out, wb.ws, variant=wb.variant)
            if s >= warmup:
                ev[(s - warmup) * nl + l][1].record()
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t_start.elapsed_time(t_stop) / steps
    hist_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    for _, pool in wb.layers:
        assert int(pool.error_flags.item()) == 0
    # algorithmic bytes of the timed steps (lengths after the step's append)
    step_bytes = [nl * wb.layer_step_bytes(base + s + 1) for s in range(warmup, total)]
    hist_launch_bytes = [wb.scan_bytes(base + s + 1) for s in range(warmup, total)]

    # decode-only per-layer time (no append), cycling through every layer
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    lens_now = base + total
    d0.record()
    for r in range(decode_reps):
        for l, (rot, pool) in enumerate(wb.layers):
            O.decode_attention(wb.params, rot, pool, qs[l][r % total], wb.out, wb.ws, variant=wb.variant)
    d1.record()
    torch.cuda.synchronize()
    decode_us = d0.elapsed_time(d1) * 1e3 / (decode_reps * nl)
    decode_bytes = wb.layer_step_bytes(lens_now) - wl.batch * wl.n_kv * 2 * (256 + 256 + 256 + 40)

    # BF16 baseline, same token contents, same shapes
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    n16 = max(decode_reps * nl // max(wb.n_bf16, 1), wb.n_bf16) // wb.n_bf16 * wb.n_bf16
    q16 = qs[0][0]
    for c in wb.bf16:   # warm
        O.bf16_decode_attention(wb.params, c, q16, wb.out, wb.ws16)
    b0.record()
    for i in range(n16):
        O.bf16_decode_attention(wb.params, wb.bf16[i % wb.n_bf16], q16, wb.out, wb.ws16)
    b1.record()
    torch.cuda.synchronize()
    bf16_us = b0.elapsed_time(b1) * 1e3 / n16
    bf16_bytes = int(np.sum(wb.lengths)) * wl.n_kv * WIN_BYTES_PER_TOKEN_HEAD
    fit_us = None
    if bf16_fit and bf16_fit < wl.batch:
        views = []
        for c in wb.bf16:
            cc = c.c()
            cc.batch = bf16_fit
            views.append(cc)
        import ctypes
        stream = torch.cuda.current_stream().cuda_stream
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record()
        for i in range(n16):
            O._check(O.lib().oscar_bf16_decode_attention(ctypes.byref(wb.params), ctypes.byref(views[i % len(views)]),
                                                         q16.data_ptr(), wb.out.data_ptr(), wb.ws16.data_ptr(),
                                                         wb.ws16.numel(), stream))
        f1.record()
        torch.cuda.synchronize()
        fit_us = f0.elapsed_time(f1) * 1e3 / n16

    # The same step (every layer: append one token per sequence, then decode)
    # captured once in a HIP graph and replayed: the GPU work of the eager
    # step without the per-launch host overhead (ctypes marshalling and the
    # launch calls, which at batch 1 take longer than some kernels).  Each
    # replay appends one more token per sequence, like a decode loop; the
    # tokens and queries are those of the last eager step.  Run last: the
    # measures above use the lengths the eager steps left.
    lens_g = base + total
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l, (rot, pool) in enumerate(wb.layers):
            O.quantize_append(wb.params, rot, pool, knew[l][total - 1], vnew[l][total - 1])
            O.decode_attention(wb.params, rot, pool, qs[l][total - 1], wb.out, wb.ws, variant=wb.variant)
    g.replay()   # warm
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(steps):
        g.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_step_ms = g0.elapsed_time(g1) / steps
    for _, pool in wb.layers:
        assert int(pool.error_flags.item()) == 0
    graph_bytes = [nl * wb.layer_step_bytes(lens_g + 1 + i + 1) for i in range(steps)]
    del g

    hist_mean_us = float(np.mean(hist_us))
    hist_bytes_mean = float(np.mean(hist_launch_bytes))
    kv_elements = float(np.mean([np.sum(base + s + 1) for s in range(warmup, total)])) * wl.n_kv * D * 2
    return {
        "step_ms": graph_step_ms,
        "value_gbps": float(np.mean(graph_bytes)) / (graph_step_ms * 1e-3) / 1e9,
        "step_ms_eager": step_ms,
        "wall_ms_per_step_eager": wall * 1e3 / steps,
        "value_gbps_eager": float(np.mean(step_bytes)) / (step_ms * 1e-3) / 1e9,
        "scan_kernel_us": hist_mean_us,
        "scan_kernel_us_p10_p90": [float(np.percentile(hist_us, 10)), float(np.percentile(hist_us, 90))],
        "scan_kernel_bytes": hist_bytes_mean,
        "kv_elements": kv_elements,
        "scan_kernel_gbps": hist_bytes_mean / (hist_mean_us * 1e-6) / 1e9,
        "decode_us_per_layer": decode_us,
        "decode_gbps": decode_bytes / (decode_us * 1e-6) / 1e9,
        "bf16_us_per_layer": bf16_us,
        "bf16_gbps": bf16_bytes / (bf16_us * 1e-6) / 1e9,
        "speedup_vs_bf16_decode": bf16_us / decode_us,
        "bytes_per_step": float(np.mean(step_bytes)),
        "bf16_fit_us_per_layer": fit_us,
    }


# ---------------------------------------------------------------------------
# Long shared prefix: bulk quantise-pack of the prefix, then decode
# ---------------------------------------------------------------------------

def run_prefix(n_cal, write_reps=10, decode_reps=20):
    """Batch 16 x 131072 tokens, 8 KV / 96 query heads, one 98304-token
    prefix on shared pages and one shared sink slot; one layer.

    - The bulk prefill-time quantise-pack of the prefix (one append of 98304
      tokens x 8 KV heads through the write kernels) is timed on its own,
      write_reps times into the same pages (seq_lens reset in between; the
      median is reported).
    - Then every sequence is completed and the decode attention timed.
      Logical bytes count the shared pages once per sequence; unique bytes
      count them once."""
    import torch
    from bit_rotated_kv_int2_amd import oscar as O
    from bit_rotated_kv_int2_amd import synth
    wl = synth.WORKLOADS["prefix-128k-b16-gqa12"]
    params = O.make_params(wl.n_kv, wl.n_q)
    rot = calibrate_layer(O, synth, wl, 0, params, n_cal)
    lengths = synth.sequence_lengths(wl)
    bt, total = synth.block_table(wl, lengths)
    pool = O.KVPool(params, wl.batch, total, bt, sink_slot=np.zeros(wl.batch, np.int32), n_sink_slots=1,
                    zero_pages=False)
    P = wl.shared_prefix
    kp, vp = gpu_kv(torch, synth, wl, 0, 0, P)
    kp, vp = kp[None].contiguous(), vp[None].contiguous()
    O.quantize_append(params, rot, pool, kp, vp, seq=0)   # warm
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(write_reps)]
    for e0, e1 in ev:
        pool.seq_lens.zero_()
        e0.record()
        O.quantize_append(params, rot, pool, kp, vp, seq=0)
        e1.record()
    torch.cuda.synchronize()
    assert int(pool.error_flags.item()) == 0 and int(pool.seq_lens[0].item()) == P
    write_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    del kp, vp
    # complete sequence 0 with its private suffix, then every other sequence
    k, v = gpu_kv(torch, synth, wl, 0, 0, int(lengths[0]))
    O.quantize_append(params, rot, pool, k[P:][None].contiguous(), v[P:][None].contiguous(), seq=0)
    del k, v
    for b in range(1, wl.batch):
        k, v = gpu_kv(torch, synth, wl, 0, b, int(lengths[b]))
        O.quantize_append(params, rot, pool, k[None], v[None], seq=b)
        del k, v
    torch.cuda.synchronize()
    assert int(pool.error_flags.item()) == 0
    out = torch.zeros((wl.batch, wl.n_q, D), dtype=torch.float32, device="cuda")
    q = torch.from_numpy(synth.decode_queries(wl, 0).view(np.int16)).cuda()
    shared_pages = (P - wl.sink) // 64   # whole 64-token pages after the sink

    def time_decode(prefix_pages):
        ws = O.alloc_workspace(O.decode_workspace_size(params, wl.batch, pool.max_pages, prefix_pages=prefix_pages))
        O.decode_attention(params, rot, pool, q, out, ws, prefix_pages=prefix_pages)
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record()
        for _ in range(decode_reps):
            O.decode_attention(params, rot, pool, q, out, ws, prefix_pages=prefix_pages)
        d1.record()
        torch.cuda.synchronize()
        assert int(pool.error_flags.item()) == 0
        return d0.elapsed_time(d1) * 1e3 / decode_reps

    dec_us = time_decode(0)
    dec_shared_us = time_decode(shared_pages)
    n_hist = np.maximum(0, lengths.astype(np.int64) - wl.sink - wl.recent)
    win = np.minimum(lengths.astype(np.int64), wl.sink + wl.recent)
    out_bytes = wl.batch * wl.n_q * D * 4
    logical = int(np.sum(n_hist)) * wl.n_kv * HIST_BYTES_PER_TOKEN_HEAD + \
        int(np.sum(win)) * wl.n_kv * WIN_BYTES_PER_TOKEN_HEAD + out_bytes
    shared_hist = (P - wl.sink) * wl.n_kv * HIST_BYTES_PER_TOKEN_HEAD
    unique = logical - (wl.batch - 1) * shared_hist - (wl.batch - 1) * wl.sink * wl.n_kv * WIN_BYTES_PER_TOKEN_HEAD
    return {"workload": wl.name, "prefix_tokens": P, "kv_heads": wl.n_kv,
            "quantize_pack_ms": write_ms,
            "quantize_pack_tokens_per_s": P / (write_ms * 1e-3),
            "quantize_pack_token_heads_per_s": P * wl.n_kv / (write_ms * 1e-3),
            "decode_us_per_layer": dec_us,
            "decode_gbps_logical": logical / (dec_us * 1e-6) / 1e9,
            "decode_gbps_unique": unique / (dec_us * 1e-6) / 1e9,
            "shared_prefix_pages": shared_pages,
            "decode_us_per_layer_shared_prefix": dec_shared_us,
            "decode_gbps_unique_shared_prefix": unique / (dec_shared_us * 1e-6) / 1e9,
            "note": "one layer; logical bytes read the shared prefix once per sequence, unique bytes once; "
                    "decode_us_per_layer: every sequence scans all its pages, "
                    "decode_us_per_layer_shared_prefix: decode option prefix_pages = the shared pages"}


# ---------------------------------------------------------------------------
# 32K context, batch 1: one decode step plus one single-token append
# ---------------------------------------------------------------------------

def run_32k(n_cal, reps=50):
    """One layer of 32768 tokens, 8 KV / 32 query heads.  A single layer
    (22 MB) stays in the 256 MB last-level cache across repeats, so these
    are cache-warm figures: decode alone, the single-token append (one token
    x 8 KV heads through the fused rotate-clip-quantise-pack-demote kernel)
    alone, and the two back to back as one step."""
    import torch
    from bit_rotated_kv_int2_amd import oscar as O
    from bit_rotated_kv_int2_amd import synth
    wl = synth.WORKLOADS["qwen3-8b-32k-b1"]
    params = O.make_params(wl.n_kv, wl.n_q)
    rot = calibrate_layer(O, synth, wl, 0, params, n_cal)
    lengths = synth.sequence_lengths(wl)
    bt, total = synth.block_table(wl, lengths, 3 * reps + 8)
    pool = O.KVPool(params, 1, total, bt, zero_pages=False)
    k, v = gpu_kv(torch, synth, wl, 0, 0, int(lengths[0]))
    O.quantize_append(params, rot, pool, k[None], v[None], seq=0)
    del k, v
    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    kn = torch.randn((3 * reps + 2, 1, 1, wl.n_kv, D), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    vn = torch.randn((3 * reps + 2, 1, 1, wl.n_kv, D), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    q = torch.randn((1, wl.n_q, D), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16).contiguous()
    ws = O.alloc_workspace(O.decode_workspace_size(params, 1, pool.max_pages))
    out = torch.zeros((1, wl.n_q, D), dtype=torch.float32, device="cuda")
    O.decode_attention(params, rot, pool, q, out, ws)
    O.quantize_append(params, rot, pool, kn[0].contiguous(), vn[0].contiguous())
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    e = [ev() for _ in range(6)]
    e[0].record()
    for _ in range(reps):
        O.decode_attention(params, rot, pool, q, out, ws)
    e[1].record()
    for i in range(reps):
        O.quantize_append(params, rot, pool, kn[1 + i].contiguous(), vn[1 + i].contiguous())
    e[2].record()
    for i in range(reps):
        O.quantize_append(params, rot, pool, kn[1 + reps + i].contiguous(), vn[1 + reps + i].contiguous())
        O.decode_attention(params, rot, pool, q, out, ws)
    e[3].record()
    torch.cuda.synchronize()
    assert int(pool.error_flags.item()) == 0
    dec_us = e[0].elapsed_time(e[1]) * 1e3 / reps
    app_us = e[1].elapsed_time(e[2]) * 1e3 / reps
    step_us = e[2].elapsed_time(e[3]) * 1e3 / reps
    L = int(pool.seq_lens.item())
    dec_bytes = (max(0, L - 320) * HIST_BYTES_PER_TOKEN_HEAD + min(L, 320) * WIN_BYTES_PER_TOKEN_HEAD) * wl.n_kv \
        + wl.n_q * D * 4
    return {"workload": wl.name, "context": L, "cache": "warm (one 22 MB layer fits the 256 MB last-level cache)",
            "decode_us": dec_us, "decode_gbps": dec_bytes / (dec_us * 1e-6) / 1e9,
            "append_one_token_us": app_us, "step_us": step_us}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle's decode on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def _oracle_decode_times(wl, pairs, reps, host_kv=False):
    """Wall seconds of `reps` oracle decodes of each (sequence, KV head) pair
    at full length, and the algorithmic bytes those decodes stand for.  The
    pool of each pair is built (oracle write path) outside the timed calls."""
    import torch
    from bit_rotated_kv_int2_amd import synth
    from oracle import oscar_ref as R
    lengths = synth.sequence_lengths(wl)
    G = wl.n_q // wl.n_kv
    q_all = synth.decode_queries(wl, 0)
    qc, kc, vc = synth.calibration_set(wl, 0, n_cal=512)
    f = synth.bf16_bits_to_f32
    times, nbytes = [], 0
    for (b, h) in pairs:
        L = int(lengths[b])
        if host_kv:
            kb, vb = synth.kv_tokens(wl, 0, b, 0, L)
            kh, vh = f(kb[:, h]).astype(np.float64), f(vb[:, h]).astype(np.float64)
        else:
            k, v = gpu_kv(torch, synth, wl, 0, b, L)
            kh = f(k[:, h].cpu().numpy().view(np.uint16)).astype(np.float64)
            vh = f(v[:, h].cpu().numpy().view(np.uint16)).astype(np.float64)
            del k, v
        cal = R.calibrate_head(f(qc[h * G:(h + 1) * G]), f(kc[h]), f(vc[h]), 1 / np.sqrt(D))
        pool = R.build_head_pool(kh, vh, cal)
        q = f(q_all[b, h * G:(h + 1) * G]).astype(np.float64)
        for _ in range(reps):
            t0 = time.perf_counter()
            R.decode_head_dense(q, pool, cal, 1 / np.sqrt(D))
            times.append(time.perf_counter() - t0)
        nbytes += reps * (max(0, L - 320) * HIST_BYTES_PER_TOKEN_HEAD + min(L, 320) * WIN_BYTES_PER_TOKEN_HEAD)
    return times, nbytes


def cpu_baseline(wl, pairs, reps):
    """The oracle (never tuned for speed) timed on the host cores, on a bounded
    sample of the benchmark workload with every BLAS thread, then single
    threaded, plus one-pair samples of the other decode workloads."""
    from bit_rotated_kv_int2_amd import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    except Exception:       # no thread control: numpy runs as configured
        threadpool_limits, blas_threads = None, None
    times, nbytes = _oracle_decode_times(wl, pairs, reps)
    total = float(np.sum(times))
    out = {"value": nbytes / total / 1e9, "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
           "host_cpus": os.cpu_count(), "seconds": total,
           "us_per_head_decode": total / len(times) * 1e6,
           "sample": f"oracle fp64 decode (dequantise + inverse-rotate + softmax attention) of "
                     f"{len(pairs)} (sequence, KV head) pairs of {wl.name} at full length, "
                     f"{reps} runs each, {blas_threads} BLAS threads; GB/s over the same algorithmic "
                     f"bytes as the GPU"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t1, b1 = _oracle_decode_times(wl, pairs[:2], 2)
        out["single_thread"] = {"value": b1 / float(np.sum(t1)) / 1e9, "unit": "GB/s", "cores": 1,
                                "us_per_head_decode": float(np.mean(t1)) * 1e6,
                                "sample": f"2 pairs of {wl.name}, 2 runs each, one thread"}
    others = {}
    for name, host in (("tiny-4k", True), ("qwen3-8b-32k-b1", False), ("qwen3-8b-100k-b1-36l", False)):
        w = synth.WORKLOADS[name]
        prs = [(0, 0)] if w.n_kv == 1 else [(0, 0), (0, 3)]
        t, nb = _oracle_decode_times(w, prs, 5 if w.max_len > 10000 else 20, host_kv=host)
        others[name] = {"us_per_head_decode": float(np.mean(t)) * 1e6, "gbps": nb / float(np.sum(t)) / 1e9,
                        "pairs": len(prs)}
    out["other_workloads"] = others
    return out


def effective_bpe(L, sink=64, recent=256, history_bits=2.0 + 16.0 / 64):
    """Stored bits per KV element: BF16 windows + INT2 codes with 16 metadata bits per 64 channels."""
    win = min(L, sink + recent)
    return (win * 16.0 + (L - win) * history_bits) / L


def _probe_lib():
    """The benchmark-only streaming-read helper library (not part of liboscar.so)."""
    import ctypes
    from bit_rotated_kv_int2_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIB_PATH)
    lib.bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    lib.bench_stream_read.restype = ctypes.c_int
    return lib


def stream_read_ceiling(torch, gib=4, reps=5):
    """Practical HBM read rate: a plain streaming-read kernel over a 4 GiB
    buffer (best of a few grid sizes, HIP events around `reps` launches)."""
    probe = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream

    def read(buf, sink, grid):
        rc = probe.bench_stream_read(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), grid, stream)
        assert rc == 0, rc
    n = gib << 30
    buf = torch.empty(n // 4, dtype=torch.int32, device="cuda").random_()
    best = None
    for grid in (256, 512, 1024):
        sink = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
        read(buf, sink, grid)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            read(buf, sink, grid)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        if best is None or us < best["us"]:
            best = {"grid": grid, "threads": 512, "bytes": n, "us": us, "gbps": n / us / 1e3}
    del buf
    torch.cuda.empty_cache()
    best["frac_of_peak"] = best["gbps"] / HBM_PEAK_GBPS
    return best


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3-8b-100k-b32-36l")
    ap.add_argument("--layers", type=int, default=None, help="override the workload's layer count")
    ap.add_argument("--decode-reps", type=int, default=5)
    ap.add_argument("--n-cal", type=int, default=512)
    ap.add_argument("--no-batch1", action="store_true", help="skip the batch-1 secondary workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefix", action="store_true",
                    help="skip the long shared-prefix workload (bulk quantise-pack + decode)")
    ap.add_argument("--variant", type=int, default=0, help="0 = MFMA int8 history kernel, 1 = VALU reference")
    ap.add_argument("--bf16-budget-gb", type=float, default=48.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="end with one plain device-to-device copy of this many MiB (scales HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "sharding over several GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_rotated_kv_int2_amd import oscar as O
    from bit_rotated_kv_int2_amd import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    O.lib()   # fail loudly if the HIP library is missing

    wl = synth.WORKLOADS[args.workload]
    nl = args.layers or wl.layers
    extra = args.warmup + args.steps + graph_extra_tokens(args.steps)
    wb = Workbench(wl, nl, extra, args.n_cal, args.bf16_budget_gb, args.variant)
    bf16_fit = None
    if wl.batch > 1:
        # sequences an all-BF16 cache of the same layers fits in the HBM the INT2 pool occupies
        int2_bytes = sum(p.pages.numel() + 2 * (p.recent_k.numel() + p.sink_k.numel()) * 2 for _, p in wb.layers)
        per_seq_bf16 = float(np.mean(wb.lengths)) * wl.n_kv * WIN_BYTES_PER_TOKEN_HEAD * nl
        bf16_fit = int(int2_bytes // per_seq_bf16)
    r = run_workload(wb, args.steps, args.warmup, args.decode_reps, bf16_fit)
    log(f"{wl.name}: {json.dumps(r)}")
    del wb
    torch.cuda.empty_cache()

    batch1 = None
    if not args.no_batch1 and wl.batch > 1:
        wl1 = synth.WORKLOADS["qwen3-8b-100k-b1-36l"]
        wb1 = Workbench(wl1, args.layers or wl1.layers, extra, args.n_cal, args.bf16_budget_gb,
                        args.variant)
        r1 = run_workload(wb1, args.steps, args.warmup, args.decode_reps * 4)
        log(f"{wl1.name}: {json.dumps(r1)}")
        batch1 = {"workload": wl1.name, "us_per_step": r1["step_ms"] * 1e3, "gbps": r1["value_gbps"],
                  "us_per_step_eager": r1["step_ms_eager"] * 1e3,
                  "decode_us_per_layer": r1["decode_us_per_layer"], "decode_gbps": r1["decode_gbps"],
                  "decode_frac_of_peak": r1["decode_gbps"] / HBM_PEAK_GBPS,
                  "scan_kernel_us": r1["scan_kernel_us"], "scan_kernel_gbps": r1["scan_kernel_gbps"],
                  "scan_kernel_frac_of_peak": r1["scan_kernel_gbps"] / HBM_PEAK_GBPS,
                  "bf16_us_per_layer": r1["bf16_us_per_layer"], "bf16_gbps": r1["bf16_gbps"],
                  "speedup_vs_bf16_decode": r1["speedup_vs_bf16_decode"],
                  "scan_kernel_traffic": measured_traffic(wl1.name)}
        del wb1
        torch.cuda.empty_cache()

    ctx32k = None
    if not args.no_batch1:
        ctx32k = run_32k(args.n_cal)
        log(f"32k: {json.dumps(ctx32k)}")

    prefix = None
    if not args.no_prefix:
        prefix = run_prefix(args.n_cal)
        # HBM bytes the scan fetched and wrote per launch (counters), next to
        # the logical and unique bytes
        prefix["scan_kernel_traffic"] = measured_traffic(prefix["workload"])
        log(f"prefix: {json.dumps(prefix)}")
        torch.cuda.empty_cache()

    ceiling = stream_read_ceiling(torch)
    log(f"stream read ceiling: {json.dumps(ceiling)}")

    cpu = None
    if not args.no_cpu_baseline:
        # about 7 s of oracle decode: 8 (sequence, KV head) pairs at full length, 10 runs each,
        # then a few seconds single threaded and on the other decode workloads
        pairs = ([(b, (3 * b) % wl.n_kv) for b in range(8)] if wl.batch >= 8 else
                 [(0, h) for h in range(min(8, wl.n_kv))])
        cpu = cpu_baseline(wl, pairs, reps=10)

    traffic = measured_traffic(wl.name)
    line = {
        "metric": METRIC,
        "value": r["value_gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "dtype_detail": "INT2 history codes on int8xint8->int32 MFMA; fp32 softmax/accumulation; bf16 windows",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "layers": nl, "kv_heads": wl.n_kv,
                   "q_heads": wl.n_q, "head_dim": D, "context": [wl.min_len, wl.max_len],
                   "page_tokens": 64, "scattered_pages": wl.scattered_pages, "parallelism": "single-gpu"},
        "us_per_step": r["step_ms"] * 1e3,
        "step_contents": "per layer: append 1 token/sequence (fused rotate-clip-quantise-pack-demote) + decode attention",
        "step_timing": "the step captured once in a HIP graph, replayed K times between events",
        "ms_per_step_eager": r["step_ms_eager"],
        "value_eager": r["value_gbps_eager"],
        "decode_us_per_layer": r["decode_us_per_layer"],
        "decode_gbps": r["decode_gbps"],
        "decode_frac_of_peak": r["decode_gbps"] / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "kernel": "decode_scan_kernel (split-K INT2 history + BF16 windows + merge)",
                     "achieved": r["scan_kernel_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": r["scan_kernel_gbps"] / HBM_PEAK_GBPS, "traffic": traffic,
                     "kv_elements_per_launch": r["kv_elements"],
                     "algorithmic_bytes_per_kv_element": r["scan_kernel_bytes"] / r["kv_elements"],
                     "fetched_bytes_per_kv_element": (None if traffic is None else traffic / r["kv_elements"]),
                     "bytes_per_launch": r["scan_kernel_bytes"], "us_per_launch": r["scan_kernel_us"],
                     "us_p10_p90": r["scan_kernel_us_p10_p90"],
                     "stream_read_ceiling_gbps": ceiling["gbps"],
                     "frac_of_stream_read_ceiling": r["scan_kernel_gbps"] / ceiling["gbps"]},
        "bf16_baseline": {"us_per_layer": r["bf16_us_per_layer"], "gbps": r["bf16_gbps"],
                          "speedup_vs_bf16_decode": r["speedup_vs_bf16_decode"],
                          "bf16_batch_in_same_hbm": bf16_fit,
                          "bf16_us_per_layer_at_that_batch": r["bf16_fit_us_per_layer"],
                          "job_throughput_ratio": (None if not r["bf16_fit_us_per_layer"] else
                                                   (wl.batch / r["decode_us_per_layer"]) /
                                                   (bf16_fit / r["bf16_fit_us_per_layer"]))},
        "effective_bits_per_kv_element": round(effective_bpe(float(np.mean(synth.sequence_lengths(wl)))), 4),
        "pages_bits_per_kv_element": 2.28,
        "batch1": batch1,
        "ctx32k_batch1": ctx32k,
        "long_prefix": prefix,
        "cpu_baseline": cpu,
    }
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = n
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
