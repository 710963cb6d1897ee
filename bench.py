#!/usr/bin/env python3
"""Benchmark of the ReHyAt hybrid attention forward on one MI355X.

One step = one whole-clip forward (block-state pass, cross-chunk scan, local
softmax + fused combine) over the Wan2.1-1.3B attention shape: B=1, H=12,
head_dim=128, 21 latent frames of 30x52 = 1560 tokens (a 5 s 480x832 clip),
T_c = 3, T_o = 1, elu+1 features, bf16 in/out with fp32 accumulation, q/k/v
resident in HBM before timing starts.

Prints ONE JSON line: tokens/s of the whole step, the local-softmax kernel
against the bf16 MFMA roofline (its duration taken from HIP events recorded
around that kernel on its own stream during the timed steps), the state pass
against the HBM roofline, the dense bidirectional softmax companion at the same
shape, the bidirectional hybrid form (§3.2 with overlap: later chunks join the
linear set) at the same shape, the same step with learned two-layer-MLP
feature maps (seeded synthetic weights), and the fp64 CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 100] [--warmup 200]

The default warm-up (200 steps, about a quarter of a second) brings the GPU
from idle to its sustained clock before the timed steps start; with only a
few warm-up steps the first timed steps run at a lower clock (about 7 % slower
at this shape).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# HBM bytes per dispatch of the local-softmax kernel at the default workload, from
# rocprofv3 FETCH_SIZE (x 2.0) + WRITE_SIZE (x 1.0), the factors a plain 1 GiB copy
# gives (profiles/local_bf16_wan_21x30x52.md).  Valid only for the kernel source
# it was measured on: reported as null once local_bf16.hip or its flags change.
LOCAL_KERNEL_TRAFFIC = {"source_sha256_16": "0f59890a5d110b3c", "workload": "wan_21x30x52",
                        "phi": "elu1", "chunk_frames": 3, "bytes": (277098.6 * 2.0 + 98288.8 * 1.0) * 1024}


LOCAL_KERNEL_SOURCES = ("local_bf16.hip", "local_common.h", "common.h")


def local_kernel_sha():
    """Hash of what the local kernel is compiled from: its sources and, from
    kernels.h (which also declares every other kernel's parameters), the
    LocalParams block and the helpers after it up to the block-state section."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_video_rehyat_amd", "csrc")
    for name in LOCAL_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(csrc, "kernels.h"), "rb") as f:
        text = f.read()
    start = text.index(b"struct LocalParams {")
    end = text.index(b"// Block-state pass:", start)
    h.update(text[start:end])
    from linear_attention_video_rehyat_amd.build import file_flags  # the kernel's compile flags
    h.update(repr(tuple(file_flags("local_bf16.hip"))).encode())
    return h.hexdigest()[:16]


def local_kernel_traffic(workload, phi, chunk_frames):
    """HBM bytes per launch measured by counters, only while the kernel source is unchanged."""
    sha = local_kernel_sha()
    t = LOCAL_KERNEL_TRAFFIC
    if (sha, workload, phi, chunk_frames) != (t["source_sha256_16"], t["workload"], t["phi"], t["chunk_frames"]):
        return None
    return t["bytes"]


class Hip:
    """Minimal HIP event API over ctypes (events on an arbitrary stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


def geometry_counts(w, Tc, To, phi_dim):
    """Algorithmic work of one forward (ReHyAt §3.3 partition).

    softmax FLOPs = 4 d sum_t |Q_t| |W_t| B H (QK^T and PV), exps = sum |Q_t||W_t| B H,
    state-pass bytes = K and V rows of every delta block read once (bf16) plus the
    fp32 block sums written once and read once by the scan."""
    F, HW, d = w.frames, w.tokens_per_frame, w.head_dim
    C = (F + Tc - 1) // Tc
    pairs = 0
    for t in range(C):
        f0, f1 = t * Tc, min((t + 1) * Tc, F)
        w0 = max(f0 - To, 0)
        pairs += (f1 - f0) * HW * (f1 - w0) * HW
    BH = w.B * w.H
    flops = 4.0 * d * pairs * BH
    lin_rows = max((C - 1) * Tc - To, 0) * HW if phi_dim > 0 else 0
    E = d * phi_dim + phi_dim
    state_bytes = 2.0 * BH * lin_rows * d * 2 + 3.0 * (C - 1) * BH * E * 4 if phi_dim > 0 else 0.0
    # bidirectional form (§3.2 with overlap): every key of the clip lies in a
    # block; 2C+1 block sums written and read, C prepared states written
    bidir_bytes = (2.0 * BH * F * HW * d * 2 + 2.0 * (2 * C + 1) * BH * E * 4 + C * BH * E * 4
                   if phi_dim > 0 and C >= 2 else 0.0)
    return {"softmax_flops": flops, "exps": float(pairs * BH), "state_bytes": state_bytes,
            "bidir_state_bytes": bidir_bytes, "chunks": C}


def time_steps(rh, hip, q, k, v, out, w, Tc, To, phi, steps, warmup, profile=True, causal=True, flush=None):
    """Times `steps` forwards.  With `flush` (a device buffer), each step is
    preceded by a write of the whole buffer, so that no input is left in the
    last-level cache (only the per-kernel event times are meaningful then)."""
    import torch
    for _ in range(warmup):
        rh.attn_fwd(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi, out=out, causal=causal)
    torch.cuda.synchronize()
    evs = [[hip.event() for _ in range(4)] for _ in range(steps)] if profile else None
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xff)
        if profile:
            rh.set_profile_events(evs[i])
        rh.attn_fwd(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi, out=out, causal=causal)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if profile:
        rh.set_profile_events(None)
    res = {"ms_per_step": (t1 - t0) * 1000.0 / steps}
    if profile:
        st = [hip.elapsed_ms(e[0], e[1]) for e in evs]
        sc = [hip.elapsed_ms(e[1], e[2]) for e in evs]
        lo = [hip.elapsed_ms(e[2], e[3]) for e in evs]
        res.update(state_ms=sum(st) / steps, scan_ms=sum(sc) / steps, local_ms=sum(lo) / steps)
        for e in evs:
            for x in e:
                hip.destroy(x)
    return res


def backward_bench(rh, inputs, q, k, v, w, Tc, To, phi, steps, cnt):
    """Training direction at the same shape: forward with lse, then the
    backward (dq, dk, dv) for a seeded output gradient, timed with torch events
    on the current stream.  The softmax-window part of the backward does 5
    GEMM-shaped products per (query, window key) pair where the forward does 2,
    plus the recomputation of QK^T in both the dk/dv and the dq kernels: its
    algorithmic work is counted as 2.5x the forward's softmax FLOPs (the usual
    convention for attention backward)."""
    import torch
    dy = inputs.make_dout(w).to(q.device)
    out, lse = rh.attn_fwd_lse(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi)
    grads = [torch.empty_like(q) for _ in range(3)]
    for _ in range(2):
        rh.attn_bwd(q, k, v, out, lse, dy, w.frames, w.tokens_per_frame, Tc, To, phi, grads=grads)
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(steps):
        rh.attn_fwd_lse(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi, out=out, lse=lse)
    e1.record()
    for _ in range(steps):
        rh.attn_bwd(q, k, v, out, lse, dy, w.frames, w.tokens_per_frame, Tc, To, phi, grads=grads)
    e2.record()
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / steps
    bwd_ms = e1.elapsed_time(e2) / steps
    flops = 2.5 * cnt["softmax_flops"]
    return {"fwd_lse_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "train_tokens_per_s": round(w.tokens / ((fwd_ms + bwd_ms) / 1000.0), 1),
            "bwd_tflops": round(flops / (bwd_ms / 1000.0) / 1e12, 2), "bwd_algorithmic_flops": flops,
            "bwd_frac": round(flops / (bwd_ms / 1000.0) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def workload_sweep(rh, hip, inputs, steps):
    """The other Wan-shaped workloads, one forward each: the CFG pair (B = 2)
    with T_c = 1, 3, 7 next to dense softmax at that shape (local-window versus
    linear-state cost), and the 21 x 45 x 80 clip with 1 % outlier keys."""
    import torch
    res = {}
    wc = inputs.WORKLOADS["wan_cfg_21x30x52"]
    q, k, v = (x.to("cuda") for x in inputs.make_qkv(wc))
    out = torch.empty_like(q)
    for Tc in (1, 3, 7):
        t = time_steps(rh, hip, q, k, v, out, wc, Tc, 1, "elu1", steps, 1)
        c = geometry_counts(wc, Tc, 1, wc.head_dim)
        res[f"cfg_B2_Tc{Tc}"] = {
            "ms_per_step": round(t["ms_per_step"], 4), "tokens_per_s": round(wc.tokens / (t["ms_per_step"] / 1000.0), 1),
            "local_ms": round(t["local_ms"], 4), "local_tflops": round(c["softmax_flops"] / (t["local_ms"] / 1000.0) / 1e12, 2),
            "state_pass_ms": round(t["state_ms"] + t["scan_ms"], 4),
            "state_pass_gbs": round(c["state_bytes"] / ((t["state_ms"] + t["scan_ms"]) / 1000.0) / 1e9, 1)}
    t = time_steps(rh, hip, q, k, v, out, wc, wc.frames, 0, "none", max(2, steps // 2), 1)
    c = geometry_counts(wc, wc.frames, 0, 0)
    res["cfg_B2_dense"] = {"ms_per_step": round(t["ms_per_step"], 4),
                           "tokens_per_s": round(wc.tokens / (t["ms_per_step"] / 1000.0), 1),
                           "tflops": round(c["softmax_flops"] / (t["local_ms"] / 1000.0) / 1e12, 2)}
    del q, k, v, out
    wo = inputs.WORKLOADS["wan_outlier_21x45x80"]
    q, k, v = (x.to("cuda") for x in inputs.make_qkv(wo))
    out = torch.empty_like(q)
    t = time_steps(rh, hip, q, k, v, out, wo, wo.chunk_frames, wo.overlap_frames, "elu1", steps, 1)
    c = geometry_counts(wo, wo.chunk_frames, wo.overlap_frames, wo.head_dim)
    res["outlier_21x45x80"] = {
        "ms_per_step": round(t["ms_per_step"], 4), "tokens_per_s": round(wo.tokens / (t["ms_per_step"] / 1000.0), 1),
        "local_ms": round(t["local_ms"], 4), "local_tflops": round(c["softmax_flops"] / (t["local_ms"] / 1000.0) / 1e12, 2),
        "state_pass_ms": round(t["state_ms"] + t["scan_ms"], 4)}
    return res


def length_scaling_bench(rh, hip, inputs, warmup):
    """Forward time against clip length: the first F = 21, 42, ..., 105 latent
    frames (1560 tokens each) of the 105-frame workload, T_c = 3, T_o = 1,
    elu+1; least-squares line, its R^2, and the 105 frames again as 35
    streaming steps of 3 frames (the chunk-wise RNN form; after a warm-up
    stream, the mean of 10 streams run back to back; and the same 35 steps
    captured in a HIP graph, replayed), with the device memory high-water of the
    streaming loop at 21 and at 105 frames."""
    import numpy as np
    import torch
    wl = inputs.WORKLOADS["wan_long_105x30x52"]
    HW = wl.tokens_per_frame
    q, k, v = (x.to("cuda") for x in inputs.make_qkv(wl))
    frames = [21, 42, 63, 84, 105]
    ms = []
    for F in frames:
        n = F * HW
        qs, ks, vs = (x[:, :, :n].contiguous() for x in (q, k, v))
        out = torch.empty_like(qs)
        wF = wl.with_(frames=F)
        # the 105-frame forward is the streaming comparison's reference: 10 steps
        t = time_steps(rh, hip, qs, ks, vs, out, wF, 3, 1, "elu1", 10 if F == frames[-1] else 5, warmup,
                       profile=False)
        ms.append(t["ms_per_step"])
        del qs, ks, vs, out
    x, y = np.array(frames, float), np.array(ms)
    a, b = np.polyfit(x, y, 1)
    r2 = 1.0 - float(((y - (a * x + b)) ** 2).sum() / ((y - y.mean()) ** 2).sum())

    def stream(F, reps=1):
        # `reps` whole streams back to back (a fresh state each), mean time per stream
        sts = [rh.StepState(1, wl.H, HW, wl.head_dim, 3, 1, "elu1") for _ in range(reps)]
        chunks = [tuple(x[:, :, 3 * i * HW:3 * (i + 1) * HW].contiguous() for x in (q, k, v))
                  for i in range(F // 3)]
        outs = [torch.empty_like(c[0]) for c in chunks]
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        t0 = time.perf_counter()
        for st in sts:
            for c, o in zip(chunks, outs):
                st.step(*c, out=o)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / reps
        return dt, torch.cuda.max_memory_allocated() - base, sts[0].nbytes

    stream(105)  # warm-up, as the forwards above are timed after theirs
    dt105, hw105, sb105 = stream(105, reps=10)
    _, hw21, sb21 = stream(21)

    def stream_graph(reps=5):
        # the 35 steps of a stream captured once in a HIP graph (from a fresh
        # state, whose buffer needs no initialisation) and replayed as whole streams
        chunks = [tuple(x[:, :, 3 * i * HW:3 * (i + 1) * HW].contiguous() for x in (q, k, v)) for i in range(35)]
        outs = [torch.empty_like(c[0]) for c in chunks]
        s = torch.cuda.Stream()
        warm = rh.StepState(1, wl.H, HW, wl.head_dim, 3, 1, "elu1")
        with torch.cuda.stream(s):
            for c, o in zip(chunks, outs):
                warm.step(*c, out=o, stream=s)
        st = rh.StepState(1, wl.H, HW, wl.head_dim, 3, 1, "elu1")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for c, o in zip(chunks, outs):
                st.step(*c, out=o, stream=s)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / reps
        del g
        rh.workspace_release(s)
        return dt

    dtg = stream_graph()
    return {"frames": frames, "ms_per_fwd": [round(m, 4) for m in ms],
            "slope_ms_per_21_frames": round(a * 21, 4), "intercept_ms": round(b, 4), "r2": round(r2, 5),
            "stream_105_frames": {"steps": 35, "ms": round(dt105 * 1000.0, 3),
                                  "vs_one_shot_105": round(dt105 * 1000.0 / ms[-1], 3),
                                  "graph_ms": round(dtg * 1000.0, 3),
                                  "graph_tokens_per_s": round(105 * HW / dtg, 1),
                                  "tokens_per_s": round(105 * HW / dt105, 1),
                                  "state_bytes": sb105, "state_bytes_at_21_frames": sb21,
                                  "extra_device_bytes_105": hw105, "extra_device_bytes_21": hw21}}


def learned_map_bench(rh, hip, inputs, q, k, v, out, w, Tc, To, hidden, steps, cnt):
    """The same step with the learned feature maps (seeded synthetic weights,
    two-layer MLP of `hidden` units per head and side, D' = 2d), and the
    feature-map kernel alone over every query row of the clip against the bf16
    MFMA roofline (2 (hidden d + 2d hidden) flops per row)."""
    import torch
    maps = []
    for side, scale in ((0, 1.0), (1, w.key_scale)):
        w1, b1, w2, b2 = inputs.make_mlp_weights(w.seed_id, side, w.H, w.head_dim, hidden, w.dtype, scale)
        maps.append(rh.MlpWeights(w1.to(torch.bfloat16).cuda(), b1.cuda(), w2.to(torch.bfloat16).cuda(),
                                  b2.cuda()))
    pair = tuple(maps)
    t = time_steps(rh, hip, q, k, v, out, w, Tc, To, pair, steps, 1)
    d = w.head_dim
    phi_out = torch.empty(w.B, w.H, w.N, 2 * d, dtype=q.dtype, device=q.device)
    for _ in range(2):
        rh.feature_mlp(q, pair[0], out=phi_out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        rh.feature_mlp(q, pair[0], out=phi_out)
    e1.record()
    torch.cuda.synchronize()
    mlp_ms = e0.elapsed_time(e1) / reps
    rows = w.B * w.H * w.N
    flops = 2.0 * rows * (hidden * d + 2 * d * hidden)
    tflops = flops / (mlp_ms / 1000.0) / 1e12
    return {"tokens_per_s": round(w.tokens / (t["ms_per_step"] / 1000.0), 1),
            "ms_per_step": round(t["ms_per_step"], 4), "hidden": hidden, "feature_dim": 2 * d,
            "map_and_state_ms": round(t["state_ms"], 4), "scan_ms": round(t["scan_ms"], 4),
            "local_ms": round(t["local_ms"], 4),
            "local_tflops": round(cnt["softmax_flops"] / (t["local_ms"] / 1000.0) / 1e12, 2),
            "feature_kernel": {"kernel": "phi_mlp_bf16_kernel", "rows": rows, "ms": round(mlp_ms, 4),
                               "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                               "algorithmic_flops": flops,
                               "hbm_gbs": round(rows * d * 2 * 3 / (mlp_ms / 1000.0) / 1e9, 1)}}


def block_bench(rh, inputs, w, Tc, To, phi, steps, attn_ms, dense_attn_ms):
    """The attention blocks around the hybrid attention at the Wan2.1-1.3B
    shape (C = 12 x 128 = 1536, seeded synthetic projection weights): one block
    with the hybrid attention and one with full softmax attention (the block
    before conversion), and stacks of 30 blocks with 25, 20, 15 and 0 of them
    converted (the pages' configurations; the first n converted).  The
    projections' share of a block is its time minus the attention's; their
    algorithmic work is 8 T C^2 FLOP per block (QKV 6 T C^2, output 2 T C^2)."""
    import torch
    H, d = w.H, w.head_dim
    C = H * d
    T = w.B * w.N
    x = inputs.make_block_input(w.seed_id, w.B, w.N, C, device="cuda")
    wts = [rh.BlockWeights(*(t.cuda() for t in inputs.make_block_weights(w.seed_id, l, C))) for l in range(30)]
    out = torch.empty_like(x)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    hyb_ms = timed(lambda: rh.block_fwd(x, wts[0], w.frames, w.tokens_per_frame, H, True, Tc, To, phi, out=out),
                   steps)
    den_ms = timed(lambda: rh.block_fwd(x, wts[0], w.frames, w.tokens_per_frame, H, False, Tc, To, phi, out=out),
                   max(2, steps // 4))
    proj_flops = 8.0 * T * C * C
    proj_ms = hyb_ms - attn_ms
    res = {"C": C, "block_hybrid_ms": round(hyb_ms, 4), "block_dense_ms": round(den_ms, 4),
           "projections_ms": round(proj_ms, 4), "projection_flops": proj_flops,
           "projections_tflops": round(proj_flops / (proj_ms / 1000.0) / 1e12, 1),
           "projections_frac": round(proj_flops / (proj_ms / 1000.0) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "dense_block_projections_ms": round(den_ms - dense_attn_ms, 4) if dense_attn_ms else None}
    stacks = {}
    for n_conv in (25, 20, 15, 0):
        flags = inputs.converted_blocks(n_conv, 30)
        ms = timed(lambda: rh.stack_fwd(x, wts, flags, w.frames, w.tokens_per_frame, H, Tc, To, phi, out=out), 2)
        stacks[f"converted_{n_conv}_of_30"] = {"ms": round(ms, 3), "tokens_per_s": round(T / (ms / 1000.0), 1)}
    res["stack_30_blocks"] = stacks
    res["stack_speedup_25_of_30"] = round(stacks["converted_0_of_30"]["ms"] / stacks["converted_25_of_30"]["ms"], 3)
    return res


def cpu_info():
    """Host CPU model and logical CPU counts (the machine and what this process may use)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "logical_cpus": os.cpu_count()}


def cpu_baseline(w, q, k, v, Tc, To, phi, target_s=15.0, full_limit_s=60.0):
    """fp64 oracle (definition form) on the host cores: every output row when a
    512-row calibration puts the full output within full_limit_s, else a
    random row sample sized to about target_s."""
    import numpy as np
    from oracle import oracle as O
    q64, k64, v64 = (x.double().numpy() for x in (q, k, v))
    N = w.N
    rng = np.random.default_rng(12345)

    def rows_for(n):
        return np.sort(rng.choice(N, size=n, replace=False)).astype(np.int64)

    n = 512
    t0 = time.perf_counter()
    O.definition(q64, k64, v64, w.frames, w.tokens_per_frame, Tc, To, phi, rows=rows_for(n))
    dt = time.perf_counter() - t0
    full = dt * N / n <= full_limit_s
    n2 = N if full else int(max(32, min(N, n * target_s / max(dt, 1e-3))))
    rows = None if full else rows_for(n2)
    t0 = time.perf_counter()
    O.definition(q64, k64, v64, w.frames, w.tokens_per_frame, Tc, To, phi, rows=rows)
    dt = time.perf_counter() - t0
    tokens = w.B * n2
    what = (f"every output row ({N} per (b,h)), all {w.B * w.H} heads" if full else
            f"{n2} random query rows of {N} per (b,h), all {w.B * w.H} heads")
    res = {"value": tokens / dt, "unit": "tokens/s", "cores": O.max_threads(), "kind": "oracle",
           "sample": f"{what}, fp64 definition form, {dt:.1f} s", "seconds": round(dt, 2),
           "full_output": full}
    res.update(cpu_info())
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="wan_21x30x52")
    ap.add_argument("--phi", default="elu1")
    ap.add_argument("--chunk-frames", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-bidir", action="store_true")
    ap.add_argument("--no-learned", action="store_true")
    ap.add_argument("--no-length", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-blocks", action="store_true")
    ap.add_argument("--no-combine", action="store_true")
    ap.add_argument("--learned-hidden", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        dst.copy_(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": 1 << 30}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: runs on one GPU only (the hot path is single-GPU; sharding it over "
              "several GPUs is not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_video_rehyat_amd as rh
    from linear_attention_video_rehyat_amd import inputs

    def progress(part):
        # one line per finished part on stderr (stdout carries only the JSON line)
        print(f"bench.py: {part} done", file=sys.stderr, flush=True)

    w = inputs.WORKLOADS[args.workload]
    Tc = args.chunk_frames or w.chunk_frames
    To = w.overlap_frames
    phi = args.phi
    phi_dim = {"none": 0, "elu1": w.head_dim, "poly2": 2 * w.head_dim}[phi]
    hip = Hip()

    q, k, v = inputs.make_qkv(w)
    qg, kg, vg = (x.to("cuda") for x in (q, k, v))
    out = torch.empty_like(qg)
    torch.cuda.synchronize()

    main_t = time_steps(rh, hip, qg, kg, vg, out, w, Tc, To, phi, args.steps, args.warmup)
    progress("main timing")
    cnt = geometry_counts(w, Tc, To, phi_dim)
    value = w.tokens / (main_t["ms_per_step"] / 1000.0)
    local_tflops = cnt["softmax_flops"] / (main_t["local_ms"] / 1000.0) / 1e12
    roofline = {"bound": "mfma", "achieved": round(local_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(local_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": local_kernel_traffic(w.name, phi, Tc), "kernel": "local_bf16_kernel",
                "ms": round(main_t["local_ms"], 4),
                "algorithmic_flops": cnt["softmax_flops"]}
    state = None
    if phi_dim > 0:
        # The HBM fraction is taken with the last-level cache flushed before
        # every step (512 MB written), so that K and V come from HBM; in the
        # back-to-back steps of the main timing part of them is still in the
        # cache (the warm_* figures, cache-assisted).
        st_ms = main_t["state_ms"] + main_t["scan_ms"]
        warm_gbs = cnt["state_bytes"] / (st_ms / 1000.0) / 1e9
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ft = time_steps(rh, hip, qg, kg, vg, out, w, Tc, To, phi, max(5, args.steps // 2), 1, flush=scratch)
        del scratch
        fms = ft["state_ms"] + ft["scan_ms"]
        gbs = cnt["state_bytes"] / (fms / 1000.0) / 1e9
        state = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(gbs / PEAK_HBM_GBS, 4), "cache": "flushed before every step",
                 "state_kernel_ms": round(ft["state_ms"], 4), "scan_ms": round(ft["scan_ms"], 4),
                 "algorithmic_bytes": cnt["state_bytes"],
                 "warm_state_kernel_ms": round(main_t["state_ms"], 4), "warm_scan_ms": round(main_t["scan_ms"], 4),
                 "warm_achieved": round(warm_gbs, 1), "warm_frac": round(warm_gbs / PEAK_HBM_GBS, 4)}
        progress("state pass (flushed)")

    combine = None
    if not args.no_combine and phi_dim > 0:
        # The linear query branch and the joint normalisation run fused in the
        # local kernel's epilogue; their cost is the local kernel's time with
        # the feature map on, less its time with it off (phi = NONE: the same
        # windows and tiles, softmax-only epilogue).  Linear FLOPs per query of
        # a chunk with a linear set: a^L = phi(q)^T S_t (2 D' d) and
        # n^L = phi(q).z_t (2 D').
        # The difference of two ~1 ms timings: the two variants alternate over
        # several rounds and the median of the per-round differences is kept.
        rounds, per = 7, max(3, args.steps // 10)
        n_ms, h_ms, diffs = [], [], []
        for _ in range(rounds):
            n_t = time_steps(rh, hip, qg, kg, vg, out, w, Tc, To, "none", per, 2)
            h_t = time_steps(rh, hip, qg, kg, vg, out, w, Tc, To, phi, per, 2)
            n_ms.append(n_t["local_ms"])
            h_ms.append(h_t["local_ms"])
            diffs.append(h_t["local_ms"] - n_t["local_ms"])
        lin_q = sum(max(min((t + 1) * Tc, w.frames) - t * Tc, 0) for t in range(1, cnt["chunks"])
                    if t * Tc - To > 0) * w.tokens_per_frame * w.B * w.H
        marginal = statistics.median(diffs)
        hyb = statistics.median(h_ms)
        combine = {"local_ms_softmax_only": round(statistics.median(n_ms), 4),
                   "local_ms_with_linear_branch": round(hyb, 4),
                   "marginal_ms": round(marginal, 4),
                   "marginal_ms_range": [round(min(diffs), 4), round(max(diffs), 4)],
                   "marginal_share_of_local": round(marginal / hyb, 4),
                   "linear_queries": lin_q,
                   "linear_gflop": round(lin_q * (2.0 * phi_dim * w.head_dim + 2.0 * phi_dim) / 1e9, 2),
                   "out_bytes": w.B * w.H * w.frames * w.tokens_per_frame * w.head_dim * 2}
        progress("fused combine")

    dense = None
    if not args.no_dense:
        d_t = time_steps(rh, hip, qg, kg, vg, out, w, w.frames, 0, "none", max(3, args.steps // 4), 1)
        dc = geometry_counts(w, w.frames, 0, 0)
        dense = {"tokens_per_s": round(w.tokens / (d_t["ms_per_step"] / 1000.0), 1),
                 "ms_per_step": round(d_t["ms_per_step"], 4),
                 "tflops": round(dc["softmax_flops"] / (d_t["local_ms"] / 1000.0) / 1e12, 2),
                 "hybrid_speedup": round(d_t["ms_per_step"] / main_t["ms_per_step"], 3),
                 "flop_ratio": round(dc["softmax_flops"] / cnt["softmax_flops"], 3)}
        progress("dense softmax")

    bidir = None
    if not args.no_bidir:
        b_t = time_steps(rh, hip, qg, kg, vg, out, w, Tc, To, phi, max(3, args.steps // 2), 1, causal=False)
        bidir = {"tokens_per_s": round(w.tokens / (b_t["ms_per_step"] / 1000.0), 1),
                 "ms_per_step": round(b_t["ms_per_step"], 4),
                 "local_ms": round(b_t["local_ms"], 4),
                 "local_tflops": round(cnt["softmax_flops"] / (b_t["local_ms"] / 1000.0) / 1e12, 2)}
        if phi_dim > 0:
            bst = b_t["state_ms"] + b_t["scan_ms"]
            bidir.update(state_kernel_ms=round(b_t["state_ms"], 4), scan_ms=round(b_t["scan_ms"], 4),
                         state_pass_gbs=round(cnt["bidir_state_bytes"] / (bst / 1000.0) / 1e9, 1),
                         state_pass_frac=round(cnt["bidir_state_bytes"] / (bst / 1000.0) / 1e9
                                               / PEAK_HBM_GBS, 4),
                         state_algorithmic_bytes=cnt["bidir_state_bytes"])
        progress("bidirectional")

    learned = None
    if not args.no_learned:
        learned = learned_map_bench(rh, hip, inputs, qg, kg, vg, out, w, Tc, To, args.learned_hidden,
                                    max(3, args.steps // 2), cnt)
        progress("learned maps")

    backward = None
    if not args.no_backward and phi in ("elu1", "poly2", "none"):
        backward = backward_bench(rh, inputs, qg, kg, vg, w, Tc, To, phi, max(3, args.steps // 2), cnt)
        progress("backward")

    sweep = None
    if not args.no_sweep and w.name == "wan_21x30x52" and phi == "elu1":
        sweep = workload_sweep(rh, hip, inputs, max(3, args.steps // 4))
        progress("other workloads")

    length = None
    if not args.no_length and w.name == "wan_21x30x52" and Tc == 3 and phi == "elu1":
        length = length_scaling_bench(rh, hip, inputs, min(args.warmup, 5))
        progress("length scaling")

    blocks = None
    if not args.no_blocks and w.name == "wan_21x30x52" and phi in ("elu1", "poly2"):
        dense_attn = None
        if dense is not None:
            dense_attn = dense["ms_per_step"]
        blocks = block_bench(rh, inputs, w, Tc, To, phi, max(3, args.steps // 4), main_t["ms_per_step"], dense_attn)
        progress("attention blocks")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, Tc, To, phi, args.cpu_seconds)
        progress("cpu baseline")

    line = {
        "metric": "hybrid-attn fwd tokens/s at Wan2.1-1.3B shape; % of MFMA/HBM roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(main_t["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/v, N(0,1)/sqrt(128) k)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "head_dim": w.head_dim,
                   "frames": w.frames, "tokens_per_frame": w.tokens_per_frame,
                   "chunk_frames": Tc, "overlap_frames": To, "feature_map": phi,
                   "tokens_per_step": w.tokens},
        "roofline": roofline,
        "state_pass": state,
        "combine": combine,
        "dense_softmax": dense,
        "bidirectional": bidir,
        "learned_map": learned,
        "backward": backward,
        "length_scaling": length,
        "other_workloads": sweep,
        "attention_blocks": blocks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
