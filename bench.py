#!/usr/bin/env python3
"""Benchmark of the W4A16 NVFP4 GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--only NAME] [--no-extra] [--no-cpu]

A step is one call of the hot path on one batch: the decode-shaped dense
linear Y[16, 14336] = g * X[16, 4096] . dequant(W)^T, the workload the HBM
target is quoted on.  Inputs are resident in HBM before the timed region.
The weight is rotated over 16 distinct copies (528 MB, more than twice the
256 MB Infinity Cache), so each step streams its weight from HBM.

Timing: W untimed eager warmup calls, then the K timed calls are captured in
one HIP graph (uploaded by one untimed replay), and the timed replay is
bracketed by torch.cuda.synchronize() on both sides.  HIP events recorded
inside the graph around every call give the per-launch kernel durations used
for the roofline fraction; the events around the whole replay give
ms_per_step.

Prints ONE JSON line (rank 0, one GPU): metric/value for the step, plus
"roofline" (dominant kernel vs HBM peak 8 TB/s), "cpu_baseline" (the CPU
oracle timed on a bounded sample of the same workload on the host cores) and
"extra" (the other workloads, each timed the same way: throughput in GB/s and
TFLOP/s with their roofline fractions).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HEADLINE = "decode_M16_N14336_K4096"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--only", default=None, help="time one workload only (for profiling runs)")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of 512 MiB per step (calibrates HBM byte counters)")
    p.add_argument("--list", action="store_true")
    return p.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "weight_only_fp4_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


# ------------------------------------------------------------- workloads ---

class Workload:
    def __init__(self, name, kind, kernel, alg_bytes, flops, launch, copies, meta, bound):
        self.name, self.kind, self.kernel = name, kind, kernel
        self.alg_bytes, self.flops, self.launch, self.copies = alg_bytes, flops, launch, copies
        self.meta, self.bound = meta, bound


def dense_bytes(M, N, K, pre, mxfp4=False):
    """Algorithmic bytes of one dense call: the weight codes (N K / 2) and scales (one byte per 16 K, MXFP4 one
    per 32), the activation, the output, the pre-scale and the global scale (NVFP4)."""
    if mxfp4:
        return 0.53125 * N * K + 2.0 * M * K + 2.0 * M * N + (2.0 * K if pre else 0.0)
    return 0.5625 * N * K + 2.0 * M * K + 2.0 * M * N + (2.0 * K if pre else 0.0) + 4.0


def make_dense(name, M, N, K, *, seed, scales="pow2_mant", g_stored=1.0 / 2688.0, divisor=False, prescale=False,
               copies=1, host_case=None, f16=False, mxfp4=False):
    import torch
    import synth
    import weight_only_fp4_amd as nv
    dev = "cuda:0"
    if host_case is not None:
        c = host_case
        x = torch.from_numpy(c.x.view("int16")).view(torch.bfloat16).to(dev)
        w = torch.from_numpy(c.w).to(dev)
        s = torch.from_numpy(c.s).to(dev)
        pre = None if c.pre is None else torch.from_numpy(c.pre.view("int16")).view(torch.bfloat16).to(dev)
        g_stored, divisor = c.g_stored, c.g_is_divisor
    else:
        x = synth.device_normal_bf16((M, K), seed, dev)
        w = synth.device_codes((N, K // 2), seed + 1, dev)
        s = (synth.device_scales((N, K // 32), seed + 2, "e8m0", dev) if mxfp4
             else synth.device_scales((N, K // 16), seed + 2, scales, dev))
        pre = synth.device_prescale(K, seed + 3, dev) if prescale else None
        if f16:   # the fp16 form: the same draws, rounded to fp16
            x = x.to(torch.float16)
            pre = None if pre is None else pre.to(torch.float16)
    g = torch.tensor([g_stored], dtype=torch.float32, device=dev)
    blob = nv.repack_mxfp4(w, s) if mxfp4 else nv.repack(w, s)
    del w, s
    blobs = [blob] + [blob.clone() for _ in range(copies - 1)]
    y = torch.empty((M, N), dtype=x.dtype, device=dev)
    ws = nv.workspace(nv.gemm_workspace_bytes(M, N, K), dev)

    def launch(i):
        if mxfp4:
            nv.gemm_mxfp4(x, blobs[i % copies], N, K, pre, out=y, workspace_buf=ws)
        else:
            nv.gemm(x, blobs[i % copies], N, K, g, divisor, pre, out=y, workspace_buf=ws)

    # the kernel the automatic dispatch runs, as the library reports it
    kernel = nv.VARIANT_KERNELS[nv.gemm_plan(M, N, K)]
    flops = 2.0 * M * N * K
    ab = dense_bytes(M, N, K, pre is not None, mxfp4)
    bound = "hbm" if flops / ab < (BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9) else "mfma"
    meta = {"M": M, "N": N, "K": K, "prescale": pre is not None, "divisor": bool(divisor), "weight_copies": copies,
            "activation": "f16" if f16 else "bf16", "weights": "mxfp4" if mxfp4 else "nvfp4"}
    wl = Workload(name, "dense", kernel, ab, flops, launch, copies, meta, bound)
    wl.tensors = dict(x=x, y=y, g=g, blobs=blobs)
    return wl


def make_grouped(name, T, fc, *, seed=1004, E=128, topk=8):
    import numpy as np
    import torch
    import synth
    import weight_only_fp4_amd as nv
    dev = "cuda:0"
    K, N = (2048, 2 * 768) if fc == "fc1" else (768, 2048)
    route = synth.zipf_routing(synth.rng(synth.routing_seed(seed)), T, E, topk)
    counts = np.bincount(route.reshape(-1), minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    active = int(np.count_nonzero(counts))
    # rotate weight copies until the active experts' weights of all copies
    # exceed twice the 256 MB Infinity Cache, so every call streams from HBM
    copies = max(1, -(-(512 << 20) // int(active * 0.5625 * N * K)))
    sd = seed * 10 + (1 if fc == "fc1" else 2)
    x = synth.device_normal_bf16((R, K), sd, dev)
    w = synth.device_codes((E, N, K // 2), sd + 1, dev)
    s = synth.device_scales((E, N, K // 16), sd + 2, "pow2_mant", dev)
    v = synth.rng(sd + 3).integers(-2, 3, size=E)
    gs = torch.tensor((np.exp2(v.astype(np.float64)) / 2688.0).astype(np.float32), device=dev)
    off = torch.from_numpy(offsets).to(dev)
    blob = nv.repack(w, s)
    del w, s
    blobs = [blob] + [blob.clone() for _ in range(copies - 1)]
    y = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
    ws = nv.workspace(nv.lib().nvfp4_w4a16_grouped_gemm_workspace_bytes(R, E, N, K), dev)

    def launch(i):
        nv.grouped_gemm(x, off, blobs[i % copies], E, N, K, gs, False, None, out=y, workspace_buf=ws)

    ab = active * 0.5625 * N * K + 2.0 * R * K + 2.0 * R * N + 4.0 * E + 4.0 * (E + 1)
    flops = 2.0 * R * N * K
    kernel = "k_gemm_small_m" if R <= 16 * E else "k_gemm_tile"
    bound = "hbm" if flops / ab < (BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9) else "mfma"
    meta = {"E": E, "topk": topk, "T": T, "R": R, "N": N, "K": K, "active_experts": active, "weight_copies": copies}
    wl = Workload(name, "grouped", kernel, ab, flops, launch, copies, meta, bound)
    wl.tensors = dict(x=x, y=y, blobs=blobs)
    return wl


def make_moe_layer(name, T, *, seed=1004, E=128, topk=8, hidden=2048, inter=768, fused=True, mxfp4=False):
    """A whole MoE layer on the device: routing, FC1 with the token gather fused (N = 2 inter) and, when fused,
    the gated SiLU in its epilogue (else a separate SiLU step), FC2 (K = inter), top-k combine.  Weight copies
    rotate as for the grouped workloads.  mxfp4: both projections in MXFP4 (fused form only)."""
    assert fused or not mxfp4
    import numpy as np
    import torch
    import synth
    import weight_only_fp4_amd as nv
    dev = "cuda:0"
    route = synth.zipf_routing(synth.rng(synth.routing_seed(seed)), T, E, topk)
    counts = np.bincount(route.reshape(-1), minlength=E)
    R, active = T * topk, int(np.count_nonzero(counts))
    w_bytes = active * (0.53125 if mxfp4 else 0.5625) * (2 * inter * hidden + hidden * inter)
    copies = max(1, -(-(512 << 20) // int(w_bytes)))
    sd = seed * 10 + 5
    ids = torch.from_numpy(route.astype(np.int32)).to(dev)
    x = synth.device_normal_bf16((T, hidden), sd, dev)
    wts = torch.from_numpy(synth.rng(sd + 1).random((T, topk)).astype(np.float32)).to(dev)
    if mxfp4:
        b1 = nv.repack_gated(synth.device_codes((E, 2 * inter, hidden // 2), sd + 2, dev),
                             synth.device_scales((E, 2 * inter, hidden // 32), sd + 3, "e8m0", dev), mxfp4=True)
        b2 = nv.repack_mxfp4(synth.device_codes((E, hidden, inter // 2), sd + 4, dev),
                             synth.device_scales((E, hidden, inter // 32), sd + 5, "e8m0", dev))
    else:
        repack1 = nv.repack_gated if fused else nv.repack
        b1 = repack1(synth.device_codes((E, 2 * inter, hidden // 2), sd + 2, dev),
                     synth.device_scales((E, 2 * inter, hidden // 16), sd + 3, "pow2_mant", dev))
        b2 = nv.repack(synth.device_codes((E, hidden, inter // 2), sd + 4, dev),
                       synth.device_scales((E, hidden, inter // 16), sd + 5, "pow2_mant", dev))
    blobs = [(b1, b2)] + [(b1.clone(), b2.clone()) for _ in range(copies - 1)]
    v = synth.rng(sd + 6).integers(-2, 3, size=(2, E))
    g1 = torch.tensor((np.exp2(v[0].astype(np.float64)) / 2688.0).astype(np.float32), device=dev)
    g2 = torch.tensor((np.exp2(v[1].astype(np.float64)) / 2688.0).astype(np.float32), device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(R, dtype=torch.int32, device=dev)
    token_row = torch.empty(R, dtype=torch.int32, device=dev)
    h = None if fused else torch.empty((R, 2 * inter), dtype=torch.bfloat16, device=dev)
    a = torch.empty((R, inter), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((R, hidden), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, hidden), dtype=torch.bfloat16, device=dev)
    L = nv.lib()
    ws1 = nv.workspace(L.nvfp4_w4a16_grouped_gemm_gather_workspace_bytes(T, R, E, 2 * inter, hidden), dev)
    ws2 = nv.workspace(L.nvfp4_w4a16_grouped_gemm_workspace_bytes(R, E, hidden, inter), dev)
    wsr = nv.workspace(L.nvfp4_moe_route_workspace_bytes(T, topk, E), dev)
    st = lambda: nv._stream(x.device)

    def launch(i):
        w1, w2 = blobs[i % copies]
        nv._check(L.nvfp4_moe_route(nv._ptr(ids), T, topk, E, nv._ptr(off), nv._ptr(row_token), nv._ptr(token_row),
                                    nv._ptr(wsr), wsr.numel(), st()))
        if mxfp4:
            nv.moe_fc1(x, row_token, off, w1, E, inter, hidden, None, nv.MOE_SILU_GLU, out=a, mxfp4=True)
            nv.grouped_gemm_mxfp4(a, off, w2, E, hidden, inter, out=y2)
        else:
            if fused:
                nv.moe_fc1(x, row_token, off, w1, E, inter, hidden, g1, nv.MOE_SILU_GLU, out=a)
            else:
                nv.grouped_gemm_gather(x, row_token, off, w1, E, 2 * inter, hidden, g1, out=h, workspace_buf=ws1)
                nv.moe_silu_mul(h, out=a)
            nv.grouped_gemm(a, off, w2, E, hidden, inter, g2, out=y2, workspace_buf=ws2)
        nv.moe_combine(y2, token_row, wts, out=out)

    # algorithmic bytes of the layer: active weights, the tokens in and out, routing ids and weights
    ab = w_bytes + 2.0 * T * hidden * 2 + 8.0 * T * topk
    flops = 2.0 * R * hidden * (2 * inter) + 2.0 * R * inter * hidden
    bound = "hbm" if flops / ab < (BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9) else "mfma"
    meta = {"E": E, "topk": topk, "T": T, "R": R, "hidden": hidden, "inter": inter, "active_experts": active,
            "weight_copies": copies, "weights": "mxfp4" if mxfp4 else "nvfp4",
            "steps_per_call": "route, FC1 (gather) with the gated SiLU in its epilogue, FC2, "
                              "combine" if fused else "route, FC1 (gather), SiLU, FC2, combine"}
    wl = Workload(name, "moe_layer", "moe_layer", ab, flops, launch, copies, meta, bound)
    wl.tensors = dict(x=x, out=out, blobs=blobs)
    return wl


def make_stream_read(name, nbytes, copies, workgroups, unroll):
    """A plain read of nbytes per step (no GEMM): the ceiling a streaming kernel reaches on this device at the
    size of a decode weight (33 MB) and of an LM-head weight (302 MB).  The buffer rotates over `copies`
    copies, more than twice the 256 MB Infinity Cache, as the GEMM weights do."""
    import torch
    import weight_only_fp4_amd as nv
    dev = "cuda:0"
    nbytes = (nbytes + 15) // 16 * 16
    bufs = [torch.full((nbytes,), 1, dtype=torch.uint8, device=dev) for _ in range(copies)]
    out = torch.zeros(workgroups, dtype=torch.int32, device=dev)

    def launch(i):
        nv.stream_read(bufs[i % copies], out, workgroups, unroll)

    meta = {"bytes": nbytes, "workgroups": workgroups, "unroll": unroll, "copies": copies,
            "note": "plain read, no GEMM: the streaming ceiling at this size"}
    wl = Workload(name, "stream", "k_stream_read", float(nbytes), 0.0, launch, copies, meta, "hbm")
    wl.tensors = dict(bufs=bufs, out=out)
    return wl


def workload_specs():
    """name -> builder (the headline first)."""
    return {
        HEADLINE: lambda: make_dense(HEADLINE, 16, 14336, 4096, seed=1001, g_stored=1 / (448 * 6), copies=16),
        "decode_M1_N14336_K4096": lambda: make_dense("decode_M1_N14336_K4096", 1, 14336, 4096, seed=1001,
                                                     g_stored=1 / (448 * 6), copies=16),
        "decode_M8_N14336_K4096": lambda: make_dense("decode_M8_N14336_K4096", 8, 14336, 4096, seed=1001,
                                                     g_stored=1 / (448 * 6), copies=16),
        "decode_M1_N4096_K14336": lambda: make_dense("decode_M1_N4096_K14336", 1, 4096, 14336, seed=1001,
                                                     g_stored=1 / (448 * 6), copies=16),
        "decode_M16_N4096_K14336": lambda: make_dense("decode_M16_N4096_K14336", 16, 4096, 14336, seed=1001,
                                                      g_stored=1 / (448 * 6), copies=16),
        "prefill_M4096_N14336_K4096": lambda: make_dense("prefill_M4096_N14336_K4096", 4096, 14336, 4096, seed=1002,
                                                         scales="log_uniform", copies=1),
        "prefill_M8192_N17408_K5120": lambda: make_dense("prefill_M8192_N17408_K5120", 8192, 17408, 5120, seed=1002,
                                                         scales="log_uniform", copies=1),
        "lmhead_M1_N131072_K4096": lambda: make_dense("lmhead_M1_N131072_K4096", 1, 131072, 4096, seed=1003,
                                                      g_stored=2688.0, divisor=True, prescale=True, copies=2),
        "lmhead_M64_N131072_K4096": lambda: make_dense("lmhead_M64_N131072_K4096", 64, 131072, 4096, seed=1003,
                                                       g_stored=2688.0, divisor=True, prescale=True, copies=2),
        "ragged_M33_N1000_K1040": lambda: make_dense("ragged_M33_N1000_K1040", 33, 1000, 1040, seed=1003,
                                                     g_stored=2688.0, divisor=True, prescale=True, copies=1),
        "tiny_M4_N256_K512": lambda: make_dense("tiny_M4_N256_K512", 4, 256, 512, seed=1000, g_stored=1 / 448,
                                                copies=1),
        "decode_f16_M16_N14336_K4096": lambda: make_dense("decode_f16_M16_N14336_K4096", 16, 14336, 4096,
                                                          seed=1001, g_stored=1 / (448 * 6), copies=16, f16=True),
        "prefill_f16_M4096_N14336_K4096": lambda: make_dense("prefill_f16_M4096_N14336_K4096", 4096, 14336, 4096,
                                                             seed=1002, scales="log_uniform", copies=1, f16=True),
        # MXFP4 weights (E8M0 scale per 32 K, no global scale) on the same kernels
        "decode_mxfp4_M16_N14336_K4096": lambda: make_dense("decode_mxfp4_M16_N14336_K4096", 16, 14336, 4096,
                                                            seed=1001, copies=16, mxfp4=True),
        "prefill_mxfp4_M4096_N14336_K4096": lambda: make_dense("prefill_mxfp4_M4096_N14336_K4096", 4096, 14336,
                                                               4096, seed=1002, copies=1, mxfp4=True),
        "moe_fc1_T16": lambda: make_grouped("moe_fc1_T16", 16, "fc1"),
        "moe_fc2_T16": lambda: make_grouped("moe_fc2_T16", 16, "fc2"),
        "moe_fc1_T2048": lambda: make_grouped("moe_fc1_T2048", 2048, "fc1"),
        "moe_fc2_T2048": lambda: make_grouped("moe_fc2_T2048", 2048, "fc2"),
        "moe_layer_T16": lambda: make_moe_layer("moe_layer_T16", 16),
        "moe_layer_T2048": lambda: make_moe_layer("moe_layer_T2048", 2048),
        "moe_layer_mxfp4_T2048": lambda: make_moe_layer("moe_layer_mxfp4_T2048", 2048, mxfp4=True),
        "moe_layer_unfused_T16": lambda: make_moe_layer("moe_layer_unfused_T16", 16, fused=False),
        "moe_layer_unfused_T2048": lambda: make_moe_layer("moe_layer_unfused_T2048", 2048, fused=False),
        # the decode weight's size (33,619,972 B) and the LM-head weight's (302,268,420 B); launch shapes from
        # a sweep of workgroups x loads in flight per lane
        "stream_read_33MB": lambda: make_stream_read("stream_read_33MB", 33619972, 16, 8192, 2),
        "stream_read_302MB": lambda: make_stream_read("stream_read_302MB", 302268420, 2, 8192, 8),
    }


# ---------------------------------------------------------------- timing ---

def time_workload(wl, steps, warmup):
    """Return dict: ms_per_step (events around the timed replay), per-launch kernel ms (events inside the graph)."""
    import torch
    for i in range(warmup):
        wl.launch(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        wl.launch(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(with_events):
        graph = torch.cuda.CUDAGraph()
        evs = [(torch.cuda.Event(enable_timing=True, external=True), torch.cuda.Event(enable_timing=True, external=True))
               for _ in range(steps)] if with_events else None
        with torch.cuda.graph(graph):
            for i in range(steps):
                if evs:
                    evs[i][0].record()
                wl.launch(warmup + i)
                if evs:
                    evs[i][1].record()
        return graph, evs

    try:
        graph, evs = capture(True)
    except Exception as exc:   # event nodes in graphs unsupported: fall back to whole-replay timing
        print(f"[bench] per-launch events in graph unavailable ({type(exc).__name__}: {exc}); using replay mean",
              file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        graph, evs = capture(False)
    graph.replay()                       # uploads the graph; untimed
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    graph.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    per = [a.elapsed_time(b) for a, b in evs] if evs else None
    del graph
    return {"ms_per_step": total_ms / steps, "wall_ms_per_step": 1e3 * wall / steps,
            "kernel_ms": (sum(per) / len(per)) if per else total_ms / steps,
            "kernel_ms_min": min(per) if per else None, "kernel_ms_source": "events_in_graph" if per else "replay_mean"}


def summarize(wl, t):
    ms = t["ms_per_step"]
    steps = {"steps": t["steps"]} if "steps" in t else {}
    kms = t["kernel_ms"]
    gbs = wl.alg_bytes / (ms * 1e-3) / 1e9
    tfl = wl.flops / (ms * 1e-3) / 1e12
    kgbs = wl.alg_bytes / (kms * 1e-3) / 1e9
    ktfl = wl.flops / (kms * 1e-3) / 1e12
    return {"us_per_step": round(ms * 1e3, 3), "us_per_launch_kernel": round(kms * 1e3, 3),
            "GBps": round(gbs, 1), "TFLOPs": round(tfl, 2),
            "hbm_frac": round(kgbs / HBM_PEAK_GBS, 4), "mfma_frac": round(ktfl / BF16_PEAK_TFLOPS, 4),
            "bound": wl.bound, "alg_bytes": wl.alg_bytes, "flops": wl.flops, **steps, **wl.meta}


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    for r in rec.get("records", []):
        if r.get("workload") == workload and r.get("kernel") == kernel and r.get("source_sha256") == source_digest():
            return r.get("hbm_bytes_per_launch")
    return None


# ----------------------------------------------------------- cpu baseline ---

def cpu_baseline(case, target_s=12.0):
    """The CPU oracle, as is, on the headline workload, repeated for about target_s seconds; weight GB/s.

    A bounded sample: whole oracle calls on the full headline shape (M x N x K) are repeated until about
    target_s seconds of host work have run (the first call sizes the repeat count)."""
    import oracle
    thr = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.gemm(case.x, case.w, case.s, case.g_stored, case.g_is_divisor, case.pre)
    first = time.perf_counter() - t0
    reps = max(1, int(round(target_s / max(first, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.gemm(case.x, case.w, case.s, case.g_stored, case.g_is_divisor, case.pre)
    dt = time.perf_counter() - t0
    wbytes = 0.5625 * case.N * case.K * reps
    # one thread on the tiny configuration (M=4, N=256, K=512), as a reference point
    import synth
    tiny = synth.tiny_case()
    t0 = time.perf_counter()
    for _ in range(10):
        oracle.gemm(tiny.x, tiny.w, tiny.s, tiny.g_stored, tiny.g_is_divisor, tiny.pre, threads=1)
    tiny_ms = (time.perf_counter() - t0) * 100.0
    return {"value": round(wbytes / dt / 1e9, 4), "unit": "GB/s", "cores": thr, "kind": "oracle",
            "sample": f"{reps} whole calls of M={case.M}, N={case.N}, K={case.K} ({dt:.1f} s, fp64, {thr} threads)",
            "cpu_model": cpu_model(), "tiny_M4_N256_K512_one_thread_ms": round(tiny_ms, 3)}


def cpu_per_config():
    """The oracle, as is, once per configuration on host arrays drawn by the same generators as the GPU
    workloads: whole calls where the oracle finishes in seconds (tiny, the decode shapes, the LM head, the ragged
    shape, MoE T=16), a seeded subset of rows where it does not (prefill, MoE T=2048; labelled "subset").  Each
    entry gives the rate in the workload's own unit (algorithmic GB/s for the HBM-bound shapes, GFLOP/s for the
    MFMA-bound ones) over the rows the oracle computed."""
    import numpy as np
    import oracle
    import synth
    thr = oracle.max_threads()
    res = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def dense(name, c, rows, unit, subset_of=None):
        x = c.x[:rows]
        dt = timed(lambda: oracle.gemm(x, c.w, c.s, c.g_stored, c.g_is_divisor, c.pre))
        if unit == "GB/s":
            v = dense_bytes(rows, c.N, c.K, c.pre is not None) / dt / 1e9
        else:
            v = 2.0 * rows * c.N * c.K / dt / 1e9
        res[name] = {"value": round(v, 4), "unit": unit, "seconds": round(dt, 3), "threads": thr,
                     "sample": (f"subset: {rows} seeded rows of M={subset_of}" if subset_of else "whole call")
                     + f", N={c.N}, K={c.K}"}

    tiny = synth.tiny_case()
    dense("tiny_M4_N256_K512", tiny, 4, "GB/s")
    for N, K in ((14336, 4096), (4096, 14336)):
        c = synth.decode_case(16, N, K)
        for M in ((1, 8, 16) if N == 14336 else (1, 16)):
            dense(f"decode_M{M}_N{N}_K{K}", c, M, "GB/s")
    lm = synth.dense_case(64, 131072, 4096, 1003, g_stored=2688.0, g_is_divisor=True, prescale=True)
    for M in (1, 64):
        dense(f"lmhead_M{M}_N131072_K4096", lm, M, "GB/s")
    del lm
    dense("ragged_M33_N1000_K1040",
          synth.dense_case(33, 1000, 1040, 1003, g_stored=2688.0, g_is_divisor=True, prescale=True), 33, "GB/s")
    for M, N, K in ((4096, 14336, 4096), (8192, 17408, 5120)):
        # the first 64 rows of a seeded draw stand for a seeded subset: rows are independent draws
        c = synth.dense_case(64, N, K, 1002, scales="log_uniform", g_stored=1.0 / 2688.0)
        dense(f"prefill_M{M}_N{N}_K{K}", c, 64, "GFLOP/s", subset_of=M)
        del c
    for T in (16, 2048):
        for fc, (N, K) in (("fc1", (1536, 2048)), ("fc2", (2048, 768))):
            c = synth.grouped_case(T, 128, 8, N, K, 1004, x_source="gather" if fc == "fc1" else "fresh")
            counts = np.diff(c.offsets)
            if T == 16:
                x, off, label = c.x, c.offsets, f"whole call: R={c.R} rows over {int((counts > 0).sum())} experts"
            else:
                # one seeded row of every active expert
                g = synth.rng(7)
                act = np.nonzero(counts)[0]
                pick = np.array([c.offsets[e] + g.integers(0, counts[e]) for e in act])
                x = c.x[pick]
                off = np.zeros(c.E + 1, dtype=np.int32)
                off[1:] = np.cumsum(counts > 0)
                label = f"subset: one seeded row of each of the {len(act)} active experts (of R={c.R})"
            dt = timed(lambda: oracle.grouped_gemm(x, off, c.w, c.s, c.g_stored, False, None))
            rows, nact = x.shape[0], int((np.diff(off) > 0).sum())
            if T == 16:
                v, unit = (nact * 0.5625 * N * K + 2.0 * rows * (K + N) + 8.0 * c.E + 4.0) / dt / 1e9, "GB/s"
            else:
                v, unit = 2.0 * rows * N * K / dt / 1e9, "GFLOP/s"
            res[f"moe_{fc}_T{T}"] = {"value": round(v, 4), "unit": unit, "seconds": round(dt, 3), "threads": thr,
                                     "sample": label + f", N={N}, K={K}"}
            del c
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def max_sclk_mhz():
    """Peak engine clock of device 0 from the HIP runtime (hipDeviceAttributeClockRate, kHz), or None."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        kHIP_ATTR_CLOCK_RATE = 5   # position of hipDeviceAttributeClockRate in hipDeviceAttribute_t
        if hip.hipDeviceGetAttribute(ctypes.byref(v), kHIP_ATTR_CLOCK_RATE, 0) == 0 and v.value > 0:
            return v.value / 1000.0
    except OSError:
        pass
    return None


def stream_copy_gbps(torch, nbytes=512 << 20, reps=10):
    """Device-to-device copy rate (bytes read + written per second), as context for the HBM numbers."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del a, b
    torch.cuda.empty_cache()
    return round(2 * nbytes / ms / 1e6, 1)


def sanity_parity(case, y):
    """Sampled outputs of the benchmarked call against the oracle (not timed)."""
    import numpy as np
    import oracle
    import synth
    g = synth.rng(5)
    rows, cols = g.integers(0, case.M, 512), g.integers(0, case.N, 512)
    ref = oracle.gemm_sampled(case.x, case.w, case.s, case.g_stored, case.g_is_divisor, case.pre, rows, cols)
    got = y.float().cpu().numpy().astype(np.float64)[rows, cols]
    ok, info = oracle.accept(got, ref)
    return {"ok": bool(ok), "rel_fro": info.get("rel_fro"), "samples": len(rows)}


# ------------------------------------------------------------------ main ---

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU: --gpus must be 1 (sharding the GEMM across "
                                   "GPUs is not implemented)", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.list:
        print("\n".join(workload_specs()))
        return
    import torch
    import weight_only_fp4_amd as nv
    nv.lib()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "cus": props.multi_processor_count, "arch": getattr(props, "gcnArchName", "")}
    sclk = max_sclk_mhz()
    if sclk:
        # dense bf16 MFMA: 4096 flop per compute unit per clock (2.5 PFLOP/s at 256 CUs and 2.4 GHz)
        device["max_sclk_mhz"] = sclk
        device["bf16_peak_at_max_sclk_tflops"] = round(props.multi_processor_count * sclk * 1e6 * 4096 / 1e12, 1)

    if args.copy_calibration:
        nbytes = 512 << 20
        a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        b = torch.empty_like(a)
        for _ in range(args.warmup):
            b.copy_(a)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            b.copy_(a)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": ms,
                          "GBps": 2 * nbytes / ms / 1e6, "steps": args.steps}), flush=True)
        return

    specs = workload_specs()
    head_name = args.only or HEADLINE
    if head_name not in specs:
        raise SystemExit(f"unknown workload {head_name}; --list shows them")

    host_case = None
    if head_name == HEADLINE:
        import synth
        host_case = synth.decode_case(16)
        wl = make_dense(HEADLINE, 16, 14336, 4096, seed=1001, copies=16, host_case=host_case)
    else:
        wl = specs[head_name]()
    print(f"[bench] timing {wl.name} ({args.steps} steps, {args.warmup} warmup)", file=sys.stderr, flush=True)
    t = time_workload(wl, args.steps, args.warmup)
    s = summarize(wl, t)
    parity = sanity_parity(host_case, wl.tensors["y"]) if host_case is not None else None

    kms = t["kernel_ms"]
    if wl.bound == "hbm":
        ach = wl.alg_bytes / (kms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = wl.flops / (kms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    roof.update({"traffic": traffic_for(wl.kernel, wl.name), "kernel": wl.kernel,
                 "alg_units_per_launch": wl.alg_bytes if wl.bound == "hbm" else wl.flops,
                 "kernel_us": round(kms * 1e3, 3), "timing": t["kernel_ms_source"]})

    value = s["GBps"] if wl.bound == "hbm" else s["TFLOPs"]
    unit = "GB/s" if wl.bound == "hbm" else "TFLOP/s"
    metric = (f"W4A16 NVFP4 GEMM weight-stream throughput ({wl.name})" if wl.bound == "hbm"
              else f"W4A16 NVFP4 GEMM throughput ({wl.name})")
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(t["ms_per_step"], 6), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl.name, **wl.meta, "parallelism": "single-gpu"},
           "roofline": roof, "device": device, "source_sha256": source_digest()[:16]}
    if parity is not None:
        out["parity"] = parity
    del wl
    torch.cuda.empty_cache()

    if not args.only and not args.no_extra:
        extra = {}
        for name, build in specs.items():
            if name == HEADLINE:
                continue
            print(f"[bench] timing {name}", file=sys.stderr, flush=True)
            w2 = build()
            # enough steps for about 20 ms of timed work (20 .. 200): a short
            # replay of an MFMA-bound call reads up to 8 % slow (measured)
            probe = time_workload(w2, 3, min(args.warmup, 5))
            n2 = int(min(200, max(20, 20.0 / max(probe["ms_per_step"], 1e-3))))
            t2 = time_workload(w2, n2, min(args.warmup, 5))
            t2["steps"] = n2
            extra[name] = summarize(w2, t2)
            if "bf16_peak_at_max_sclk_tflops" in device:
                extra[name]["mfma_frac_at_max_sclk"] = round(extra[name]["TFLOPs"] / device["bf16_peak_at_max_sclk_tflops"], 4)
            del w2
            torch.cuda.empty_cache()
        out["extra"] = extra
        out["context"] = {"stream_copy_GBps": stream_copy_gbps(torch),
                          "note": "512 MiB device copy, bytes read + written per second"}

    if not args.only and not args.no_cpu:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(host_case)
        if not args.no_extra:
            print("[bench] timing the CPU oracle per configuration", file=sys.stderr, flush=True)
            out["cpu_baseline"]["per_config"] = cpu_per_config()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
