#!/usr/bin/env python3
"""Benchmark of the K2 MoE layer forward on one MI355X.

One step = one call of the whole layer (router GEMM, top-K, permutation, grouped gate/up and down
SwiGLU GEMMs, combine) on a batch of synthetic tokens whose inputs and weights are already resident
in HBM.  The printed line's value is the decode workload (T=64, the 384-expert K2 layer); the
prefill workload (T=8192) is measured in the same run and reported beside it.  Per-kernel times
come from HIP events recorded around every kernel launch inside the timed steps.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill|skew|ep_share|tiny]

Profiling helpers (rocprofv3 runs the bench; this file turns its CSV output into the summaries kept
under profiles/):

    rocprofv3 --kernel-trace --stats -d DIR -o run --output-format csv -- python bench.py ...
    python bench.py --profile-summary DIR            # markdown table of the kernel statistics
    rocprofv3 --pmc FETCH_SIZE -d FDIR -o run --output-format csv -- python bench.py --pmc-calibrate ...
    rocprofv3 --pmc WRITE_SIZE -d WDIR -o run --output-format csv -- python bench.py --pmc-calibrate ...
    python bench.py --traffic-summary WORKLOAD FDIR WDIR   # HBM bytes per dispatch, copy-calibrated
    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 \
              SQ_INSTS_VALU_MFMA_MOPS_F16 -d DIR -o run --output-format csv -- python bench.py ...
    python bench.py --mfma-summary WORKLOAD DIR            # matrix-core busy % per dispatch
    python bench.py --lds-summary WORKLOAD DIR             # LDS busy % per dispatch
"""
import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "K2 MoE layer tokens/s at T=64 decode & T=8192 prefill; % HBM / % MFMA peak"
HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15         # dense bf16 MFMA FLOP/s
F32_PEAK = 157.3e12        # fp32 vector FLOP/s

# Library kernel names (as the library reports them) -> a substring of the kernel symbol rocprofv3
# prints, and the source files that make the kernel (its measured traffic is only reported while
# their digest is unchanged).
KERNEL_SYMBOLS = {
    "gateup_stream": ("::stream_kernel<true", ["gemm_stream.hip", "tile_core.h", "kernels.h"]),
    "down_stream": ("::stream_kernel<false", ["gemm_stream.hip", "tile_core.h", "kernels.h"]),
    "gateup_skinny": ("::skinny_kernel<true", ["gemm_skinny.hip", "tile_core.h", "kernels.h"]),
    "down_skinny": ("::skinny_kernel<false", ["gemm_skinny.hip", "tile_core.h", "kernels.h"]),
    "gateup_tile": ("::gateup_tile_kernel", ["gemm_tile.hip", "tile_gemm.h", "tile_core.h", "kernels.h"]),
    "down_tile": ("::down_tile_kernel", ["gemm_tile.hip", "tile_gemm.h", "tile_core.h", "kernels.h"]),
    "router_logits": ("::router_logits_kernel", ["route.hip", "tile_core.h", "kernels.h"]),
    "combine": ("::combine_kernel", ["combine.hip", "kernels.h"]),
    "router_logits_f32": ("::router_logits_f32_kernel", ["route.hip", "tile_core.h", "kernels.h"]),
    "gateup_f32": ("::gateup_f32_kernel", ["gemm_simple.hip", "kernels.h"]),
    "down_f32": ("::down_f32_kernel", ["gemm_simple.hip", "kernels.h"]),
    "gateup_q4": ("::q_stream_kernel<(moe::QFormat)0, true", ["gemm_quant.hip", "tile_core.h", "kernels.h"]),
    "down_q4": ("::q_stream_kernel<(moe::QFormat)0, false", ["gemm_quant.hip", "tile_core.h", "kernels.h"]),
    "gateup_fp8": ("::q_stream_kernel<(moe::QFormat)1, true", ["gemm_quant.hip", "tile_core.h", "kernels.h"]),
    "down_fp8": ("::q_stream_kernel<(moe::QFormat)1, false", ["gemm_quant.hip", "tile_core.h", "kernels.h"]),
    "gateup_tile_fp8": ("::gateup_tile_fp8_kernel", ["gemm_tile.hip", "tile_gemm.h", "tile_core.h", "kernels.h"]),
    "down_tile_fp8": ("::down_tile_fp8_kernel", ["gemm_tile.hip", "tile_gemm.h", "tile_core.h", "kernels.h"]),
    "gateup_tile_q4": ("::gateup_tile_q4_kernel", ["gemm_tile_q4.hip", "tile_gemm.h", "tile_core.h", "kernels.h"]),
    "down_tile_q4": ("::down_tile_q4_kernel", ["gemm_tile_q4.hip", "tile_gemm.h", "tile_core.h", "kernels.h"]),
}
QUANT_STREAM = ("gateup_q4", "down_q4", "gateup_fp8", "down_fp8")  # the quantized weight-stream kernels
Q4_BYTES = 0.5 + 2 / 32    # bytes per 4-bit weight: the code plus its share of a binary16 scale per 32
FP8_BYTES = 1 + 4 / 128 ** 2  # bytes per FP8 weight: the code plus its share of an fp32 scale per 128 x 128
QUANT_BYTES = {"int4": Q4_BYTES, "fp8": FP8_BYTES}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
CALIB_BYTES = 1 << 30      # the calibration copy reads and writes this many bytes
CALIB_SYMBOL = "neg_kernel"


def sources_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SYMBOLS[kernel][1]:
        with open(os.path.join(ROOT, "moe_layer_forward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """Counter-measured HBM bytes per launch of `kernel` on `workload`, from the committed PMC
    summary, or None when there is none or the kernel's sources changed since it was taken."""
    if kernel not in KERNEL_SYMBOLS or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        text = fh.read()
    for block in re.findall(r"```json\n(.*?)\n```", text, re.S):
        for rec in json.loads(block):
            if rec["workload"] == workload and rec["kernel"] == kernel:
                return rec["traffic_bytes"] if rec["sources"] == sources_digest(kernel) else None
    return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """Raw HIP events (the runtime torch has loaded), recorded by the library around each kernel."""

    def __init__(self, n):
        import torch  # noqa: F401

        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev[i] = h
        self.n = n

    def slice(self, start, count):
        return ctypes.cast(ctypes.byref(self.ev, start * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p)), count

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.ev[i])


def measure_peaks():
    """Measured peaks of this GPU (the published ones are HBM_PEAK and BF16_PEAK): a streaming read
    of 4 GiB, a 2 GiB copy (read + write bytes) and a loop of independent bf16 MFMAs, each the best
    of 5 timed launches on torch's current stream."""
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "moe_layer_forward_amd", "libmoe_peaks.so"))
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
    lib.peaks_read.argtypes = [vp, i64, i32, vp]
    lib.peaks_read_vgpr.argtypes = [vp, i64, vp, vp]
    lib.peaks_copy.argtypes = [vp, vp, i64, vp]
    lib.peaks_mfma.argtypes = [i32, i32, vp, vp]
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")

    def best(launch):
        times = []
        for r in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = launch()
            b.record()
            if rc:
                raise RuntimeError(f"peaks launch failed ({rc})")
            torch.cuda.synchronize()
            if r:
                times.append(a.elapsed_time(b) * 1e-3)
        return min(times)

    rd = 4 << 30
    buf = torch.empty(rd, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    t_read = best(lambda: lib.peaks_read(buf.data_ptr(), rd, 512, stream))
    t_read_v = best(lambda: lib.peaks_read_vgpr(buf.data_ptr(), rd, sink.data_ptr(), stream))
    half = rd // 2
    t_copy = best(lambda: lib.peaks_copy(buf.data_ptr(), buf.data_ptr() + half, half, stream))
    del buf
    torch.cuda.empty_cache()
    blocks, iters = 256 * 4, 2000
    t_mfma = best(lambda: lib.peaks_mfma(blocks, iters, sink.data_ptr(), stream))
    flops = blocks * 4 * 4 * iters * 32768
    return {"hbm_read_GB_s": max(rd / t_read, rd / t_read_v) / 1e9, "hbm_read_lds_GB_s": rd / t_read / 1e9,
            "hbm_read_vgpr_GB_s": rd / t_read_v / 1e9, "hbm_copy_GB_s": 2 * half / t_copy / 1e9,
            "mfma_bf16_TFLOP_s": flops / t_mfma / 1e12,
            "how": "streaming read of 4 GiB (the better of direct-to-LDS non-temporal 1 KiB loads, 8 waves per "
                   "CU, and 16-byte register loads); 2 GiB copy counted as read + write; 4 independent "
                   "v_mfma_f32_32x32x16_bf16 chains per wave, 16 waves per CU; best of 5"}


def vendor_gemm(E=385, M=192, H=7168, I=2048, reps=10):
    """Context for the prefill GEMMs: the vendor library (torch.bmm, i.e. hipBLASLt) on the same
    shapes as dense batched products -- every expert with exactly M rows, no row gather, no SwiGLU
    epilogue, weights already laid out K x N.  Returns ms and TFLOP/s per product."""
    import torch

    out = {}
    for name, K, N in (("gate_up", H, 2 * I), ("down", I, H)):
        a = torch.randn(E, M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(E, K, N, device="cuda", dtype=torch.bfloat16)  # contiguous right operand
        for _ in range(3):
            c = torch.bmm(a, b)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            c = torch.bmm(a, b)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        out[name] = {"E": E, "M": M, "K": K, "N": N, "ms": ms, "TFLOP_s": 2.0 * E * M * K * N / ms / 1e9,
                     "weight_GB_s": E * K * N * 2 / ms / 1e6}
        del a, b, c
        torch.cuda.empty_cache()
    return out


STREAM_ROWS, STREAM_MIN_GROUPS = 32, 16   # the device plan's split (kStreamRows, kStreamMinGroups)
SKINNY_ROWS = 64   # calls of at most this many rows in all (and more than the stream kernels take) run skinny


def plan_families(w, ids):
    """Which groups the library's plan hands to the weight-stream kernels and which to the tile
    kernels, from the realised routing (host mirror of moe_api.cpp's kernel choice and the device
    plan's split at kStreamRows).  Returns {family: [(group, rows,
    tokens)]}, tokens being the set of token ids whose rows the group reads (None = every token: the
    shared expert's or the dense FFN's group)."""
    if w.routing == "dense":
        groups = [(0, w.T, None)]
    else:
        ids = np.asarray(ids)
        groups = []
        for e in range(w.E):
            t_idx = np.nonzero((ids == e).any(axis=1))[0]
            rows = int((ids == e).sum())
            if rows:
                groups.append((e, rows, t_idx))
        if w.n_shared:
            groups.append((w.E, w.T, None))
    n_groups = (1 if w.routing == "dense" else w.E + w.n_shared)
    max_rows = w.T if w.routing == "dense" else w.T * w.K + w.T * w.n_shared
    if max_rows <= 4 * n_groups:
        return {"stream": groups, "tile": [], "skinny": []}
    if w.quant == "none" and w.dtype == "bf16" and max_rows <= SKINNY_ROWS and w.H % 64 == 0 and w.I % 64 == 0:
        return {"stream": [], "tile": [], "skinny": groups}
    cut = STREAM_ROWS if n_groups >= STREAM_MIN_GROUPS else 0
    return {"stream": [g for g in groups if g[1] <= cut], "tile": [g for g in groups if g[1] > cut], "skinny": []}


def kernel_work(name, w, fams, n_touched):
    """Algorithmic (bytes, flops) of one launch of a grouped-GEMM kernel: the weights of the groups the
    plan gives that kernel, once each (routed experts in their storage format: FP8 or 4-bit codes and
    scales; the shared expert and unquantized experts in bf16); the token rows those groups read (each
    token's row once; with quantized experts the routed groups read the binary16 rows, the shared
    expert the bf16 ones), or their h rows; the outputs written once.  Weight re-reads (per row pass
    of the stream kernels, per row tile of the tile kernels) are traffic, not algorithmic bytes."""
    eb = 2 if w.dtype == "bf16" else 4
    if fams is None:
        return None, None
    fam = ("tile" if "_tile" in name else "skinny" if "_skinny" in name
           else "stream" if (name.endswith("_stream") or name in QUANT_STREAM) else None)
    if fam is None:
        return None, None
    groups = fams[fam]
    if not groups:
        return None, None
    qb = QUANT_BYTES.get(w.quant)
    rows = sum(g[1] for g in groups)
    every = any(g[2] is None for g in groups)  # the shared expert's (or the dense FFN's) group
    routed = [g[2] for g in groups if g[2] is not None]
    tok_routed = len(np.unique(np.concatenate(routed))) if routed else 0
    w_elems = sum(eb if (qb is None or g[2] is None) else qb for g in groups)  # bytes per weight element
    if qb is None:
        a_bytes = (w.T if every else tok_routed) * w.H * eb
    else:
        a_bytes = tok_routed * w.H * 2 + (w.T * w.H * 2 if every else 0)
    if name.startswith("gateup"):
        return w_elems * 2 * w.I * w.H + a_bytes + rows * w.I * eb, rows * 2 * 2 * w.I * w.H
    if name.startswith("down"):
        return w_elems * w.H * w.I + rows * w.I * eb + rows * w.H * eb, rows * 2 * w.H * w.I
    return None, None


def roofline_of(name, w, kb, kf, us):
    """Roofline of one kernel launch: bound by HBM when its algorithmic flops per byte sit below the
    ridge of the published peaks, else by the matrix cores."""
    peak_flops = BF16_PEAK if w.dtype == "bf16" else F32_PEAK
    s = us * 1e-6
    if kf / kb < peak_flops / HBM_PEAK:
        r = {"bound": "hbm", "achieved": kb / s / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
             "frac": kb / s / HBM_PEAK}
    else:
        r = {"bound": "mfma", "achieved": kf / s / 1e12, "peak": peak_flops / 1e12, "unit": "TFLOP/s",
             "frac": kf / s / peak_flops}
    r.update({"traffic": load_traffic(w.name, name), "kernel": name, "bytes_per_launch": kb,
              "flops_per_launch": kf, "avg_launch_us": us})
    if r["frac"] > 1.0:
        log(f"warning: {w.name} {name}: roofline fraction {r['frac']:.3f} > 1 -- the algorithmic count is wrong")
    return r


def layer_work(w, n_touched):
    """Algorithmic bytes and flops of the whole layer: every touched expert's and the shared expert's
    weights once, the router weight, x read and y written once."""
    eb = 2 if w.dtype == "bf16" else 4
    routed_eb = QUANT_BYTES.get(w.quant, eb)
    bytes_ = (n_touched * routed_eb + w.n_shared * eb) * 3 * w.H * w.I + 2 * w.T * w.H * eb
    flops = (w.T * w.K + w.T * w.n_shared) * 2 * 3 * w.H * w.I
    if w.routing not in ("preassigned", "dense"):
        bytes_ += w.E * w.H * eb
        flops += 2 * w.T * w.E * w.H
    return bytes_, flops


def run(w, weights, steps, warmup, graph=True):
    import numpy as np
    import torch

    import moe_layer_forward_amd as moe
    from moe_layer_forward_amd import workloads as wl

    acts = wl.device_activations(w)
    cfg = moe.config_for(w)
    T = w.T
    y = torch.empty((T, w.H), dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32, device="cuda")
    if w.routing == "dense":
        # the dense first-layer FFN: one group of all T rows on the grouped-SwiGLU kernels
        ws = moe.alloc_workspace(cfg, moe.MOE_OP_GROUPED_SWIGLU, T, 1)
        offs = torch.tensor([0, T], dtype=torch.int32, device="cuda")

        def step():
            moe.moe_grouped_swiglu(cfg, offs, T, acts["x"], weights["w_gate"], weights["w_up"], weights["w_down"],
                                   y_dtype=moe.MOE_BF16, workspace=ws, out=y)
    elif w.routing == "preassigned":
        ws = moe.alloc_workspace(cfg, moe.MOE_OP_FORWARD_ROUTED, T)
        wg, wu, wd = (weights[k][:w.E] for k in ("w_gate", "w_up", "w_down"))

        def step():
            moe.moe_forward_routed(cfg, acts["x"], acts["topk_ids"], acts["topk_weights"], wg, wu, wd,
                                   weights["ws_gate"], weights["ws_up"], weights["ws_down"], workspace=ws, out=y)
    elif w.quant in ("int4", "fp8"):
        q4 = w.quant == "int4"
        ws = moe.alloc_workspace(cfg, moe.MOE_OP_FORWARD_Q4 if q4 else moe.MOE_OP_FORWARD_FP8, T)
        qw = {k: weights[k] for k in moe.QUANT_KEYS}
        fwd = moe.moe_forward_q4 if q4 else moe.moe_forward_fp8

        def step():
            fwd(cfg, acts["x"], weights["w_router"], qw, weights["ws_gate"], weights["ws_up"], weights["ws_down"],
                logit_offset=acts.get("logit_offset"), workspace=ws, out=y)
    else:
        ws = moe.alloc_workspace(cfg, moe.MOE_OP_FORWARD, T)

        def step():
            moe.moe_forward(cfg, acts["x"], weights["w_router"], weights["w_gate"], weights["w_up"],
                            weights["w_down"], weights["ws_gate"], weights["ws_up"], weights["ws_down"],
                            logit_offset=acts.get("logit_offset"), workspace=ws, out=y)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # kernels per step (the library reports what it launched)
    probe = HipEvents(64)
    moe.moe_profile_events(*probe.slice(0, 64))
    step()
    torch.cuda.synchronize()
    names = [moe.moe_profile_kernel(i) for i in range(moe.moe_profile_count())]
    moe.moe_profile_events(None, 0)
    probe.close()
    per = 2 * len(names)
    ev = HipEvents(per * steps)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_profile_events(*ev.slice(i * per, per))
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    moe.moe_profile_events(None, 0)

    kern = {n: 0.0 for n in names}
    for i in range(steps):
        for j, n in enumerate(names):
            kern[n] += ev.elapsed_ms(i * per + 2 * j, i * per + 2 * j + 1) / steps
    # GPU time of each step: the first kernel's start to the last kernel's end
    step_ms = sorted(ev.elapsed_ms(i * per, i * per + per - 1) for i in range(steps))
    ev.close()
    ms = (t1 - t0) * 1e3 / steps

    # the same step captured once as a HIP graph and replayed (a serving loop's launch mode): the
    # library launches only kernels on the caller's stream, so the call is capturable as it is
    graph_ms = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / steps
        del g

    flushed_ms = None
    if w.routing == "preassigned":
        # this workload's 0.35 GB of weights could stay in the 256 MB last-level cache between calls:
        # time it again with 1 GiB written between the calls
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(steps):
            flush.fill_(0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        flushed_ms = sorted(times)[len(times) // 2]
        del flush

    # routing actually realised (counts touched experts for the byte accounting)
    ids_np = None
    if w.routing == "dense":
        counts = np.array([T])
    else:
        if w.routing == "preassigned":
            ids = acts["topk_ids"]
        else:
            ids, _ = moe.moe_route(cfg, acts["x"], weights["w_router"], logit_offset=acts.get("logit_offset"))
        ids_np = ids.cpu().numpy()
        counts = np.bincount(ids_np.ravel(), minlength=w.E)
    n_touched = int((counts > 0).sum())
    lb, lf = layer_work(w, n_touched)
    fams = plan_families(w, None if w.routing == "dense" else ids_np)
    per_kernel = {}
    for n, us in kern.items():
        kb, kf = kernel_work(n, w, fams, n_touched)
        if kb:
            per_kernel[n] = roofline_of(n, w, kb, kf, us * 1e3)
    dom = max(kern, key=kern.get)
    roof = per_kernel.get(dom)
    peak_flops = BF16_PEAK if w.dtype == "bf16" else F32_PEAK
    s = ms * 1e-3
    layer = {"GB_s": lb / s / 1e9, "TFLOP_s": lf / s / 1e12, "hbm_frac": lb / s / HBM_PEAK,
             "mfma_frac": lf / s / peak_flops, "alg_bytes": lb, "alg_flops": lf, "touched_experts": n_touched,
             "rows_per_expert_max": int(counts.max()), "rows_per_expert_mean": float(counts.sum() / max(n_touched, 1)),
             "experts_le2_rows": int((counts <= 2).sum()),
             "step_gpu_ms": {"median": step_ms[len(step_ms) // 2], "min": step_ms[0], "max": step_ms[-1]}}
    if graph_ms is not None:
        layer["graph_ms_per_step"] = graph_ms
        layer["graph_tokens_per_s"] = T / (graph_ms * 1e-3)
    if flushed_ms is not None:
        layer["flushed_ms_median"] = flushed_ms
        layer["flushed_mfma_frac"] = lf / (flushed_ms * 1e-3) / peak_flops
    if fams is not None:
        layer["groups_on_stream_kernels"] = len(fams["stream"])
        layer["groups_on_tile_kernels"] = len(fams["tile"])
        layer["groups_on_skinny_kernels"] = len(fams["skinny"])
    return {"tokens_per_s": T / s, "ms_per_step": ms, "roofline": roof, "layer": layer,
            "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
            "kernels_roofline": {k: {f: v[f] for f in ("bound", "achieved", "unit", "frac", "bytes_per_launch",
                                                       "flops_per_launch")}
                                 for k, v in per_kernel.items()}}


def _time_oracle(w, n_tokens):
    """Seconds of the oracle's own arithmetic on the first n_tokens tokens of the workload, and the
    seconds spent regenerating expert weights beside it (not counted)."""
    import numpy as np

    import oracle
    from moe_layer_forward_amd import workloads as wl

    tokens = np.arange(n_tokens)
    x = wl.host_x_rows(w, tokens)
    router = wl.host_router(w)
    gen = [0.0]

    def expert(e):
        g0 = time.perf_counter()
        r = wl.host_expert(w, e)
        gen[0] += time.perf_counter() - g0
        return r

    shared = wl.host_shared(w)
    t0 = time.perf_counter()
    oracle.moe_forward(x, router, expert, shared, w.K, w.rsf, logit_offset=wl.logit_offsets(w))
    return time.perf_counter() - t0 - gen[0], gen[0]


def cpu_baseline(w, n_tokens, n_tokens_1t=4):
    """The oracle as it stands, on the first n_tokens tokens of the workload, on the host cores (and
    on the first n_tokens_1t tokens with one BLAS thread).  Only the oracle's own arithmetic is timed
    (weight regeneration excluded)."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits, threads = None, 1
    el, gen = _time_oracle(w, n_tokens)
    out = {"value": n_tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"first {n_tokens} tokens of the {w.name} workload (T={w.T}), all {w.K}+{w.n_shared} experts "
                     f"each, float64 numpy; {el:.2f} s of oracle arithmetic timed, plus {gen:.1f} s of "
                     f"input (expert weight) regeneration not timed"}
    if threadpool_limits is not None and n_tokens_1t > 0:
        with threadpool_limits(limits=1, user_api="blas"):
            el1, _ = _time_oracle(w, n_tokens_1t)
        out["one_thread"] = {"value": n_tokens_1t / el1, "unit": "tokens/s", "cores": 1,
                             "sample": f"first {n_tokens_1t} tokens, one BLAS thread; {el1:.2f} s timed"}
    return out


def cpu_baseline_sampled(w, n_experts=8, n_shared_rows=512, seed=7):
    """The oracle on a bounded sample of a large workload, extrapolated to the whole batch and labelled
    "sampled": the routing of every token (oracle.route), the SwiGLU of n_experts routed experts
    (drawn at random among the touched ones) over all of their rows, scaled to all routed rows by row
    count, and the shared expert on n_shared_rows rows, scaled to T rows (oracle.swiglu_expert).
    Only the oracle's arithmetic is timed (input regeneration is not); the combine is not timed."""
    import oracle
    from moe_layer_forward_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    rng = np.random.default_rng(seed)
    x = wl.host_x(w)
    t_route = 0.0
    if w.routing == "preassigned":
        ids = wl.preassigned(w)[0]
    else:
        t0 = time.perf_counter()
        ids = oracle.route(x, wl.host_router(w), w.K, w.rsf, logit_offset=wl.logit_offsets(w))[0]
        t_route = time.perf_counter() - t0
    counts = np.bincount(ids.ravel(), minlength=w.E)
    touched = np.nonzero(counts)[0]
    pick = np.sort(rng.choice(touched, min(n_experts, len(touched)), replace=False))
    t_exp, rows_exp = 0.0, 0
    for e in pick:
        t_idx = np.nonzero((ids == e).any(axis=1))[0]
        if w.routing == "preassigned" and len(t_idx) > n_shared_rows:
            t_idx = t_idx[:n_shared_rows]
        wts = wl.host_expert(w, int(e))
        t0 = time.perf_counter()
        oracle.swiglu_expert(x[t_idx], *wts)
        t_exp += time.perf_counter() - t0
        rows_exp += len(t_idx)
    t_routed = t_exp / rows_exp * ids.size
    t_shared = 0.0
    if w.n_shared:
        sh = wl.host_shared(w)
        m = min(n_shared_rows, w.T)
        t0 = time.perf_counter()
        oracle.swiglu_expert(x[:m], *sh)
        t_shared = (time.perf_counter() - t0) * w.T / m
    total = t_route + t_routed + t_shared
    return {"value": w.T / total, "unit": "tokens/s", "cores": threads, "kind": "oracle", "sampled": True,
            "sample": f"{w.name} (T={w.T}): "
                      + (f"routing of all {w.T} tokens ({t_route:.2f} s), " if t_route else "routing given, ")
                      + f"SwiGLU of {len(pick)} of {len(touched)} touched routed experts over all their "
                        f"{rows_exp} rows ({t_exp:.2f} s, scaled by rows to {ids.size} routed rows), shared "
                        f"expert on {min(n_shared_rows, w.T)} rows (scaled to {w.T}); float64 numpy; "
                        f"combine not timed; extrapolated total {total:.1f} s"}


def _csv_rows(d, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def profile_summary(d):
    """Markdown table of a rocprofv3 --kernel-trace --stats run (its *kernel_stats.csv)."""
    rows = _csv_rows(d, "kernel_stats.csv")
    print("| kernel | calls | average µs | min µs | max µs | total ms | % of GPU time |")
    print("|---|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("(anonymous namespace)::", "")
        if name.endswith(")"):  # drop the parameter list, keep template arguments such as (moe::QFormat)1
            name = name[:name.rfind("(")]
        print(f"| `{name[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")


def _counter_means(d, counter):
    """Mean counter value per dispatch, keyed by kernel symbol."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic_summary(workload, fdir, wdir):
    """HBM bytes per dispatch of the library's kernels from a FETCH_SIZE run and a WRITE_SIZE run,
    each scaled by what the same counter reads for a copy of CALIB_BYTES (read and written)."""
    fetch, write = _counter_means(fdir, "FETCH_SIZE"), _counter_means(wdir, "WRITE_SIZE")

    def pick(means, sym):
        hits = [v for k, v in means.items() if sym in k]
        return sum(hits) / len(hits) if hits else None

    cf, cw = pick(fetch, CALIB_SYMBOL), pick(write, CALIB_SYMBOL)
    if not cf or not cw:
        raise SystemExit("the calibration copy is missing (run the bench with --pmc-calibrate)")
    kf, kw = CALIB_BYTES / (cf * 1024), CALIB_BYTES / (cw * 1024)
    print(f"Calibration: a copy of {CALIB_BYTES} bytes (torch.neg, bf16) reads FETCH_SIZE = {cf:.0f} KiB and "
          f"WRITE_SIZE = {cw:.0f} KiB per dispatch, so the counters are scaled by {kf:.4f} (fetch) and "
          f"{kw:.4f} (write).\n")
    print("| kernel | FETCH_SIZE KiB / dispatch | WRITE_SIZE KiB / dispatch | HBM bytes / launch (scaled) |")
    print("|---|---|---|---|")
    recs = []
    for name, (sym, _) in KERNEL_SYMBOLS.items():
        f, w_ = pick(fetch, sym), pick(write, sym)
        if f is None or w_ is None:
            continue
        fb, wb = f * 1024 * kf, w_ * 1024 * kw
        print(f"| {name} | {f:.0f} | {w_:.0f} | {fb + wb:.4g} |")
        recs.append({"workload": workload, "kernel": name, "sources": sources_digest(name), "fetch_kib": f,
                     "write_kib": w_, "fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb})
    print("\n```json\n" + json.dumps(recs, indent=1) + "\n```")


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F16")
SIMDS = 256 * 4            # MI355X: 256 CUs x 4 SIMDs
XCDS = 8                   # GRBM_GUI_ACTIVE has one instance per XCD, all counting the same cycles


def mfma_summary(workload, d):
    """Matrix-core busy time of the library's kernels from one rocprofv3 --pmc pass over
    MFMA_COUNTERS.  busy % = SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (GPU cycles x SIMDs), the
    expression of rocprofv3's MfmaUtil metric, whose GPU cycles are the largest GRBM_GUI_ACTIVE
    instance; the CSV holds the sum over the XCDs' instances, hence / XCDS.  The cycles per µs give
    the clock the kernel ran at.  MFMA work from the MOPS counters (one count per 512 FLOP)."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] not in MFMA_COUNTERS:
            continue
        rec = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        rec[r["Counter_Name"]] = float(r["Counter_Value"])
    print("| kernel | dispatches | µs | clock MHz | MFMA busy % of cycles | MFMA TFLOP / dispatch | TFLOP/s | "
          "% of 2.5 PFLOP/s |")
    print("|---|---|---|---|---|---|---|---|")
    recs = []
    for name, (sym, _) in KERNEL_SYMBOLS.items():
        hits = [v for v in per.values() if sym in v["name"] and all(c in v for c in MFMA_COUNTERS)]
        if not hits:
            continue
        n = len(hits)
        mean = {c: sum(h[c] for h in hits) / n for c in MFMA_COUNTERS}
        us = sum(h["ns"] for h in hits) / n / 1e3
        cycles = mean["GRBM_GUI_ACTIVE"] / XCDS
        busy = 100 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMDS)
        tflop = (mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + mean["SQ_INSTS_VALU_MFMA_MOPS_F16"]) * 512 / 1e12
        rate = tflop / (us * 1e-6)
        print(f"| {name} | {n} | {us:.1f} | {cycles / us:.0f} | {busy:.1f} | {tflop:.4g} | {rate:.0f} | "
              f"{100 * rate * 1e12 / BF16_PEAK:.1f} |")
        recs.append({"workload": workload, "kernel": name, "dispatches": n, "us": us, "clock_mhz": cycles / us,
                     "mfma_busy_pct": busy, "mfma_tflop": tflop, **{c: mean[c] for c in MFMA_COUNTERS}})
    print("\n```json\n" + json.dumps(recs, indent=1) + "\n```")


LDS_COUNTERS = ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE")
CUS = 256                  # MI355X compute units


def lds_summary(workload, d):
    """LDS use of the library's kernels from one rocprofv3 --pmc pass over LDS_COUNTERS: LDS busy % of
    cycles = SQ_LDS_IDX_ACTIVE (summed over CUs) / (GPU cycles x CUs), the expression of rocprofv3's
    LdsUtil metric (GPU cycles: GRBM_GUI_ACTIVE of one XCD, the CSV summing the XCDs' instances);
    bank-conflict cycles per LDS-active cycle, and LDS instructions per dispatch."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] not in LDS_COUNTERS:
            continue
        rec = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        rec[r["Counter_Name"]] = float(r["Counter_Value"])
    print("| kernel | dispatches | µs | LDS busy % of cycles | bank-conflict cycles per LDS-active cycle | "
          "LDS instructions / dispatch |")
    print("|---|---|---|---|---|---|")
    recs = []
    for name, (sym, _) in KERNEL_SYMBOLS.items():
        hits = [v for v in per.values() if sym in v["name"] and all(c in v for c in LDS_COUNTERS)]
        if not hits:
            continue
        n = len(hits)
        mean = {c: sum(h[c] for h in hits) / n for c in LDS_COUNTERS}
        us = sum(h["ns"] for h in hits) / n / 1e3
        cycles = mean["GRBM_GUI_ACTIVE"] / XCDS
        busy = 100 * mean["SQ_LDS_IDX_ACTIVE"] / (cycles * CUS)
        conf = mean["SQ_LDS_BANK_CONFLICT"] / max(mean["SQ_LDS_IDX_ACTIVE"], 1.0)
        print(f"| {name} | {n} | {us:.1f} | {busy:.1f} | {conf:.3f} | {mean['SQ_INSTS_LDS']:.4g} |")
        recs.append({"workload": workload, "kernel": name, "dispatches": n, "us": us, "lds_busy_pct": busy,
                     "bank_conflicts_per_active": conf, **{c: mean[c] for c in LDS_COUNTERS}})
    print("\n```json\n" + json.dumps(recs, indent=1) + "\n```")


def main():
    if len(sys.argv) >= 2 and sys.argv[1] == "--lds-summary":
        return lds_summary(sys.argv[2], sys.argv[3])
    if len(sys.argv) >= 2 and sys.argv[1] == "--profile-summary":
        return profile_summary(sys.argv[2])
    if len(sys.argv) >= 2 and sys.argv[1] == "--traffic-summary":
        return traffic_summary(*sys.argv[2:5])
    if len(sys.argv) >= 2 and sys.argv[1] == "--mfma-summary":
        return mfma_summary(*sys.argv[2:4])
    from moe_layer_forward_amd import workloads as wl
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=list(wl.WORKLOADS))
    ap.add_argument("--also", default="prefill,skew,ep_share,tiny,dense_decode,dense_prefill,decode_int4,decode_fp8,"
                                      "prefill_fp8,prefill_int4",
                    help="comma-separated workloads measured in the same run and reported beside it ('none')")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="first run one copy of known size (the traffic summary's counter calibration)")
    ap.add_argument("--cpu-tokens", type=int, default=64, help="tokens in the oracle's CPU-baseline sample (0: skip)")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring this GPU's read/copy/MFMA peaks")
    ap.add_argument("--no-graph", action="store_true", help="skip timing the step as a replayed HIP graph")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time torch.bmm (hipBLASLt) on the prefill GEMM shapes and print that (context)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this implementation runs on one GPU; --gpus must be 1 (the layer is not sharded "
              "across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.vendor_gemm:
        print(json.dumps({"vendor_gemm": vendor_gemm()}), flush=True)
        return
    main_w = wl.WORKLOADS[args.workload]
    if args.pmc_calibrate:
        a = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
    weights_cache = {}

    def weights_for(w):
        # the four full-size MoE workloads share one weight set; the dense workloads share another;
        # the 4-bit workload has its own (the same weights, quantized)
        shared_moe = w.w_seed == 100 and w.routing != "dense" and w.quant == "none"
        key = (w.w_seed, w.routing == "dense", w.dtype, w.H, w.I, 384 if shared_moe else w.E, w.quant)
        if key not in weights_cache:
            src = wl.WORKLOADS["decode"] if shared_moe else w
            log(f"generating weights for {src.name} ...")
            t0 = time.perf_counter()
            weights_cache[key] = wl.device_weights(src)
            torch.cuda.synchronize()
            phases["weights"] = round(phases["weights"] + time.perf_counter() - t0, 2)
        return weights_cache[key]

    phases = {"weights": 0.0, "workloads": {}, "cpu_baseline": {}}
    t_start = time.perf_counter()
    wt = weights_for(main_w)
    log(f"running {main_w.name} ...")
    t0 = time.perf_counter()
    res = run(main_w, wt, args.steps, args.warmup, graph=not args.no_graph)
    phases["workloads"][main_w.name] = round(time.perf_counter() - t0, 2)
    out = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": main_w.dtype, "data": "synthetic (seeded Irwin-Hall(8) ~normal draws)",
        "config": {"workload": main_w.name, "T": main_w.T, "H": main_w.H, "I": main_w.I, "E": main_w.E,
                   "K": main_w.K, "n_shared": main_w.n_shared, "routed_scaling_factor": main_w.rsf,
                   "parallelism": "1 GPU"},
        "roofline": res["roofline"], "layer": res["layer"], "kernels_us": res["kernels_us"],
        "kernels_roofline": res["kernels_roofline"],
    }
    for name in [n for n in args.also.split(",") if n and n not in ("none", args.workload)]:
        w2 = wl.WORKLOADS[name]
        wt2 = weights_for(w2)
        log(f"running {w2.name} ...")
        t0 = time.perf_counter()
        r2 = run(w2, wt2, args.steps, args.warmup, graph=not args.no_graph)
        phases["workloads"][w2.name] = round(time.perf_counter() - t0, 2)
        out[w2.name] = {"value": r2["tokens_per_s"], "unit": "tokens/s", "ms_per_step": r2["ms_per_step"],
                        "config": {"workload": w2.name, "T": w2.T},
                        "dtype": {"int4": "f16 x int4 (routed), bf16 (shared)",
                                  "fp8": "f16 x e4m3 (routed), bf16 (shared)"}.get(w2.quant, w2.dtype),
                        "roofline": r2["roofline"],
                        "layer": r2["layer"], "kernels_us": r2["kernels_us"],
                        "kernels_roofline": r2["kernels_roofline"]}
    weights_cache.clear()
    torch.cuda.empty_cache()
    if not args.no_peaks:
        log("measuring this GPU's peaks ...")
        t0 = time.perf_counter()
        pk = measure_peaks()
        # the best HBM-bound kernel of this run, beside the read kernels: the "measured read" roof is
        # the highest of them, so no fraction of it exceeds 1
        best = max(((r["achieved"], f"{wn}/{kn}") for wn, kr in
                    [(out["config"]["workload"], out["kernels_roofline"])] +
                    [(k, v["kernels_roofline"]) for k, v in out.items() if isinstance(v, dict) and
                     "kernels_roofline" in v]
                    for kn, r in kr.items() if r["bound"] == "hbm"), default=(0.0, None))
        pk["hbm_read_best_GB_s"] = max(pk["hbm_read_GB_s"], best[0])
        pk["hbm_read_best_of"] = "read kernels" if pk["hbm_read_GB_s"] >= best[0] else f"kernel {best[1]}"
        out["measured_peaks"] = pk
        for layer in [out["layer"]] + [v["layer"] for v in out.values() if isinstance(v, dict) and "layer" in v]:
            layer["hbm_frac_of_measured_read"] = layer["GB_s"] / pk["hbm_read_best_GB_s"]
            layer["mfma_frac_of_measured"] = layer["TFLOP_s"] / pk["mfma_bf16_TFLOP_s"]
        phases["peaks"] = round(time.perf_counter() - t0, 2)
    if args.cpu_tokens > 0:
        log("timing the oracle on the host ...")
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(main_w, min(args.cpu_tokens, main_w.T))
        phases["cpu_baseline"][main_w.name] = round(time.perf_counter() - t0, 2)
        for name in ("prefill", "skew", "ep_share"):
            if name in out and isinstance(out[name], dict):
                log(f"timing the oracle on a sample of {name} ...")
                t0 = time.perf_counter()
                out[name]["cpu_baseline"] = cpu_baseline_sampled(wl.WORKLOADS[name])
                phases["cpu_baseline"][name] = round(time.perf_counter() - t0, 2)
    phases["total"] = round(time.perf_counter() - t_start, 2)
    out["phases_s"] = phases
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
