"""The five synthetic workloads of the K2 MoE layer, and how their inputs are made.

Shapes and distributions (all draws seeded, see ``synth``):

==========  =====  ====  ====  ===  ==  ======  ==================================
name          T      H     I    E   K  dtype   routing
==========  =====  ====  ====  ===  ==  ======  ==================================
tiny           64   256   128   16   2  f32     sigmoid router
decode         64  7168  2048  384   8  bf16    sigmoid router
prefill      8192  7168  2048  384   8  bf16    sigmoid router (near-uniform)
skew         4096  7168  2048  384   8  bf16    router + Zipf-shaped logit offsets
ep_share    16384  7168  2048    3   1  bf16    pre-dispatched ids/weights, no router
dense_*     64 /   7168 18432    1   1  bf16    none: the dense SwiGLU FFN of the
            8192                                 model's first layer, all tokens
decode_int4    64  7168  2048  384   8  bf16    as decode; routed experts stored as
                                                 4-bit codes + binary16 scales
decode_fp8     64  7168  2048  384   8  bf16    as decode; routed experts stored as
                                                 E4M3 codes + fp32 128x128-block scales
prefill_fp8  8192  7168  2048  384   8  bf16    as prefill; routed experts as decode_fp8
prefill_int4 8192  7168  2048  384   8  bf16    as prefill; routed experts as decode_int4
==========  =====  ====  ====  ===  ==  ======  ==================================


Each MoE workload has one always-on shared expert of the routed experts'
shape and the routed scaling factor 2.827.  The dense workloads are the
7168 -> 18432 -> 7168 SwiGLU FFN of layer 0 (no router, no experts): one
group of all T rows on the grouped-SwiGLU kernels, weight 1.

Distributions: activations N(0, 1); router weight N(0, 0.02); gate/up
N(0, 1/sqrt(H)); down N(0, 1/sqrt(I)) -- "N(0, a)" reads a as a standard
deviation.  Draws are Irwin-Hall(8) approximately-normal variates (see
``synth``).  The four full-shape workloads share one weight set (seed 100);
their activations use the workload number (2..5) as seed; tiny uses seed 1.

decode_int4 has decode's tokens and weights; its routed experts are those bf16
weights quantized per group of 32 inputs (s = f16(max|w| / 7), q = clamp(rint(w / s),
-8, 7)) -- the checkpoint-conversion step, done on the device for the GPU and on
the host for the oracle by two implementations of the same rule (``synth``).
decode_fp8 likewise quantizes them per 128 x 128 block (s = max|w| / 448, c = E4M3
round-to-nearest-even of w / s); prefill_fp8 and prefill_int4 have prefill's tokens and
those codes.

Synthetic streams: 0 activations, 1 router, 2 gate, 3 up, 4 down, 5/6/7 shared
gate/up/down, 11/12/13 dense gate/up/down (Philox, index = expert id); 8 skew
permutation, 9 EP-share ids, 10 EP-share weights (numpy PCG64 from
SeedSequence([seed, stream])).

Skew offsets: o_e = -1.1 * ln(r_e) added to expert e's logit before the
sigmoid, r a seeded permutation of 1..E -- a Zipf(s = 1.1)-shaped popularity
prior.  Exact Zipf counts are impossible under top-8 (the hottest expert
would need more picks than there are tokens), so the offsets shape the
logits and the realised histogram is reported.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

from . import synth

RSF_K2 = 2.827

S_X, S_ROUTER, S_GATE, S_UP, S_DOWN, S_SGATE, S_SUP, S_SDOWN = range(8)
S_SKEW, S_EP_IDS, S_EP_W = 8, 9, 10
S_DGATE, S_DUP, S_DDOWN = 11, 12, 13
DENSE_I = 18432  # intermediate size of the dense first-layer FFN


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    K: int
    dtype: str                    # 'bf16' | 'f32'
    x_seed: int
    w_seed: int
    routing: str = "router"       # 'router' | 'skew' | 'preassigned' | 'dense'
    n_shared: int = 1
    rsf: float = RSF_K2
    sigma_x: float = 1.0
    sigma_router: float = 0.02
    quant: str = "none"           # 'none' | 'int4' | 'fp8' (routed experts stored as codes + scales)
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def sigma_gate_up(self) -> float:
        return 1.0 / math.sqrt(self.H)

    @property
    def sigma_down(self) -> float:
        return 1.0 / math.sqrt(self.I)

    @property
    def pairs(self) -> int:
        return self.T * self.K

    def with_tokens(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 128, 16, 2, "f32", x_seed=1, w_seed=1),
    "decode": Workload("decode", 64, 7168, 2048, 384, 8, "bf16", x_seed=2, w_seed=100),
    "prefill": Workload("prefill", 8192, 7168, 2048, 384, 8, "bf16", x_seed=3, w_seed=100),
    "skew": Workload("skew", 4096, 7168, 2048, 384, 8, "bf16", x_seed=4, w_seed=100, routing="skew"),
    "ep_share": Workload("ep_share", 16384, 7168, 2048, 3, 1, "bf16", x_seed=5, w_seed=100,
                         routing="preassigned"),
    "dense_decode": Workload("dense_decode", 64, 7168, DENSE_I, 1, 1, "bf16", x_seed=6, w_seed=100,
                             routing="dense", n_shared=0),
    "dense_prefill": Workload("dense_prefill", 8192, 7168, DENSE_I, 1, 1, "bf16", x_seed=7, w_seed=100,
                              routing="dense", n_shared=0),
    "decode_int4": Workload("decode_int4", 64, 7168, 2048, 384, 8, "bf16", x_seed=2, w_seed=100, quant="int4"),
    "decode_fp8": Workload("decode_fp8", 64, 7168, 2048, 384, 8, "bf16", x_seed=2, w_seed=100, quant="fp8"),
    "prefill_fp8": Workload("prefill_fp8", 8192, 7168, 2048, 384, 8, "bf16", x_seed=3, w_seed=100, quant="fp8"),
    "prefill_int4": Workload("prefill_int4", 8192, 7168, 2048, 384, 8, "bf16", x_seed=3, w_seed=100, quant="int4"),
}


def custom(name, T, H, I, E, K, dtype="bf16", x_seed=11, w_seed=12, routing="router", n_shared=1, quant="none"):
    """A workload with the same recipe at other sizes (parity cases)."""
    return Workload(name, T, H, I, E, K, dtype, x_seed, w_seed, routing, n_shared, quant=quant)


# --------------------------------------------------------------------------- host side
def _np_rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def logit_offsets(w: Workload):
    """fp32 [E] skew offsets, or None."""
    if w.routing != "skew":
        return None
    r = _np_rng(w.x_seed, S_SKEW).permutation(w.E) + 1
    return (-1.1 * np.log(r.astype(np.float64))).astype(np.float32)


def preassigned(w: Workload):
    """(ids int32 [T,K], weights fp32 [T,K]) for the pre-dispatched EP share."""
    ids = _np_rng(w.x_seed, S_EP_IDS).integers(0, w.E, size=(w.T, w.K)).astype(np.int32)
    wts = (_np_rng(w.x_seed, S_EP_W).uniform(0.05, 0.6, size=(w.T, w.K)) * w.rsf).astype(np.float32)
    return ids, wts


def _to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def host_x_rows(w: Workload, rows) -> np.ndarray:
    return _to_f64(synth.host_rows(w.x_seed, S_X, 0, w.H, rows, w.sigma_x, w.dtype), w.dtype)


def host_x(w: Workload) -> np.ndarray:
    return host_x_rows(w, np.arange(w.T))


def host_router(w: Workload) -> np.ndarray:
    return _to_f64(synth.host_tensor(w.w_seed, S_ROUTER, 0, (w.E, w.H), w.sigma_router, w.dtype), w.dtype)


def _expert_streams(w: Workload):
    return (S_DGATE, S_DUP, S_DDOWN) if w.routing == "dense" else (S_GATE, S_UP, S_DOWN)


def host_expert(w: Workload, e: int):
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) of routed expert e (the dense FFN for 'dense'), float64."""
    sg, su, sd = _expert_streams(w)
    g = synth.host_tensor(w.w_seed, sg, e, (w.I, w.H), w.sigma_gate_up, w.dtype)
    u = synth.host_tensor(w.w_seed, su, e, (w.I, w.H), w.sigma_gate_up, w.dtype)
    d = synth.host_tensor(w.w_seed, sd, e, (w.H, w.I), w.sigma_down, w.dtype)
    return _to_f64(g, w.dtype), _to_f64(u, w.dtype), _to_f64(d, w.dtype)


def host_expert_q4(w: Workload, e: int):
    """4-bit storage of routed expert e: ((codes, scales) of W_gate, W_up, W_down), quantized on the host
    from the expert's bf16 weights (``synth.host_quantize_q4``)."""
    sg, su, sd = _expert_streams(w)
    out = []
    for stream, shape, sigma in ((sg, (w.I, w.H), w.sigma_gate_up), (su, (w.I, w.H), w.sigma_gate_up),
                                 (sd, (w.H, w.I), w.sigma_down)):
        out.append(synth.host_quantize_q4(synth.host_tensor(w.w_seed, stream, e, shape, sigma, "bf16")))
    return tuple(out)


def host_expert_fp8(w: Workload, e: int):
    """8-bit storage of routed expert e: ((codes, scales) of W_gate, W_up, W_down), quantized on the host
    from the expert's bf16 weights (``synth.host_quantize_fp8``)."""
    sg, su, sd = _expert_streams(w)
    out = []
    for stream, shape, sigma in ((sg, (w.I, w.H), w.sigma_gate_up), (su, (w.I, w.H), w.sigma_gate_up),
                                 (sd, (w.H, w.I), w.sigma_down)):
        out.append(synth.host_quantize_fp8(synth.host_tensor(w.w_seed, stream, e, shape, sigma, "bf16")))
    return tuple(out)


def host_shared(w: Workload):
    if w.n_shared == 0:
        return None
    g = synth.host_tensor(w.w_seed, S_SGATE, 0, (w.I, w.H), w.sigma_gate_up, w.dtype)
    u = synth.host_tensor(w.w_seed, S_SUP, 0, (w.I, w.H), w.sigma_gate_up, w.dtype)
    d = synth.host_tensor(w.w_seed, S_SDOWN, 0, (w.H, w.I), w.sigma_down, w.dtype)
    return _to_f64(g, w.dtype), _to_f64(u, w.dtype), _to_f64(d, w.dtype)


# --------------------------------------------------------------------------- device side
def device_weights(w: Workload, device="cuda"):
    """Router, routed-expert and shared-expert weights of the workload (the dense FFN as expert 0 for
    'dense'), generated in HBM.  For quant 'int4' the routed experts come as gate/up/down codes
    (int32 words) and scales (int16 words holding binary16), quantized on the device
    (``synth.device_quantize_q4``) from the same bf16 weights, a chunk of experts at a time; for
    'fp8' as uint8 E4M3 codes and float32 block scales (``synth.device_quantize_fp8``)."""
    import torch

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {}
    if w.routing not in ("preassigned", "dense"):
        t["w_router"] = synth.device_fill(torch.empty((w.E, w.H), dtype=dt, device=device), w.w_seed, S_ROUTER,
                                          0, 1, w.E * w.H, w.sigma_router)
    sg, su, sd = _expert_streams(w)
    mats = (("gate", sg, (w.I, w.H), w.sigma_gate_up), ("up", su, (w.I, w.H), w.sigma_gate_up),
            ("down", sd, (w.H, w.I), w.sigma_down))
    if w.quant == "int4":
        if w.dtype != "bf16":
            raise ValueError("4-bit experts are quantized from bf16 weights")
        chunk = min(w.E, 32)
        for name, stream, (n, k), sigma in mats:
            codes = torch.empty((w.E, n, k // 8), dtype=torch.int32, device=device)
            scales = torch.empty((w.E, n, k // 32), dtype=torch.int16, device=device)
            buf = torch.empty((chunk, n, k), dtype=torch.bfloat16, device=device)
            for e0 in range(0, w.E, chunk):
                m = min(chunk, w.E - e0)
                synth.device_fill(buf[:m], w.w_seed, stream, e0, m, n * k, sigma)
                synth.device_quantize_q4(buf[:m], codes[e0:e0 + m], scales[e0:e0 + m])
            t[f"{name}_codes"], t[f"{name}_scales"] = codes, scales
            del buf
    elif w.quant == "fp8":
        if w.dtype != "bf16":
            raise ValueError("FP8 experts are quantized from bf16 weights")
        chunk = min(w.E, 32)
        for name, stream, (n, k), sigma in mats:
            codes = torch.empty((w.E, n, k), dtype=torch.uint8, device=device)
            scales = torch.empty((w.E, n // 128, k // 128), dtype=torch.float32, device=device)
            buf = torch.empty((chunk, n, k), dtype=torch.bfloat16, device=device)
            for e0 in range(0, w.E, chunk):
                m = min(chunk, w.E - e0)
                synth.device_fill(buf[:m], w.w_seed, stream, e0, m, n * k, sigma)
                synth.device_quantize_fp8(buf[:m], codes[e0:e0 + m], scales[e0:e0 + m])
            t[f"{name}_codes"], t[f"{name}_scales"] = codes, scales
            del buf
    else:
        for name, stream, (n, k), sigma in mats:
            t[f"w_{name}"] = synth.device_fill(torch.empty((w.E, n, k), dtype=dt, device=device), w.w_seed, stream,
                                               0, w.E, n * k, sigma)
    if w.n_shared:
        t["ws_gate"] = synth.device_fill(torch.empty((w.I, w.H), dtype=dt, device=device), w.w_seed, S_SGATE, 0,
                                         1, w.I * w.H, w.sigma_gate_up)
        t["ws_up"] = synth.device_fill(torch.empty((w.I, w.H), dtype=dt, device=device), w.w_seed, S_SUP, 0, 1,
                                       w.I * w.H, w.sigma_gate_up)
        t["ws_down"] = synth.device_fill(torch.empty((w.H, w.I), dtype=dt, device=device), w.w_seed, S_SDOWN, 0,
                                         1, w.H * w.I, w.sigma_down)
    return t


def device_activations(w: Workload, device="cuda"):
    """Token rows (and skew offsets / pre-assigned routing) of the workload, in HBM."""
    import torch

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {"x": synth.device_fill(torch.empty((w.T, w.H), dtype=dt, device=device), w.x_seed, S_X, 0, 1,
                                w.T * w.H, w.sigma_x)}
    off = logit_offsets(w)
    if off is not None:
        t["logit_offset"] = torch.from_numpy(off).to(device)
    if w.routing == "preassigned":
        ids, wts = preassigned(w)
        t["topk_ids"] = torch.from_numpy(ids).to(device)
        t["topk_weights"] = torch.from_numpy(wts).to(device)
    return t


def device_inputs(w: Workload, device="cuda"):
    """All inputs of the workload, resident in HBM (torch tensors)."""
    t = device_weights(w, device)
    t.update(device_activations(w, device))
    return t
