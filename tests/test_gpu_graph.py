"""The layer call inside a captured HIP graph (torch.cuda.CUDAGraph), bf16 and quantized experts.

The library launches only kernels on the caller's stream (no allocation, copy, memset or
synchronisation inside a call), so a serving loop can capture `moe_forward` once and replay it.
Every replay must reproduce the eager call bit for bit (the kernels are deterministic: fixed
reduction orders, no floating-point atomics); replays are interleaved with eager work and
synchronisations, and the inputs are changed in place between replays.
"""
import pytest

import moe_layer_forward_amd as moe
from moe_layer_forward_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("T", [24, 300], ids=["stream_kernels", "tile_kernels"])
def test_forward_graph_replays_match_eager(T):
    torch = _torch()
    w = wl.custom(f"graph_{T}", T=T, H=512, I=256, E=40, K=4, x_seed=41, w_seed=42)
    t = wl.device_inputs(w)
    cfg = moe.config_for(w)
    ws = moe.alloc_workspace(cfg, moe.MOE_OP_FORWARD, T)
    y = torch.empty((T, w.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.K), dtype=torch.float32, device="cuda")

    def call():
        moe.moe_forward(cfg, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], t["ws_gate"],
                        t["ws_up"], t["ws_down"], workspace=ws, out=y, routing_out=(ids, wts))

    x0 = t["x"].clone()
    x1 = torch.flip(x0, dims=[0]).contiguous()  # a second input: the tokens in reverse order
    refs = []
    for xin in (x0, x1):
        t["x"].copy_(xin)
        call()
        torch.cuda.synchronize()
        refs.append((y.clone(), ids.clone(), wts.clone()))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    for rep in range(4):
        which = rep % 2
        t["x"].copy_(x1 if which else x0)
        y.zero_()
        ids.fill_(-1)
        g.replay()
        scratch = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        y_ref, ids_ref, w_ref = refs[which]
        assert torch.equal(ids, ids_ref), f"replay {rep}: routing differs"
        assert torch.equal(wts, w_ref), f"replay {rep}: routing weights differ"
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"replay {rep}: output differs"
        assert torch.isfinite(scratch)
    del g


@pytest.mark.parametrize("quant,T,E", [("int4", 24, 40), ("fp8", 24, 40), ("int4", 300, 8), ("fp8", 300, 8)],
                         ids=["int4_stream", "fp8_stream", "int4_tiles", "fp8_tiles"])
def test_quantized_forward_graph_replays_match_eager(quant, T, E):
    # T=24 over 40 experts: the weight-stream kernels; T=300 over 8: the tile kernels (~150 rows per group)
    torch = _torch()
    w = wl.custom(f"graph_{quant}_{T}", T=T, H=512, I=256, E=E, K=4, x_seed=43, w_seed=44, quant=quant)
    t = wl.device_inputs(w)
    cfg = moe.config_for(w)
    fwd, op = ((moe.moe_forward_q4, moe.MOE_OP_FORWARD_Q4) if quant == "int4"
               else (moe.moe_forward_fp8, moe.MOE_OP_FORWARD_FP8))
    ws = moe.alloc_workspace(cfg, op, T)
    y = torch.empty((T, w.H), dtype=torch.bfloat16, device="cuda")
    q = {k: t[k] for k in moe.QUANT_KEYS}

    def call():
        fwd(cfg, t["x"], t["w_router"], q, t["ws_gate"], t["ws_up"], t["ws_down"], workspace=ws, out=y)

    x0 = t["x"].clone()
    x1 = torch.flip(x0, dims=[0]).contiguous()
    refs = []
    for xin in (x0, x1):
        t["x"].copy_(xin)
        call()
        torch.cuda.synchronize()
        refs.append(y.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    for rep in range(4):
        which = rep % 2
        t["x"].copy_(x1 if which else x0)
        y.zero_()
        g.replay()
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), refs[which].view(torch.int16)), f"replay {rep}: output differs"
        assert torch.isfinite(scratch)
    del g
