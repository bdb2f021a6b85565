"""moe_forward_noalloc: the layer with the library's fixed per-GPU scratch instead of a caller
workspace (for callers that cannot allocate).  Its results must equal moe_forward's on the same
inputs bit for bit (the same kernels in the same launch configuration), on two calls in a row, the
second smaller, so the second runs on the first one's leftover scratch contents."""
import numpy as np
import pytest

import moe_layer_forward_amd as moe
from moe_layer_forward_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _both(w, t):
    """(moe_forward results, moe_forward_noalloc results) on the same inputs: y, ids, weights."""
    torch = _torch()
    cfg = moe.config_for(w)
    args = (cfg, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], t["ws_gate"], t["ws_up"], t["ws_down"])
    ref = moe.moe_forward(*args, logit_offset=t.get("logit_offset"), return_routing=True)
    y = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((w.T, w.K), -1, dtype=torch.int32, device="cuda")
    wts = torch.full((w.T, w.K), float("nan"), dtype=torch.float32, device="cuda")
    got = moe.moe_forward_noalloc(*args, logit_offset=t.get("logit_offset"), out=y, routing_out=(ids, wts))
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("sizes", [(300, 20), (600, 64)], ids=["tile_then_stream", "skew_then_decode_like"])
def test_noalloc_matches_forward_two_calls(sizes):
    """Two calls in a row, the second with fewer tokens: the first on the tile kernels (more than 4 rows
    per group), the second on the weight-stream kernels; the second pair uses skewed routing and 4800
    pairs, so its first call mixes both kernel families and the permutation's chunked path."""
    _torch()
    T1, T2 = sizes
    routing = "skew" if T1 == 600 else "router"
    H, I, E, K = (512, 256, 40, 4) if T1 == 300 else (512, 256, 64, 8)
    for T in (T1, T2):
        w = wl.custom("noalloc", T=T, H=H, I=I, E=E, K=K, routing=routing)
        t = wl.device_inputs(w)
        (y_r, ids_r, w_r), (y_n, ids_n, w_n) = _both(w, t)
        assert _torch().equal(ids_r, ids_n), f"T={T}: routing ids differ"
        assert _torch().equal(w_r, w_n), f"T={T}: routing weights differ"
        assert _torch().equal(y_r, y_n), f"T={T}: outputs differ"
        print(f"noalloc T={T}: identical to moe_forward", flush=True)


def test_noalloc_rejects_beyond_its_scratch():
    """A call whose workspace would exceed the fixed scratch returns MOE_ERR_WORKSPACE and launches
    nothing (the output keeps its contents)."""
    torch = _torch()
    cfg = moe.make_config(hidden_size=1024, moe_intermediate_size=512, n_routed_experts=16, top_k=4)
    T = 1
    while moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD, T) <= moe.MOE_NOALLOC_SCRATCH_BYTES:
        T *= 2
    x = torch.zeros((T, 1024), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((16, 1024), dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros((16, 512, 1024), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((16, 1024, 512), dtype=torch.bfloat16, device="cuda")
    sg = torch.zeros((512, 1024), dtype=torch.bfloat16, device="cuda")
    sd = torch.zeros((1024, 512), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, 1024), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(cfg, x, wr, wg, wg, wd, sg, sg, sd, out=y)
    assert e.value.status == moe.MOE_ERR_WORKSPACE and "scratch" in e.value.message
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
