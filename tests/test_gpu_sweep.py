"""Seeded sweep of small layer shapes within the documented limits (hidden and intermediate sizes
multiples of 128 -- of 256 for 4-bit experts --, up to 64 experts, top-1 to top-8, with and without
the shared expert, router and Zipf-skewed routing, bf16 / 4-bit / FP8 routed experts, 1 to 700
tokens), every token against the oracle through the C ABI.  The shapes reach combinations the
hand-picked cases do not: one or two K steps, a single expert, odd numbers of 128-blocks, more than
4096 (token, expert) pairs, and both kernel families in one call.  A second seeded sweep draws
quantized layers (4-bit and FP8 alternately) with many rows per group, so that they run on the tile
kernels: groups of one to several row tiles, skewed routing, small groups streaming beside tiles.
"""
import numpy as np
import pytest

import moe_layer_forward_amd as moe
from moe_layer_forward_amd import workloads as wl

from parity import Y_TOL, check_routing, oracle_forward_tokens, rel_l2, to_np

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(c):
    rng = np.random.default_rng([2026, c])
    quant = str(rng.choice(["none", "none", "int4", "fp8"]))
    H = int(rng.choice([256, 512, 768] if quant == "int4" else [128, 256, 384, 512, 640]))
    I = int(rng.choice([256, 512] if quant == "int4" else [128, 256, 384, 640]))
    E = int(rng.integers(1, 65))
    K = int(rng.integers(1, min(8, E) + 1))
    T = int(rng.choice([1, 2, 5, 17, 64, 130, 300, 700]))
    shared = int(rng.integers(0, 2))
    routing = str(rng.choice(["router", "skew"]))
    return quant, T, H, I, E, K, shared, routing


@pytest.mark.parametrize("c", range(N_CASES))
def test_sweep_case(c):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    quant, T, H, I, E, K, shared, routing = _case(c)
    print(f"case {c}: quant={quant} T={T} H={H} I={I} E={E} K={K} shared={shared} routing={routing}", flush=True)
    w = wl.custom(f"sweep{c}", T, H, I, E, K, x_seed=300 + c, w_seed=400 + c, routing=routing, n_shared=shared,
                  quant=quant)
    t = wl.device_inputs(w)
    cfg = moe.config_for(w)
    if quant == "none":
        y, ids, wts = moe.moe_forward(cfg, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"],
                                      t.get("ws_gate"), t.get("ws_up"), t.get("ws_down"),
                                      logit_offset=t.get("logit_offset"), return_routing=True)
    else:
        fwd = moe.moe_forward_q4 if quant == "int4" else moe.moe_forward_fp8
        y, ids, wts = fwd(cfg, t["x"], t["w_router"], {k: t[k] for k in moe.QUANT_KEYS}, t.get("ws_gate"),
                          t.get("ws_up"), t.get("ws_down"), logit_offset=t.get("logit_offset"), return_routing=True)
    torch.cuda.synchronize()
    ids_g, w_g, y_g = to_np(ids), to_np(wts), to_np(y)
    y_ref, ids_ref, w_ref, gap = oracle_forward_tokens(w, np.arange(T), ids_gpu=ids_g)
    check_routing(ids_g, w_g, ids_ref, w_ref, gap)
    err = rel_l2(y_g, y_ref)
    print(f"   max rel L2 {err.max():.3g}", flush=True)
    assert np.isfinite(y_g).all()
    assert err.max() <= Y_TOL["bf16"]


N_TILE_CASES = 12


def _tile_case(c):
    """Quantized layers with many rows per group: the tile kernels (and, with 16 groups or more, the
    small groups on the stream kernels beside them), groups of one to several row tiles."""
    rng = np.random.default_rng([2027, c])
    quant = ("int4", "fp8")[c % 2]
    T = int(rng.choice([150, 300, 700, 1200]))
    sizes = [256, 512, 768] if quant == "int4" else [256, 384, 640]
    if T == 1200:
        sizes = sizes[:2]
    H, I = int(rng.choice(sizes)), int(rng.choice(sizes))
    E = int(rng.integers(2, 25))
    K = int(rng.integers(1, min(8, E) + 1))
    shared = int(rng.integers(0, 2))
    routing = str(rng.choice(["router", "skew"]))
    return quant, T, H, I, E, K, shared, routing


@pytest.mark.parametrize("c", range(N_TILE_CASES))
def test_quant_tile_sweep_case(c):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    quant, T, H, I, E, K, shared, routing = _tile_case(c)
    print(f"tile case {c}: quant={quant} T={T} H={H} I={I} E={E} K={K} shared={shared} routing={routing}",
          flush=True)
    w = wl.custom(f"tsweep{c}", T, H, I, E, K, x_seed=500 + c, w_seed=600 + c, routing=routing, n_shared=shared,
                  quant=quant)
    t = wl.device_inputs(w)
    fwd = moe.moe_forward_q4 if quant == "int4" else moe.moe_forward_fp8
    y, ids, wts = fwd(moe.config_for(w), t["x"], t["w_router"], {k: t[k] for k in moe.QUANT_KEYS}, t.get("ws_gate"),
                      t.get("ws_up"), t.get("ws_down"), logit_offset=t.get("logit_offset"), return_routing=True)
    torch.cuda.synchronize()
    ids_g, w_g, y_g = to_np(ids), to_np(wts), to_np(y)
    y_ref, ids_ref, w_ref, gap = oracle_forward_tokens(w, np.arange(T), ids_gpu=ids_g)
    check_routing(ids_g, w_g, ids_ref, w_ref, gap)
    err = rel_l2(y_g, y_ref)
    print(f"   max rel L2 {err.max():.3g}", flush=True)
    assert np.isfinite(y_g).all()
    assert err.max() <= Y_TOL["bf16"]
