"""Parity of the layer with 4-bit routed experts (moe_forward_q4, through the C ABI) with the CPU oracle.

The oracle evaluates the layer in float64 on the dequantized weights (q * s of the host quantizer's
codes and scales); the GPU multiplies in binary16 with fp32 accumulation (the tile kernels round each
weight to f16(q s) first), so the bf16 output bar (per-row relative L2 <= 2e-2) applies.  Cases:
small sizes on every token, on the weight-stream kernels (one or two rows per expert) and on the tile
kernels (many rows per expert: partial and multi-tile groups, ragged tails, the groups of at most 32
rows on the stream kernels beside tiles, an empty tile list, no shared expert, more than 4096
(token, expert) pairs, where the permutation runs as chunked kernels), the tiles while another stream
loads HBM, and the full decode and prefill shapes.  The two quantizers (device for the GPU inputs,
host for the oracle) are checked bit-exact against each other.
"""
import numpy as np
import pytest

import moe_layer_forward_amd as moe
from moe_layer_forward_amd import synth
from moe_layer_forward_amd import workloads as wl

from parity import (Y_TOL, check_routing, oracle_forward_tokens, oracle_outputs_shared_weights, oracle_route,
                    rel_l2, to_np)

pytestmark = pytest.mark.gpu

Q4_KEYS = ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")


def _torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _forward_q4(w, t, score_bias=None):
    cfg = moe.config_for(w)
    return moe.moe_forward_q4(cfg, t["x"], t["w_router"], {k: t[k] for k in Q4_KEYS}, t.get("ws_gate"),
                              t.get("ws_up"), t.get("ws_down"), score_bias=score_bias,
                              logit_offset=t.get("logit_offset"), return_routing=True)


def _check(w, t, tokens=None):
    torch = _torch()
    y, ids, wts = _forward_q4(w, t)
    torch.cuda.synchronize()
    tokens = np.arange(w.T) if tokens is None else np.asarray(tokens)
    ids_g, w_g, y_g = to_np(ids)[tokens], to_np(wts)[tokens], to_np(y)[tokens]
    y_ref, ids_ref, w_ref, gap = oracle_forward_tokens(w, tokens, ids_gpu=ids_g)
    differ = check_routing(ids_g, w_g, ids_ref, w_ref, gap)
    err = rel_l2(y_g, y_ref)
    print(f"{w.name}: T={w.T} checked {len(tokens)} tokens, near-tie swaps {len(differ)}, "
          f"max rel L2 {err.max():.3g}, p99 {np.percentile(err, 99):.3g}", flush=True)
    assert np.isfinite(y_g).all()
    assert err.max() <= Y_TOL["bf16"]
    return y, ids, wts


@pytest.mark.parametrize("T,H,I,E,K,shared", [
    # stream kernels only (at most 4 rows per group)
    (5, 768, 512, 40, 4, 0),     # one or two rows per expert, no shared expert
    (16, 512, 256, 40, 8, 1),    # ~3 rows per expert, 16 shared rows in four 4-row passes
    # tile kernels (192-row tiles)
    (70, 512, 256, 8, 2, 1),     # ~17.5 rows per expert in one partial tile each; K loops all tail
    (600, 1024, 768, 8, 2, 1),   # ~150 rows per expert, 600 shared rows in 4 tiles (ragged); gate/up K
                                 # loop through the steady state, down (12 steps) all tail
    (400, 512, 512, 4, 2, 1),    # ~200 rows per expert: two tiles each, the second a few rows
    (256, 1024, 768, 32, 4, 1),  # 17 groups or more: groups of <= 32 rows on the stream kernels beside
                                 # tiles
    (32, 512, 256, 16, 2, 1),    # every group small, the 32-row shared expert too: empty tile list
    (300, 512, 512, 8, 3, 0),    # tiles without a shared expert
    (200, 256, 512, 16, 2, 1),   # the shared expert's 200 rows in two tiles; H = 256: 2 K blocks
    (600, 256, 256, 32, 8, 1),   # 4800 pairs: the chunked permutation, separate binary16 rows and plan
    (2000, 256, 256, 8, 4, 1),   # ~1000 rows per expert + 2000 shared rows: 32 or more row tiles, dealt to
                                 # the XCDs in blocks of 4 consecutive tiles (one group's, and straddling)
], ids=["no_shared", "shared_passes", "tile_ragged", "tile_steady", "two_tiles", "small_beside_tiles",
        "empty_tile_list", "tile_no_shared", "shared_tiles", "many_pairs", "block_dealing"])
def test_q4_small_every_token(T, H, I, E, K, shared):
    _torch()
    w = wl.custom(f"q4_{T}", T, H, I, E, K, x_seed=31, w_seed=32, n_shared=shared, quant="int4")
    _check(w, wl.device_inputs(w))


def test_q4_single_token():
    _torch()
    w = wl.custom("q4_one", 1, 512, 256, 16, 8, x_seed=33, w_seed=34, quant="int4")
    _check(w, wl.device_inputs(w))


def test_q4_tiles_skewed_routing_with_bias():
    # Zipf-skewed routing plus a score bias: hot experts over several tiles beside many small groups
    torch = _torch()
    w = wl.custom("q4_skew", 200, 512, 256, 32, 4, x_seed=36, w_seed=37, routing="skew", quant="int4")
    t = wl.device_inputs(w)
    bias = torch.linspace(-0.05, 0.05, w.E, device="cuda", dtype=torch.float32)
    y, ids, wts = _forward_q4(w, t, score_bias=bias)
    torch.cuda.synchronize()
    tokens = np.arange(w.T)
    y_ref, ids_ref, w_ref, gap = oracle_forward_tokens(w, tokens, ids_gpu=to_np(ids), score_bias=to_np(bias))
    check_routing(to_np(ids), to_np(wts), ids_ref, w_ref, gap)
    err = rel_l2(to_np(y), y_ref)
    print(f"q4 skew + bias: max rel L2 {err.max():.3g}", flush=True)
    assert err.max() <= Y_TOL["bf16"]


def test_q4_tiles_under_concurrent_memory_traffic():
    # as for the FP8 tiles: each call runs while a torch stream copies 1 GiB buffers, so the tiles'
    # loads land late; every call must match the oracle on every token
    torch = _torch()
    w = wl.custom("q4_traffic", 256, 1024, 768, 32, 4, x_seed=38, w_seed=39, quant="int4")
    t = wl.device_inputs(w)
    big = torch.empty(256 << 20, dtype=torch.float32, device="cuda")
    big2 = torch.empty_like(big)
    side = torch.cuda.Stream()
    cfg = moe.config_for(w)
    y_ref = None
    for rep in range(3):
        ws = moe.alloc_workspace(cfg, moe.MOE_OP_FORWARD_Q4, w.T)
        ws.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(12):
                big2.copy_(big)
        y, ids, wts = moe.moe_forward_q4(cfg, t["x"], t["w_router"], {k: t[k] for k in Q4_KEYS}, t["ws_gate"],
                                         t["ws_up"], t["ws_down"], return_routing=True, workspace=ws)
        torch.cuda.synchronize()
        if y_ref is None:
            y_ref, ids_ref, w_ref, gap = oracle_forward_tokens(w, np.arange(w.T), ids_gpu=to_np(ids))
            check_routing(to_np(ids), to_np(wts), ids_ref, w_ref, gap)
        err = rel_l2(to_np(y), y_ref)
        print(f"q4 under traffic, call {rep}: max rel L2 {err.max():.3g}", flush=True)
        assert err.max() <= Y_TOL["bf16"]
    del big, big2


def test_device_quantizer_matches_host():
    torch = _torch()
    rows, cols = 96, 7168
    bits = synth.host_tensor(35, 2, 0, (rows, cols), 1.0 / np.sqrt(7168), "bf16")
    # groups with special content: all zero, one large value, a constant negative group, a scale in
    # the binary16 subnormal range (q clamps to 7), a scale that rounds to zero (q = 0)
    bits = bits.copy()
    bits[0, :32] = 0
    bits[1, 32:64] = 0
    bits[1, 40] = 0x4300        # 128.0
    bits[2, 64:96] = 0xC000     # -2.0 everywhere
    bits[3, :32] = 0x3500       # 2^-21: s = 2^-24, w / s = 8
    bits[4, :32] = 0x3380       # 2^-24: max|w| / 7 rounds to a zero scale
    w = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    codes = torch.empty((rows, cols // 8), dtype=torch.int32, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.int16, device="cuda")
    synth.device_quantize_q4(w, codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = synth.host_quantize_q4(bits)
    np.testing.assert_array_equal(codes.cpu().numpy().view(np.uint32), c_ref)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint16), s_ref)


def test_q4_rejects_f32_and_unaligned_sizes():
    torch = _torch()
    x = torch.zeros((4, 384), dtype=torch.bfloat16, device="cuda")
    q = {k: torch.zeros(4, dtype=torch.int32 if k.endswith("codes") else torch.int16, device="cuda")
         for k in Q4_KEYS}
    wr = torch.zeros((8, 384), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for cfg in (moe.make_config(384, 256, 8, 2, 0), moe.make_config(512, 256, 8, 2, 0, dtype="f32")):
        with pytest.raises(moe.MoeError) as e:
            moe.moe_forward_q4(cfg, x, wr, q, workspace=ws)
        assert e.value.status == moe.MOE_ERR_UNSUPPORTED


PREFILL_SAMPLE = 256  # seeded prefill tokens whose outputs are compared


@pytest.mark.timeout(1200)
def test_int4_full_size():
    """decode_int4 (every token, weight-stream kernels) and prefill_int4 (routing of every token, outputs
    of a seeded sample: every expert, groups of ~170 rows on the 192-row tiles, a few in two tiles) at
    the full shape, one weight set, each in the benchmark's launch configuration (one moe_forward_q4
    call)."""
    torch = _torch()
    wd, wp = wl.WORKLOADS["decode_int4"], wl.WORKLOADS["prefill_int4"]
    t = wl.device_weights(wd)
    runs = {}
    for w in (wd, wp):
        print(f"running {w.name} (T={w.T}) on the GPU", flush=True)
        tw = dict(t, **wl.device_activations(w))
        y, ids, wts = _forward_q4(w, tw)
        torch.cuda.synchronize()
        runs[w.name] = (to_np(y), to_np(ids), to_np(wts))
        del tw, y, ids, wts
    del t
    torch.cuda.empty_cache()
    for w in (wd, wp):
        _, ids_g, wts_g = runs[w.name]
        x, ids_ref, w_ref, gap, _ = oracle_route(w, np.arange(w.T))
        check_routing(ids_g, wts_g, ids_ref, w_ref, gap)
    rng = np.random.default_rng(20261205)
    sample = np.sort(rng.choice(wp.T, PREFILL_SAMPLE, replace=False))
    cases = [(wd, np.arange(wd.T), runs[wd.name][1]), (wp, sample, runs[wp.name][1][sample])]
    refs = oracle_outputs_shared_weights(cases)
    for (w, tokens, ids_g), (y_ref, ids_r, w_r, gap_r) in zip(cases, refs):
        y_g, _, w_g = runs[w.name]
        check_routing(ids_g, w_g[tokens], ids_r, w_r, gap_r)
        err = rel_l2(y_g[tokens], y_ref)
        print(f"{w.name}: outputs of {len(tokens)} tokens checked, max rel L2 {err.max():.3g}, "
              f"p99 {np.percentile(err, 99):.3g}", flush=True)
        assert np.isfinite(y_g).all()
        assert err.max() <= Y_TOL["bf16"]
