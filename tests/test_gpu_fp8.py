"""Parity of the layer with FP8 routed experts (moe_forward_fp8, through the C ABI) with the CPU oracle.

The oracle evaluates the layer in float64 on the dequantized weights (E4M3 value times its 128 x 128
block scale, from the host quantizer's codes and scales); the GPU multiplies in binary16 with fp32
accumulation, so the bf16 output bar (per-row relative L2 <= 2e-2) applies.

Two kernel families run the experts: with at most 4 rows per group on average the weight-stream
kernels take every group; otherwise the tile kernels take the groups of more than 32 rows (all of
them with fewer than 16 groups), the shared expert's included, and the stream kernels the rest.
Cases, every token: stream-only shapes (no shared expert; a long W_down row whose scales do not fit
the chained down kernel; hidden_size at its 8192 limit; a skewed routing whose hot experts take
several 16-row passes; a single token) and tile shapes (groups of one or more 256-row tiles with
ragged tails; odd numbers of 128-blocks and a last output slab of 128 columns; K loops long enough
for the unrolled steady state and short ones that are all tail; small groups beside tiles, also while
other work loads HBM concurrently; a shared expert small enough for the stream kernels beside an
empty tile list; no shared expert; more than 4096 (token, expert) pairs); and the full decode and
prefill shapes (every decode token, a seeded
sample of prefill tokens, in one oracle pass).  The two quantizers (device for the GPU inputs, host
for the oracle) are checked bit-exact against each other.
"""
import numpy as np
import pytest

import moe_layer_forward_amd as moe
from moe_layer_forward_amd import synth
from moe_layer_forward_amd import workloads as wl

from parity import (Y_TOL, check_routing, oracle_forward_tokens, oracle_outputs_shared_weights, oracle_route, rel_l2,
                    to_np)

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _check(w, t, tokens=None, bias=None):
    torch = _torch()
    cfg = moe.config_for(w)
    y, ids, wts = moe.moe_forward_fp8(cfg, t["x"], t["w_router"], {k: t[k] for k in moe.QUANT_KEYS},
                                      t.get("ws_gate"), t.get("ws_up"), t.get("ws_down"),
                                      score_bias=None if bias is None else torch.from_numpy(bias).cuda(),
                                      logit_offset=t.get("logit_offset"), return_routing=True)
    torch.cuda.synchronize()
    tokens = np.arange(w.T) if tokens is None else np.asarray(tokens)
    ids_g, w_g, y_g = to_np(ids)[tokens], to_np(wts)[tokens], to_np(y)[tokens]
    y_ref, ids_ref, w_ref, gap = oracle_forward_tokens(w, tokens, ids_gpu=ids_g, score_bias=bias)
    differ = check_routing(ids_g, w_g, ids_ref, w_ref, gap)
    err = rel_l2(y_g, y_ref)
    print(f"{w.name}: T={w.T} checked {len(tokens)} tokens, near-tie swaps {len(differ)}, "
          f"max rel L2 {err.max():.3g}, p99 {np.percentile(err, 99):.3g}", flush=True)
    assert np.isfinite(y_g).all()
    assert err.max() <= Y_TOL["bf16"]
    return y, ids, wts


@pytest.mark.parametrize("T,H,I,E,K,shared", [
    # stream kernels only (at most 4 rows per group)
    (5, 768, 512, 40, 4, 0),     # one or two rows per expert, no shared expert; chained down blocks
    (8, 256, 4608, 8, 2, 1),     # W_down rows of 36 blocks: scales too many for the chained down kernel
    (6, 8192, 256, 8, 2, 1),     # hidden_size 8192: 64 gate/up scale blocks per row, one per lane
    # tile kernels
    (70, 512, 256, 8, 2, 1),     # ~17.5 rows per expert in one partial tile each; K loops all tail
    (40, 384, 640, 12, 3, 1),    # 3 x 5 blocks: a down output slab of 128 columns (its scales clamp)
    (600, 896, 640, 8, 2, 1),    # ~150 rows per expert, 600 shared rows in 3 tiles (ragged); gate/up
                                 # K loop through the steady state, down (10 steps) all tail
    (256, 1024, 768, 32, 4, 1),  # 17 groups or more: groups of <= 32 rows on the stream kernels
                                 # beside tiles; both K loops through the steady state
    (32, 512, 256, 16, 2, 1),    # every group small, the 32-row shared expert too: empty tile list
    (300, 512, 384, 8, 3, 0),    # tiles without a shared expert
    (200, 256, 512, 16, 2, 1),   # the shared expert's 200 rows in one tile
    (600, 256, 256, 32, 8, 1),   # 4800 pairs: the chunked permutation, separate binary16 rows and plan
    (2000, 256, 256, 8, 4, 1),   # ~1000 rows per expert + 2000 shared rows: 32 or more row tiles, dealt to
                                 # the XCDs in blocks of 4 consecutive tiles (one group's, and straddling)
], ids=["no_shared", "long_down_rows", "h_8192", "tile_ragged", "odd_blocks", "tile_steady",
        "small_beside_tiles", "empty_tile_list", "tile_no_shared", "shared_tile", "many_pairs", "block_dealing"])
def test_fp8_small_every_token(T, H, I, E, K, shared):
    _torch()
    w = wl.custom(f"fp8_{T}", T, H, I, E, K, x_seed=41, w_seed=42, n_shared=shared, quant="fp8")
    _check(w, wl.device_inputs(w))


def test_fp8_tiles_under_concurrent_memory_traffic():
    # the tile kernels' loads land late when other work loads HBM: each call runs while a torch stream
    # copies 1 GiB buffers concurrently, and every call must match the oracle (a K step reads every
    # weight row of its K block, so the whole block has to have landed, not only part of its rows)
    torch = _torch()
    w = wl.custom("fp8_traffic", 256, 1024, 768, 32, 4, x_seed=41, w_seed=42, quant="fp8")
    t = wl.device_inputs(w)
    big = torch.empty(256 << 20, dtype=torch.float32, device="cuda")
    big2 = torch.empty_like(big)
    side = torch.cuda.Stream()
    cfg = moe.config_for(w)
    y_ref = None
    for rep in range(3):
        ws = moe.alloc_workspace(cfg, moe.MOE_OP_FORWARD_FP8, w.T)
        ws.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(12):
                big2.copy_(big)
        y, ids, wts = moe.moe_forward_fp8(cfg, t["x"], t["w_router"], {k: t[k] for k in moe.QUANT_KEYS},
                                          t["ws_gate"], t["ws_up"], t["ws_down"], return_routing=True, workspace=ws)
        torch.cuda.synchronize()
        if y_ref is None:
            tokens = np.arange(w.T)
            y_ref, ids_ref, w_ref, gap = oracle_forward_tokens(w, tokens, ids_gpu=to_np(ids))
            check_routing(to_np(ids), to_np(wts), ids_ref, w_ref, gap)
        err = rel_l2(to_np(y), y_ref)
        print(f"fp8 under traffic, call {rep}: max rel L2 {err.max():.3g}", flush=True)
        assert err.max() <= Y_TOL["bf16"]
    del big, big2


def test_fp8_stream_skewed_passes():
    # at most 4 rows per group on average (stream kernels only), hot experts of up to 32 rows: two
    # 16-row passes
    _torch()
    w = wl.custom("fp8_stream_skew", 32, 512, 256, 40, 4, x_seed=49, w_seed=50, routing="skew", quant="fp8")
    _check(w, wl.device_inputs(w))


def test_fp8_skewed_routing_with_bias():
    # Zipf-shaped logit offsets (a few experts with many rows, many with one or two) and a score bias
    # that enters the selection only
    _torch()
    w = wl.custom("fp8_skew", 200, 512, 256, 32, 4, x_seed=46, w_seed=47, routing="skew", quant="fp8")
    bias = (np.random.default_rng(48).standard_normal(w.E) * 0.1).astype(np.float32)
    _check(w, wl.device_inputs(w), bias=bias)


def test_fp8_single_token():
    _torch()
    w = wl.custom("fp8_one", 1, 512, 256, 16, 8, x_seed=43, w_seed=44, quant="fp8")
    _check(w, wl.device_inputs(w))


def test_device_fp8_quantizer_matches_host():
    torch = _torch()
    n_mats, rows, cols = 2, 256, 384
    bits = synth.host_tensor(45, 2, 0, (n_mats * rows, cols), 1.0 / np.sqrt(cols), "bf16").copy()
    # blocks with special content: all zero; one large value over tiny ones (E4M3 subnormal codes);
    # a constant negative block (every code at -448); a value between two codes
    bits[0:128, 0:128] = 0
    bits[0:128, 128:256] = 0x3380          # 2^-24 ...
    bits[5, 130] = 0x4300                  # ... and one 128.0
    bits[128:256, 0:128] = 0xC000          # -2.0
    bits[256:384, 256:384] = 0x3F90        # 1.125: s = 1.125 / 448, every code 448 ...
    bits[260, 300] = 0x3F80                # ... and 1.0 = 398.2 s, between the codes 384 and 416
    w = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16).view(n_mats, rows, cols)
    codes = torch.empty((n_mats, rows, cols), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n_mats, rows // 128, cols // 128), dtype=torch.float32, device="cuda")
    synth.device_quantize_fp8(w, codes, scales)
    torch.cuda.synchronize()
    for m in range(n_mats):
        c_ref, s_ref = synth.host_quantize_fp8(bits[m * rows:(m + 1) * rows])
        np.testing.assert_array_equal(codes[m].cpu().numpy(), c_ref)
        np.testing.assert_array_equal(scales[m].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    c0 = codes[0].cpu().numpy()
    assert (c0[0:128, 0:128] == 0).all()
    assert set(np.unique(c0[0:128, 128:256] & 0x7F).tolist()) <= {0, 0x7E}  # 2^-24 / s rounds to zero


def test_fp8_rejects_f32_and_unsupported_sizes():
    torch = _torch()
    wr = torch.zeros((8, 384), dtype=torch.bfloat16, device="cuda")
    q = {k: torch.zeros(4, dtype=torch.uint8 if k.endswith("codes") else torch.float32, device="cuda")
         for k in moe.QUANT_KEYS}
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for H, I, dtype in ((384, 192, "bf16"), (8320, 256, "bf16"), (256, 8320, "bf16"), (512, 256, "f32")):
        cfg = moe.make_config(H, I, 8, 2, 0, dtype=dtype)
        x = torch.zeros((4, H), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(moe.MoeError) as e:
            moe.moe_forward_fp8(cfg, x, wr, q, workspace=ws)
        assert e.value.status == moe.MOE_ERR_UNSUPPORTED


PREFILL_SAMPLE = 256  # seeded prefill tokens whose outputs are compared


@pytest.mark.timeout(1200)
def test_fp8_full_size():
    """decode_fp8 (every token) and prefill_fp8 (routing of every token, outputs of a seeded sample:
    every expert, groups of ~170 rows on the tile kernels) at the full shape, one weight set, each in
    the benchmark's launch configuration (one moe_forward_fp8 call)."""
    torch = _torch()
    wd, wp = wl.WORKLOADS["decode_fp8"], wl.WORKLOADS["prefill_fp8"]
    t = wl.device_weights(wd)
    runs = {}
    for w in (wd, wp):
        print(f"running {w.name} (T={w.T}) on the GPU", flush=True)
        tw = dict(t, **wl.device_activations(w))
        y, ids, wts = moe.moe_forward_fp8(moe.config_for(w), tw["x"], tw["w_router"], {k: tw[k] for k in moe.QUANT_KEYS},
                                          tw.get("ws_gate"), tw.get("ws_up"), tw.get("ws_down"), return_routing=True)
        torch.cuda.synchronize()
        runs[w.name] = (to_np(y), to_np(ids), to_np(wts))
        del tw, y, ids, wts
    del t
    torch.cuda.empty_cache()
    # routing of every prefill token
    _, ids_p, wts_p = runs[wp.name]
    x, ids_ref, w_ref, gap, _ = oracle_route(wp, np.arange(wp.T))
    check_routing(ids_p, wts_p, ids_ref, w_ref, gap)
    rng = np.random.default_rng(20261204)
    sample = np.sort(rng.choice(wp.T, PREFILL_SAMPLE, replace=False))
    cases = [(wd, np.arange(wd.T), runs[wd.name][1]), (wp, sample, ids_p[sample])]
    refs = oracle_outputs_shared_weights(cases)
    for (w, tokens, ids_g), (y_ref, ids_r, w_r, gap_r) in zip(cases, refs):
        y_g, _, w_g = runs[w.name]
        check_routing(ids_g, w_g[tokens], ids_r, w_r, gap_r)
        err = rel_l2(y_g[tokens], y_ref)
        print(f"{w.name}: outputs of {len(tokens)} tokens checked, max rel L2 {err.max():.3g}, "
              f"p99 {np.percentile(err, 99):.3g}", flush=True)
        assert np.isfinite(y_g).all()
        assert err.max() <= Y_TOL["bf16"]
