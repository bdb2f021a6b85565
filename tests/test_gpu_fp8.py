"""Parity of the layer with FP8 routed experts (moe_forward_fp8, through the C ABI) with the CPU oracle.

The oracle evaluates the layer in float64 on the dequantized weights (E4M3 value times its 128 x 128
block scale, from the host quantizer's codes and scales); the GPU multiplies in binary16 with fp32
accumulation, so the bf16 output bar (per-row relative L2 <= 2e-2) applies.  Cases: small sizes on
every token (several 16-row passes per expert and a ragged tail; no shared expert; odd numbers of
128-blocks, where the down kernel runs one column block per work-group and the K loops end on
padded steps; a long W_down row whose scales do not fit the chained down kernel; hidden_size at
its 8192 limit; more than 4096 (token, expert) pairs), and the full decode shape on sampled tokens.
The two quantizers (device for the GPU inputs, host for the oracle) are checked bit-exact against
each other.
"""
import numpy as np
import pytest

import moe_layer_forward_amd as moe
from moe_layer_forward_amd import synth
from moe_layer_forward_amd import workloads as wl

from parity import Y_TOL, check_routing, oracle_forward_tokens, oracle_route, rel_l2, to_np

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
    (70, 512, 256, 8, 2, 1),     # ~17.5 rows per expert: two 16-row passes, ragged
    (5, 768, 512, 40, 4, 0),     # one or two rows per expert, no shared expert; chained down blocks
    (40, 384, 640, 12, 3, 1),    # 3 x 5 blocks: one down column block per work-group, padded K steps
    (8, 256, 4608, 8, 2, 1),     # W_down rows of 36 blocks: scales too many for the chained down kernel
    (6, 8192, 256, 8, 2, 1),     # hidden_size 8192: 64 gate/up scale blocks per row, one per lane
    (200, 256, 512, 16, 2, 1),   # the shared expert's 200 rows in seven 32-row passes
    (600, 256, 256, 32, 8, 1),   # 4800 pairs: the chunked permutation, separate binary16 rows and plan
], ids=["passes", "no_shared", "odd_blocks", "long_down_rows", "h_8192", "shared_passes", "many_pairs"])
def test_fp8_small_every_token(T, H, I, E, K, shared):
    _torch()
    w = wl.custom(f"fp8_{T}", T, H, I, E, K, x_seed=41, w_seed=42, n_shared=shared, quant="fp8")
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


def test_decode_fp8_full_size():
    torch = _torch()
    w = wl.WORKLOADS["decode_fp8"]
    t = wl.device_inputs(w)
    torch.cuda.synchronize()
    y, ids, wts = _check(w, t, tokens=[0, 17, 38, 63])
    x, ids_ref, w_ref, gap, _ = oracle_route(w, np.arange(w.T))
    check_routing(to_np(ids), to_np(wts), ids_ref, w_ref, gap)
    del t
    torch.cuda.empty_cache()
