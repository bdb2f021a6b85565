"""Parity of the layer with 4-bit routed experts (moe_forward_q4, through the C ABI) with the CPU oracle.

The oracle evaluates the layer in float64 on the dequantized weights (q * s of the host quantizer's
codes and scales); the GPU multiplies in binary16 with fp32 accumulation, so the bf16 output bar
(per-row relative L2 <= 2e-2) applies.  Cases: small sizes on every token (several 16-row passes
per expert and a ragged tail; no shared expert; the shared expert over many row passes; more than
4096 (token, expert) pairs, where the permutation runs as chunked kernels), and the
full decode shape on sampled tokens.  The two quantizers (device for the GPU inputs, host for the
oracle) are checked bit-exact against each other.
"""
import numpy as np
import pytest

import moe_layer_forward_amd as moe
from moe_layer_forward_amd import synth
from moe_layer_forward_amd import workloads as wl

from parity import Y_TOL, check_routing, oracle_forward_tokens, oracle_route, rel_l2, to_np

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
    (70, 512, 256, 8, 2, 1),     # ~17.5 rows per expert: two passes, ragged
    (5, 768, 512, 40, 4, 0),     # one or two rows per expert, no shared expert
    (200, 256, 512, 16, 2, 1),   # the shared expert's 200 rows in seven 32-row passes
    (600, 256, 256, 32, 8, 1),   # 4800 pairs: the chunked permutation, separate binary16 rows and plan
], ids=["passes", "no_shared", "shared_passes", "many_pairs"])
def test_q4_small_every_token(T, H, I, E, K, shared):
    _torch()
    w = wl.custom(f"q4_{T}", T, H, I, E, K, x_seed=31, w_seed=32, n_shared=shared, quant="int4")
    _check(w, wl.device_inputs(w))


def test_q4_single_token():
    _torch()
    w = wl.custom("q4_one", 1, 512, 256, 16, 8, x_seed=33, w_seed=34, quant="int4")
    _check(w, wl.device_inputs(w))


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


@pytest.mark.timeout(900)
def test_decode_int4_full_size():
    torch = _torch()
    w = wl.WORKLOADS["decode_int4"]
    t = wl.device_inputs(w)
    torch.cuda.synchronize()
    y, ids, wts = _check(w, t)  # every token
    x, ids_ref, w_ref, gap, _ = oracle_route(w, np.arange(w.T))
    check_routing(to_np(ids), to_np(wts), ids_ref, w_ref, gap)
    del t
    torch.cuda.empty_cache()
