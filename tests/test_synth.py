"""The seeded input generator: known answers, statistics, host/device agreement."""
import math
import os

import numpy as np
import pytest

from moe_layer_forward_amd import synth
from moe_layer_forward_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                v = [int(t, 16) for t in line.split()]
                rows.append((v[:4], v[4:6], v[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,out", _kat())
def test_philox_known_answers(ctr, key, out):
    assert synth.philox4x32_10(ctr, key).tolist() == out


def test_statistics_match_requested_sigma():
    for sigma in (1.0, 0.02, 1.0 / math.sqrt(7168)):
        a = synth.host_tensor(7, 3, 5, (400_000,), sigma, "f32").astype(np.float64)
        assert abs(a.mean()) < 0.01 * sigma
        assert a.std() == pytest.approx(sigma, rel=0.01)
        assert np.abs(a).max() <= 4.9 * sigma + 1e-12
        # Irwin-Hall(8) excess kurtosis is -1.2/8 = -0.15
        z = a / a.std()
        assert (z**4).mean() - 3.0 == pytest.approx(-0.15, abs=0.03)


def test_rows_and_offsets_agree_with_whole_tensor():
    full = synth.host_tensor(3, 2, 9, (20, 33), 0.5, "bf16")
    rows = synth.host_rows(3, 2, 9, 33, [4, 0, 19], 0.5, "bf16")
    np.testing.assert_array_equal(rows, full[[4, 0, 19]])
    tail = synth.host_tensor(3, 2, 9, (100,), 0.5, "bf16", elem0=20 * 33 - 100)
    np.testing.assert_array_equal(tail, full.reshape(-1)[-100:])
    other = synth.host_tensor(3, 2, 10, (20, 33), 0.5, "bf16")
    assert not np.array_equal(other, full)


def test_bf16_rounding_is_nearest_even():
    import torch

    f = synth.host_tensor(1, 1, 1, (100_000,), 3.0, "f32")
    b = synth.host_tensor(1, 1, 1, (100_000,), 3.0, "bf16")
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_workload_offsets_and_preassigned():
    off = wl.logit_offsets(wl.WORKLOADS["skew"])
    assert off.shape == (384,) and off.dtype == np.float32
    np.testing.assert_allclose(np.sort(np.exp(-off.astype(np.float64) / 1.1)), np.arange(1, 385), rtol=1e-5)
    ids, wts = wl.preassigned(wl.WORKLOADS["ep_share"])
    assert ids.shape == (16384, 1) and set(np.unique(ids).tolist()) == {0, 1, 2}
    assert wts.min() >= 0.05 * 2.827 * (1 - 1e-6) and wts.max() <= 0.6 * 2.827 * (1 + 1e-6)


@pytest.mark.gpu
def test_device_generator_matches_host():
    import torch

    w = wl.custom("gen", T=40, H=320, I=192, E=5, K=2)
    t = wl.device_inputs(w)
    torch.cuda.synchronize()
    xb = t["x"].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(xb, synth.host_tensor(w.x_seed, wl.S_X, 0, (w.T, w.H), 1.0, "bf16"))
    for e in (0, 3, 4):
        g, u, d = (t[k][e].view(torch.int16).cpu().numpy().view(np.uint16) for k in ("w_gate", "w_up", "w_down"))
        np.testing.assert_array_equal(g, synth.host_tensor(w.w_seed, wl.S_GATE, e, (w.I, w.H), w.sigma_gate_up, "bf16"))
        np.testing.assert_array_equal(u, synth.host_tensor(w.w_seed, wl.S_UP, e, (w.I, w.H), w.sigma_gate_up, "bf16"))
        np.testing.assert_array_equal(d, synth.host_tensor(w.w_seed, wl.S_DOWN, e, (w.H, w.I), w.sigma_down, "bf16"))
    tf = wl.device_inputs(wl.WORKLOADS["tiny"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(tf["w_router"].cpu().numpy(),
                                  synth.host_tensor(1, wl.S_ROUTER, 0, (16, 256), 0.02, "f32"))


def test_dense_workload_draws_its_own_weights():
    """The dense first-layer FFN uses its own weight streams, not routed expert 0's."""
    d = wl.custom("d", T=2, H=128, I=256, E=1, K=1, routing="dense", n_shared=0)
    m = wl.custom("m", T=2, H=128, I=256, E=1, K=1)
    for a, b in zip(wl.host_expert(d, 0), wl.host_expert(m, 0)):
        assert a.shape == b.shape and not np.array_equal(a, b)
    assert wl.WORKLOADS["dense_decode"].I == 18432 and wl.WORKLOADS["dense_prefill"].T == 8192
