"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Sizes the oracle finishes in seconds (several tiles and a ragged tail), then the full workload sizes
in the launch configuration the benchmark times, checked on sampled tokens plus properties that
hold at any size.  Edge cases: a single token, identical tokens, exact ties, one hot expert, no
shared expert, score bias, empty groups, poisoned unused experts, determinism.
"""
import numpy as np
import pytest

import moe_layer_forward_amd as moe
import oracle
from moe_layer_forward_amd import workloads as wl

from parity import (NEAR_TIE, W_TOL, Y_TOL, check_routing, near_tie_count, oracle_forward_preassigned,
                    oracle_forward_tokens, oracle_outputs_shared_weights, oracle_route, rel_l2, to_np)

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _forward(w, t, score_bias=None):
    cfg = moe.config_for(w)
    return moe.moe_forward(cfg, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], t.get("ws_gate"),
                           t.get("ws_up"), t.get("ws_down"), score_bias=score_bias,
                           logit_offset=t.get("logit_offset"), return_routing=True)


def _check_full(w, t, tokens=None, score_bias=None, bias_np=None):
    torch = _torch()
    y, ids, wts = _forward(w, t, score_bias)
    torch.cuda.synchronize()
    tokens = np.arange(w.T) if tokens is None else np.asarray(tokens)
    ids_g, w_g, y_g = to_np(ids)[tokens], to_np(wts)[tokens], to_np(y)[tokens]
    y_ref, ids_ref, w_ref, gap = oracle_forward_tokens(w, tokens, ids_gpu=ids_g, score_bias=bias_np)
    differ = check_routing(ids_g, w_g, ids_ref, w_ref, gap)
    err = rel_l2(y_g, y_ref)
    print(f"{w.name}: T={w.T} checked {len(tokens)} tokens, near-tie swaps {len(differ)}, "
          f"max rel L2 {err.max():.3g}, p99 {np.percentile(err, 99):.3g}", flush=True)
    assert err.max() <= Y_TOL[w.dtype]
    return y, ids, wts


# ----------------------------------------------------------------- small sizes, every token
def test_tiny_fp32_every_token():
    _torch()
    w = wl.WORKLOADS["tiny"]
    _check_full(w, wl.device_inputs(w))


@pytest.mark.parametrize("T", [20, 300], ids=["stream_kernels", "tile_kernels"])
def test_small_bf16_every_token(T):
    _torch()
    w = wl.custom("small", T=T, H=512, I=256, E=40, K=4)
    _check_full(w, wl.device_inputs(w))


def test_mixed_group_sizes_every_token():
    # skewed routing: groups of a few rows (weight-stream kernels) beside groups of hundreds of rows
    # (tile kernels) in the same layer call; few row tiles, so the down GEMM splits K and its
    # reduction must leave the stream kernels' rows alone
    _torch()
    w = wl.custom("mixed", T=512, H=512, I=512, E=48, K=4, routing="skew")
    y, ids, _ = _check_full(w, wl.device_inputs(w))
    counts = np.bincount(to_np(ids).ravel(), minlength=w.E)
    assert ((counts > 0) & (counts <= 32)).sum() >= 5 and (counts > 32).sum() >= 5, counts


def test_single_token_and_no_shared_expert():
    _torch()
    w = wl.custom("one", T=1, H=256, I=128, E=16, K=3)
    _check_full(w, wl.device_inputs(w))
    w0 = wl.custom("noshared", T=50, H=256, I=256, E=12, K=2, n_shared=0)
    _check_full(w0, wl.device_inputs(w0))


def test_score_bias_selects_only():
    torch = _torch()
    w = wl.custom("bias", T=64, H=384, I=128, E=24, K=4)
    bias = (np.random.default_rng(5).standard_normal(w.E) * 0.2).astype(np.float32)
    t = wl.device_inputs(w)
    _check_full(w, t, score_bias=torch.from_numpy(bias).cuda(), bias_np=bias)


# ----------------------------------------------------------------- full sizes (shared weight set)
@pytest.fixture(scope="module")
def k2_weights():
    torch = _torch()
    t = wl.device_weights(wl.WORKLOADS["decode"])
    torch.cuda.synchronize()
    yield t
    del t
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def k2_runs(k2_weights):
    """The layer at the decode, prefill and skew workloads (full size, the benchmark's launch
    configuration: one moe_forward call each), as host arrays (y, ids, weights)."""
    torch = _torch()
    out = {}
    for name in ("decode", "prefill", "skew"):
        w = wl.WORKLOADS[name]
        print(f"running {name} (T={w.T}) on the GPU", flush=True)
        t = dict(k2_weights, **wl.device_activations(w))
        y, ids, wts = _forward(w, t)
        torch.cuda.synchronize()
        out[name] = (to_np(y), to_np(ids), to_np(wts))
        del t, y, ids, wts
    return out


OUTPUT_SAMPLE = 512  # seeded token sample whose outputs are compared at prefill and skew


@pytest.mark.timeout(900)
def test_full_size_routing_every_token(k2_runs):
    """Routing of every token at decode (64), prefill (8192) and skew (4096) against oracle.route:
    ids exact outside oracle near-ties (counted), weights within 1e-5."""
    for name in ("decode", "prefill", "skew"):
        w = wl.WORKLOADS[name]
        y, ids, wts = k2_runs[name]
        _full_routing_properties(w, ids, wts)
        x, ids_ref, w_ref, gap, _ = oracle_route(w, np.arange(w.T))
        differ = check_routing(ids, wts, ids_ref, w_ref, gap)
        counts = np.bincount(ids.ravel(), minlength=w.E)
        print(f"{name}: routing of all {w.T} tokens checked; oracle near-ties {near_tie_count(gap)}, "
              f"id sets that differ (all near-ties) {len(differ)}; rows per expert max {counts.max()}, "
              f"touched {(counts > 0).sum()}", flush=True)
        assert np.isfinite(y).all()
        if name == "skew":
            print(f"skew histogram: max {counts.max()} ({counts.max() / counts.mean():.1f}x mean), "
                  f"experts with <= 2 tokens: {(counts <= 2).sum()}, untouched: {(counts == 0).sum()}",
                  flush=True)
            assert counts.max() > 10 * counts.mean()


@pytest.mark.timeout(900)
def test_full_size_outputs(k2_runs):
    """Outputs against the oracle: every decode token, and a seeded 512-token sample of prefill and
    of skew (all their experts: ~385 groups, hot experts of several row tiles), in one oracle pass."""
    rng = np.random.default_rng(20261203)
    cases = []
    for name in ("decode", "prefill", "skew"):
        w = wl.WORKLOADS[name]
        tokens = np.arange(w.T) if w.T <= OUTPUT_SAMPLE else np.sort(rng.choice(w.T, OUTPUT_SAMPLE, replace=False))
        cases.append((w, tokens, k2_runs[name][1][tokens]))
    refs = oracle_outputs_shared_weights(cases)
    for (w, tokens, ids_g), (y_ref, ids_ref, w_ref, gap) in zip(cases, refs):
        y_g, _, w_g = k2_runs[w.name]
        check_routing(ids_g, w_g[tokens], ids_ref, w_ref, gap)
        err = rel_l2(y_g[tokens], y_ref)
        print(f"{w.name}: outputs of {len(tokens)} tokens checked, max rel L2 {err.max():.3g}, "
              f"p99 {np.percentile(err, 99):.3g}", flush=True)
        assert err.max() <= Y_TOL["bf16"]


def _full_routing_properties(w, ids_n, w_n):
    assert ids_n.min() >= 0 and ids_n.max() < w.E
    s = np.sort(ids_n, axis=1)
    assert np.all(s[:, 1:] != s[:, :-1]), "duplicate expert in a token's top-K"
    np.testing.assert_allclose(w_n.sum(axis=1), w.rsf, atol=2e-6 * w.K)
    assert np.all(w_n > 0)


@pytest.mark.timeout(600)
def test_ep_share_full_size(k2_weights):
    torch = _torch()
    w = wl.WORKLOADS["ep_share"]
    a = wl.device_activations(w)
    cfg = moe.config_for(w)
    y = moe.moe_forward_routed(cfg, a["x"], a["topk_ids"], a["topk_weights"], k2_weights["w_gate"][:3],
                               k2_weights["w_up"][:3], k2_weights["w_down"][:3], k2_weights["ws_gate"],
                               k2_weights["ws_up"], k2_weights["ws_down"])
    torch.cuda.synchronize()
    tokens = np.sort(np.random.default_rng(5).choice(w.T, OUTPUT_SAMPLE, replace=False))
    y_ref = oracle_forward_preassigned(w, tokens)
    err = rel_l2(to_np(y)[tokens], y_ref)
    print(f"ep_share: outputs of {len(tokens)} rows checked, max rel L2 {err.max():.3g}, "
          f"p99 {np.percentile(err, 99):.3g}", flush=True)
    assert err.max() <= Y_TOL["bf16"]
    assert np.isfinite(to_np(y)).all()


# ----------------------------------------------------------------- the dense first-layer FFN
def _dense(w, t):
    """The dense SwiGLU FFN on the grouped kernels: one group of all T rows, weight 1."""
    torch = _torch()
    offs = torch.tensor([0, w.T], dtype=torch.int32, device="cuda")
    y = moe.moe_grouped_swiglu(moe.config_for(w), offs, w.T, t["x"], t["w_gate"], t["w_up"], t["w_down"],
                               y_dtype=moe.MOE_BF16)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T", [3, 17, 40, 64, 200],
                         ids=["stream_kernels", "skinny_2_blocks", "skinny_ragged", "skinny_64_rows", "tile_kernels"])
def test_dense_ffn_every_token(T):
    _torch()
    w = wl.custom("dense_small", T=T, H=512, I=1152, E=1, K=1, routing="dense", n_shared=0)
    t = wl.device_inputs(w)
    y = _dense(w, t)
    err = rel_l2(to_np(y), oracle.swiglu_expert(wl.host_x(w), *wl.host_expert(w, 0)))
    print(f"dense T={T}: max rel L2 {err.max():.3g}", flush=True)
    assert err.max() <= Y_TOL["bf16"]


@pytest.mark.parametrize("T,H,I", [(16, 2048, 4096), (100, 2048, 4096), (300, 4096, 1024)],
                         ids=["skinny", "one_tile", "two_tiles"])
def test_dense_ffn_split_k_every_token(T, H, I):
    """Few rows and a wide layer: the down GEMM splits K into ranges of fp32 partial sums, reduced in
    K-range order (skinny: at most 64 rows, K ranges of the skinny kernels, W_down rows 8 KiB apart so
    the work-groups start at different K steps; one_tile: 16 ranges of the tile kernels; two_tiles, the
    second one ragged: the layer too narrow to split); every token against the oracle."""
    _torch()
    w = wl.custom("dense_split", T=T, H=H, I=I, E=1, K=1, routing="dense", n_shared=0)
    # the workspace holds the K-range partial sums only when K is split: at least 2 ranges of
    # T rows x H fp32 beside h and the plan
    ws = moe.moe_workspace_size(moe.config_for(w), moe.MOE_OP_GROUPED_SWIGLU, w.T, 1)
    if T <= 100:
        assert ws >= 2 * w.T * w.H * 4 + w.T * w.I * 2
    t = wl.device_inputs(w)
    y = _dense(w, t)
    err = rel_l2(to_np(y), oracle.swiglu_expert(wl.host_x(w), *wl.host_expert(w, 0)))
    print(f"dense split-K T={w.T} H={w.H} I={w.I}: max rel L2 {err.max():.3g}", flush=True)
    assert err.max() <= Y_TOL["bf16"]
    # the K ranges are added in K-range order whichever work-group finishes last: bit-identical reruns
    for _ in range(3):
        assert _torch().equal(_dense(w, t), y)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_tokens", [("dense_decode", 64), ("dense_prefill", 256)])
def test_dense_full_size(name, n_tokens):
    _torch()
    w = wl.WORKLOADS[name]
    tokens = np.arange(w.T) if n_tokens >= w.T else np.sort(np.random.default_rng(6).choice(w.T, n_tokens,
                                                                                           replace=False))
    t = wl.device_inputs(w)
    y = _dense(w, t)
    y_ref = oracle.swiglu_expert(wl.host_x_rows(w, tokens), *wl.host_expert(w, 0))
    err = rel_l2(to_np(y)[tokens], y_ref)
    print(f"{name}: T={w.T} checked {len(tokens)} tokens, max rel L2 {err.max():.3g}", flush=True)
    assert err.max() <= Y_TOL["bf16"]
    assert np.isfinite(to_np(y)).all()


# ----------------------------------------------------------------- the individual calls
def test_route_call():
    torch = _torch()
    w = wl.custom("route", T=200, H=1024, I=128, E=96, K=6)
    t = wl.device_inputs(w)
    ids, wts = moe.moe_route(moe.config_for(w), t["x"], t["w_router"])
    torch.cuda.synchronize()
    x, ids_ref, w_ref, gap, _ = oracle_route(w, np.arange(w.T))
    differ = check_routing(to_np(ids), to_np(wts), ids_ref, w_ref, gap)
    # order: key descending (scores descending without bias)
    s_ref = oracle.route(x, wl.host_router(w), w.K, w.rsf)[3]
    ids_n = to_np(ids)
    for tk in range(w.T):
        if tk in differ:
            continue
        ks = s_ref[tk, ids_n[tk]].astype(np.float32)
        assert np.all(ks[:-1] >= ks[1:])


def test_permute_call_integer_exact():
    torch = _torch()
    r = np.random.default_rng(3)
    # up to 4096 pairs the permutation runs as one work-group (16 waves), above as chunked kernels
    for T, K, E in [(1, 1, 1), (37, 3, 11), (5000, 8, 384), (700, 2, 7), (512, 8, 512), (513, 8, 384),
                    (4096, 1, 3)]:
        ids = np.stack([r.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
        cfg = moe.make_config(hidden_size=256, moe_intermediate_size=128, n_routed_experts=E, top_k=K)
        x = torch.randn((T, 256), dtype=torch.bfloat16, device="cuda")
        off, row_token, pair_row, x_perm = moe.moe_permute(cfg, torch.from_numpy(ids).cuda(), x)
        torch.cuda.synchronize()
        o_off, o_rt, o_pr = oracle.permute(ids, E)
        np.testing.assert_array_equal(to_np(off), o_off)
        np.testing.assert_array_equal(to_np(row_token), o_rt)
        np.testing.assert_array_equal(to_np(pair_row), o_pr)
        assert torch.equal(x_perm, x[row_token.long()])


@pytest.mark.parametrize("y_bf16", [False, True])
@pytest.mark.parametrize("sizes", [[30, 0, 55, 0, 95], [3, 0, 5, 1, 0], [16, 0, 17, 0, 31], [1, 0, 63],
                                   [2, 40, 0, 7, 300, 1, 33, 32, 0, 5, 17, 64, 3, 0, 9, 120, 1, 31, 0, 2, 8, 0, 50, 4],
                                   [2100, 0, 1500, 1100, 800, 600, 400, 300, 260, 40, 20]],
                         ids=["tile_kernels", "stream_kernels", "skinny_kernels", "skinny_one_and_63",
                              "many_groups_both", "chunked_dealing"])
def test_grouped_swiglu_and_combine_calls(y_bf16, sizes):
    # skinny_*: at most 64 rows in all and more than 4 per group: the skinny kernels (16 / 17 / 31 rows:
    # one, two and two MFMA row blocks; empty groups between and at the end)
    # many_groups_both: 24 groups, so the groups of at most 32 rows go to the weight-stream kernels and
    # the others (33 .. 300 rows) to the tile kernels in the same call
    # chunked_dealing: 35 row tiles (groups of 1 to 9 tiles), so blocks of 4 consecutive tiles go to the
    # XCDs: blocks of one group's tiles (run slab by slab) beside blocks that straddle groups
    torch = _torch()
    w = wl.custom("gs", T=90, H=256, I=384, E=len(sizes), K=2)
    t = wl.device_inputs(w)
    # groups with 0 rows in the middle and at the end; rows gathered through row_index
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(off[-1])
    row_index = np.random.default_rng(1).integers(0, w.T, size=rows).astype(np.int32)
    scale = np.random.default_rng(2).uniform(0.5, 2.0, size=rows).astype(np.float32)
    cfg = moe.config_for(w)
    y_rows = moe.moe_grouped_swiglu(cfg, torch.from_numpy(off).cuda(), rows, t["x"], t["w_gate"], t["w_up"],
                                    t["w_down"], row_index=torch.from_numpy(row_index).cuda(),
                                    row_scale=torch.from_numpy(scale).cuda(),
                                    y_dtype=moe.MOE_BF16 if y_bf16 else moe.MOE_F32)
    torch.cuda.synchronize()
    x = wl.host_x(w)
    ref = np.zeros((rows, w.H))
    for g in range(len(sizes)):
        a, b = off[g], off[g + 1]
        if b > a:
            ref[a:b] = scale[a:b, None] * oracle.swiglu_expert(x[row_index[a:b]], *wl.host_expert(w, g))
    err = rel_l2(to_np(y_rows), ref)
    assert err.max() <= Y_TOL["bf16"]

    # combine: token t takes rows pair_row[t, :] with weights, plus a shared row block (rows 0..T-1)
    T, K = min(40, rows), 3
    r = np.random.default_rng(4)
    pair_row = np.stack([r.choice(rows, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    wts = r.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    y_sh = y_rows[:T].contiguous()
    ccfg = moe.make_config(hidden_size=w.H, moe_intermediate_size=w.I, n_routed_experts=w.E, top_k=K)
    y = moe.moe_combine(ccfg, y_rows, torch.from_numpy(pair_row).cuda(), torch.from_numpy(wts).cuda(), y_sh)
    torch.cuda.synchronize()
    y_ref = oracle.combine(to_np(y_rows), pair_row, wts, to_np(y_sh))
    assert rel_l2(to_np(y), y_ref).max() <= Y_TOL["bf16"]


# ----------------------------------------------------------------- edge cases and properties
def test_exact_ties_zero_router():
    torch = _torch()
    w = wl.custom("ties", T=64, H=256, I=128, E=16, K=4)
    t = wl.device_inputs(w)
    t["w_router"].zero_()
    y, ids, wts = _forward(w, t)
    torch.cuda.synchronize()
    assert (to_np(ids) == np.arange(4)[None, :]).all()
    np.testing.assert_allclose(to_np(wts), w.rsf / 4, rtol=1e-6)
    x = wl.host_x(w)
    y_ref = oracle.moe_forward_given_routing(x, np.tile(np.arange(4), (64, 1)), np.full((64, 4), w.rsf / 4),
                                             lambda e: wl.host_expert(w, e), wl.host_shared(w))
    assert rel_l2(to_np(y), y_ref).max() <= Y_TOL["bf16"]


def test_identical_tokens_and_one_hot_expert():
    torch = _torch()
    w = wl.custom("hot", T=256, H=256, I=128, E=32, K=2)
    t = wl.device_inputs(w)
    t["x"][:] = t["x"][0:1].clone()             # every token identical: one expert set takes all rows
    y, ids, wts = _forward(w, t)
    torch.cuda.synchronize()
    ids_n = to_np(ids)
    assert (ids_n == ids_n[0:1]).all()
    y_n = to_np(y)
    assert (y_n == y_n[0:1]).all()
    x0 = wl.host_x_rows(w, [0])
    ids_r, w_r, _, _ = oracle.route(x0, wl.host_router(w), w.K, w.rsf)
    y_ref = oracle.moe_forward_given_routing(x0, ids_r, w_r, lambda e: wl.host_expert(w, e), wl.host_shared(w))
    assert rel_l2(y_n[:1], y_ref).max() <= Y_TOL["bf16"]
    # one hot expert through a logit offset: expert 7 is in every token's set
    off = np.zeros(w.E, np.float32)
    off[7] = 30.0
    t2 = wl.device_inputs(w)
    y2, ids2, _ = moe.moe_forward(moe.config_for(w), t2["x"], t2["w_router"], t2["w_gate"], t2["w_up"],
                                  t2["w_down"], t2["ws_gate"], t2["ws_up"], t2["ws_down"],
                                  logit_offset=torch.from_numpy(off).cuda(), return_routing=True)
    torch.cuda.synchronize()
    assert (to_np(ids2)[:, 0] == 7).all()


@pytest.mark.parametrize("T,E,K", [(8, 40, 2), (300, 128, 1)], ids=["stream_kernels", "tile_kernels"])
def test_determinism_and_poison(T, E, K):
    torch = _torch()
    w = wl.custom("det", T=T, H=512, I=256, E=E, K=K)
    t = wl.device_inputs(w)
    y1, ids1, _ = _forward(w, t)
    y2, ids2, _ = _forward(w, t)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(ids1, ids2)
    used = set(to_np(ids1).ravel().tolist())
    unused = [e for e in range(w.E) if e not in used]
    if not unused:
        pytest.skip("every expert is used")
    for e in unused:
        t["w_gate"][e].fill_(float("nan"))
        t["w_down"][e].fill_(float("nan"))
    y3, _, _ = _forward(w, t)
    torch.cuda.synchronize()
    assert torch.equal(y1, y3)
