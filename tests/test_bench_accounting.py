"""Host logic of the benchmark's roofline accounting (no GPU).

``bench.plan_families`` mirrors the library's kernel choice (moe_api.cpp) and the device plan's split
of the groups between the weight-stream and the tile kernels; ``bench.kernel_work`` charges each
grouped-GEMM launch the algorithmic bytes and flops of the groups its family takes.  A roofline
fraction is only evidence if every group lands in exactly one family and every group's weights are
charged once, in their storage format, to that family alone: these tests check both on the shapes of
every benchmarked workload, with synthetic routings of the same shape (uniform for the router
workloads, Zipf-skewed for skew, the workload's own pre-assigned ids for the EP share).
"""
import importlib.util
import os

import numpy as np
import pytest

from moe_layer_forward_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _ids(w, seed=5):
    """[T, K] distinct expert ids per token: uniform for a router workload, Zipf(1.1) popularity for skew."""
    rng = np.random.default_rng(seed)
    if w.routing == "preassigned":
        return wl.preassigned(w)[0]
    if w.routing == "dense":
        return None
    logp = np.zeros(w.E) if w.routing == "router" else -1.1 * np.log(1.0 + rng.permutation(w.E))
    keys = logp[None, :] + rng.gumbel(size=(w.T, w.E))  # Gumbel top-K: K distinct draws from p
    return np.argsort(-keys, axis=1)[:, :w.K].astype(np.int32)


def _rows_of(w, ids):
    if w.routing == "dense":
        return {0: w.T}
    rows = {e: int(c) for e, c in enumerate(np.bincount(ids.ravel(), minlength=w.E)) if c}
    if w.n_shared:
        rows[w.E] = w.T
    return rows


def _gemm_kernels(w, fam):
    q = {"int4": "q4", "fp8": "fp8"}.get(w.quant)
    if fam == "stream":
        return ("gateup_stream", "down_stream") if q is None else (f"gateup_{q}", f"down_{q}")
    if fam == "tile":
        return ("gateup_tile", "down_tile") if q is None else (f"gateup_tile_{q}", f"down_tile_{q}")
    return ("gateup_skinny", "down_skinny")


BENCHED = ["decode", "prefill", "skew", "ep_share", "dense_decode", "dense_prefill", "decode_int4", "decode_fp8",
           "prefill_fp8", "prefill_int4"]


@pytest.mark.parametrize("name", BENCHED)
def test_families_partition_the_groups(name):
    w = wl.WORKLOADS[name]
    ids = _ids(w)
    rows = _rows_of(w, ids)
    fams = bench.plan_families(w, ids)
    seen = [g[0] for groups in fams.values() for g in groups]
    assert sorted(seen) == sorted(rows), "every touched group (and the shared one) in exactly one family"
    for groups in fams.values():
        for g, r, toks in groups:
            assert r == rows[g]
            if toks is not None:  # a routed group reads the rows of the tokens routed to it
                assert set(toks.tolist()) == set(np.nonzero((ids == g).any(axis=1))[0].tolist())
    expect = {"decode": "stream", "decode_int4": "stream", "decode_fp8": "stream", "dense_decode": "skinny",
              "dense_prefill": "tile", "ep_share": "tile", "prefill": "tile", "prefill_fp8": "tile",
              "prefill_int4": "tile"}
    if name in expect:
        assert len(fams[expect[name]]) == len(rows), f"{name}: every group on the {expect[name]} kernels"
    else:  # skew: at least 16 groups, so the groups of at most 32 rows stream and the others tile
        assert {g[0] for g in fams["stream"]} == {g for g, r in rows.items() if r <= bench.STREAM_ROWS}
        assert {g[0] for g in fams["tile"]} == {g for g, r in rows.items() if r > bench.STREAM_ROWS}
        assert fams["stream"] and fams["tile"]


@pytest.mark.parametrize("name", BENCHED)
def test_each_groups_weights_charged_once(name):
    w = wl.WORKLOADS[name]
    ids = _ids(w)
    rows = _rows_of(w, ids)
    fams = bench.plan_families(w, ids)
    n_touched = len(rows) - (w.n_shared if w.routing != "dense" else 0)
    qb = bench.QUANT_BYTES.get(w.quant)
    eb = 2 if w.dtype == "bf16" else 4
    routed_b = qb if qb is not None else eb
    if w.routing == "dense":
        weights = eb * 3 * w.H * w.I
    else:
        weights = (n_touched * routed_b + w.n_shared * eb) * 3 * w.H * w.I
    total_rows = sum(rows.values())
    kb_sum, kf_sum = 0.0, 0.0
    for fam, groups in fams.items():
        if not groups:
            continue
        for kname in _gemm_kernels(w, fam):
            kb, kf = bench.kernel_work(kname, w, fams, n_touched)
            assert kb is not None and kf is not None, f"{kname} is charged nothing"
            kb_sum += kb
            kf_sum += kf
    # flops: every row through gate/up (4 H I) and down (2 H I) exactly once
    assert kf_sum == pytest.approx(total_rows * 6 * w.H * w.I, rel=1e-12)
    # bytes: the weights once, plus, per family, the token rows its groups read once (bf16 x, or for
    # quantized experts the routed groups' binary16 rows and the shared group's bf16 rows), the h rows
    # gate/up writes and down reads, and the y rows down writes
    row_bytes = 0
    for fam, groups in fams.items():
        if not groups:
            continue
        fam_rows = sum(g[1] for g in groups)
        every = any(g[2] is None for g in groups)
        routed = [g[2] for g in groups if g[2] is not None]
        toks = len(np.unique(np.concatenate(routed))) if routed else 0
        if qb is None:
            x_bytes = (w.T if every else toks) * w.H * eb
        else:
            x_bytes = toks * w.H * 2 + (w.T * w.H * 2 if every else 0)
        row_bytes += x_bytes + fam_rows * w.I * eb + fam_rows * (w.I + w.H) * eb
    assert kb_sum == pytest.approx(weights + row_bytes, rel=1e-12)
