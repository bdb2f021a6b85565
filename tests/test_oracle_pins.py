"""Pins of the CPU oracle to facts fixed by the pages and by mathematics (no GPU).

Each test names the property it checks and why a plausible oracle mistake
would fail it:

* rational routing golden cases (sign of the sigmoid, the order of the
  top-K, tie-break, bias-for-selection-only, normalisation and scale);
* the weights of every token sum to 2.827 and the ids are K distinct experts;
* closed-form experts (diagonal / permutation matrices) pin SiLU on the gate
  (not the up) projection and the orientation of the down projection;
* W_router = 0 (all scores 1/2): ids 0..K-1, weights rsf/K, shared weight 1;
* a brute-force dense evaluation of every expert with a 0/weight mask, and a
  repeated-argmax top-K, against the sparse dispatch path;
* equivariance under token permutation and expert relabelling;
* poison (NaN) in unselected experts never reaches the output;
* the per-expert parameter count 3 x 7168 x 2048 = 44,040,192.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from moe_layer_forward_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RSF = 2.827


def _rng(seed):
    return np.random.default_rng(seed)


def _random_layer(seed, T=24, H=32, I=16, E=12, n_shared=1):
    r = _rng(seed)
    x = r.standard_normal((T, H))
    wr = r.standard_normal((E, H)) * 0.3
    experts = [(r.standard_normal((I, H)) / math.sqrt(H), r.standard_normal((I, H)) / math.sqrt(H),
                r.standard_normal((H, I)) / math.sqrt(I)) for _ in range(E)]
    shared = (r.standard_normal((I, H)) / math.sqrt(H), r.standard_normal((I, H)) / math.sqrt(H),
              r.standard_normal((H, I)) / math.sqrt(I)) if n_shared else None
    return x, wr, experts, shared


# ----------------------------------------------------------------- golden routing
def _load_rational_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "routing_rational.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
                cases.append(cur)
            elif key == "k":
                cur["k"] = int(vals[0])
            elif key in ("p", "w"):
                cur[key] = [Fraction(v) for v in vals]
            elif key == "bias":
                cur["bias"] = np.array([float(v) for v in vals], np.float32)
            elif key == "ids":
                cur["ids"] = [int(v) for v in vals]
    return cases


RATIONAL = _load_rational_cases()


@pytest.mark.parametrize("case", RATIONAL, ids=[c["name"] for c in RATIONAL])
@pytest.mark.parametrize("via", ["matmul", "offset"])
def test_rational_routing_golden(case, via):
    p = np.array([float(v) for v in case["p"]])
    logits = np.log(p / (1.0 - p))
    E = len(p)
    if via == "matmul":      # x = [1], W_router[:, 0] = logits
        x, wr, off = np.ones((1, 1)), logits[:, None], None
    else:                    # W_router = 0, the logits come in as offsets
        x, wr, off = np.ones((1, 3)), np.zeros((E, 3)), logits
    bias = case["bias"] if np.any(case["bias"] != 0) else None
    ids, w, gap, s = oracle.route(x, wr, case["k"], RSF, score_bias=bias, logit_offset=off)
    assert ids[0].tolist() == case["ids"]
    expected = np.array([RSF * float(v) for v in case["w"]])
    np.testing.assert_allclose(w[0], expected, rtol=1e-14, atol=0)
    np.testing.assert_allclose(s[0], p, rtol=1e-14)


# ----------------------------------------------------------------- invariants
@pytest.mark.parametrize("use_bias", [False, True])
def test_weights_sum_to_scale_and_ids_distinct(use_bias):
    x, wr, _, _ = _random_layer(1, T=200, H=48, E=384)
    bias = _rng(2).standard_normal(384).astype(np.float32) * 0.05 if use_bias else None
    ids, w, gap, s = oracle.route(x, wr, 8, RSF, score_bias=bias)
    assert ids.shape == (200, 8) and w.shape == (200, 8)
    np.testing.assert_allclose(w.sum(axis=1), RSF, rtol=0, atol=2e-6)
    for row in ids:
        assert len(set(row.tolist())) == 8
        assert row.min() >= 0 and row.max() < 384
    assert np.all(s > 0) and np.all(s < 1)
    assert np.all(w > 0)
    assert np.all(gap >= 0)


def test_selected_keys_dominate_unselected():
    x, wr, _, _ = _random_layer(3, T=50, H=20, E=40)
    ids, w, gap, s = oracle.route(x, wr, 5, RSF)
    key = s.astype(np.float32)
    for t in range(50):
        sel = set(ids[t].tolist())
        worst_sel = min(key[t, e] for e in sel)
        best_rest = max(key[t, e] for e in range(40) if e not in sel)
        assert worst_sel >= best_rest
        # listed in key-descending order
        assert all(key[t, ids[t, i]] >= key[t, ids[t, i + 1]] for i in range(4))


def test_topk_matches_repeated_argmax():
    """Selection by a full stable sort equals K rounds of 'take the largest key,
    smaller id on ties' written out in plain Python."""
    x, wr, _, _ = _random_layer(4, T=30, H=16, E=24)
    # force some exact ties
    wr[5] = wr[3]
    wr[17] = wr[3]
    ids, _, _, s = oracle.route(x, wr, 6, RSF)
    key = s.astype(np.float32)
    for t in range(30):
        remaining = list(range(24))
        picked = []
        for _ in range(6):
            best = remaining[0]
            for e in remaining[1:]:
                if key[t, e] > key[t, best]:
                    best = e
            picked.append(best)
            remaining.remove(best)
        assert ids[t].tolist() == picked


# ----------------------------------------------------------------- closed-form experts
def _diag_expert(a, b, c, H):
    return a * np.eye(H), b * np.eye(H), c * np.eye(H)


def _silu_scalar(z):
    return z / (1.0 + math.exp(-z))


def test_swiglu_closed_form_gate_up_down_orientation():
    """W_gate = a P1, W_up = b P2, W_down = P3 (permutation matrices, H = I = 5):
    y_i = sum_j P3[i, j] * SiLU(a (P1 x)_j) * b (P2 x)_j, evaluated element by element."""
    H = 5
    P1 = np.eye(H)[[1, 2, 3, 4, 0]]
    P2 = np.eye(H)[[4, 3, 2, 1, 0]]
    P3 = np.eye(H)[[2, 0, 4, 1, 3]]
    a, b = 0.7, -1.3
    x = np.array([[0.5, -1.0, 2.0, 0.25, -0.75], [1.5, 0.1, -0.2, -2.0, 0.9]])
    y = oracle.swiglu_expert(x, a * P1, b * P2, P3)
    for t in range(2):
        p1x = [x[t, int(np.argmax(P1[j]))] for j in range(H)]
        p2x = [x[t, int(np.argmax(P2[j]))] for j in range(H)]
        h = [_silu_scalar(a * p1x[j]) * b * p2x[j] for j in range(H)]
        expect = [h[int(np.argmax(P3[i]))] for i in range(H)]
        np.testing.assert_allclose(y[t], expect, rtol=1e-14, atol=1e-15)


def test_silu_known_values():
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4, sigmoid(0) = 1/2
    z = np.array([math.log(3.0), -math.log(3.0), 0.0])
    np.testing.assert_allclose(oracle.sigmoid(z), [0.75, 0.25, 0.5], rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(z), [0.75 * math.log(3.0), -0.25 * math.log(3.0), 0.0],
                               rtol=1e-15, atol=1e-300)


def test_zero_router_closed_form_layer():
    """W_router = 0: every score is 1/2, so the ids are 0..K-1 (ties -> smaller id),
    each weight is rsf/K, and the shared expert enters with weight 1."""
    H, E, K = 4, 6, 3
    coeff = [(0.5 + 0.1 * e, 1.0 - 0.2 * e, 0.3 + 0.05 * e) for e in range(E)]
    experts = [_diag_expert(*c, H) for c in coeff]
    sa, sb, sc = 0.9, 0.4, -1.1
    shared = _diag_expert(sa, sb, sc, H)
    x = np.array([[0.3, -0.6, 1.2, 2.0], [-1.0, 0.5, 0.0, 0.7]])
    y, ids, w, gap = oracle.moe_forward(x, np.zeros((E, H)), lambda e: experts[e], shared, K, RSF)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    np.testing.assert_allclose(w, RSF / K, rtol=1e-15)
    assert np.all(gap == 0)
    for t in range(2):
        for j in range(H):
            z = x[t, j]
            routed = sum((RSF / K) * coeff[e][2] * _silu_scalar(coeff[e][0] * z) * coeff[e][1] * z
                         for e in range(K))
            sh = sc * _silu_scalar(sa * z) * sb * z
            assert y[t, j] == pytest.approx(routed + sh, rel=1e-13, abs=1e-15)


def test_k_equals_e_selects_all():
    x, wr, experts, shared = _random_layer(5, T=10, E=7)
    ids, w, gap, s = oracle.route(x, wr, 7, RSF)
    for t in range(10):
        assert sorted(ids[t].tolist()) == list(range(7))
        np.testing.assert_allclose(w[t], RSF * s[t, ids[t]] / s[t].sum(), rtol=1e-14)
    assert np.all(np.isinf(gap))


def test_routed_part_linear_in_scale_and_shared_separate():
    x, wr, experts, shared = _random_layer(6)
    y1, *_ = oracle.moe_forward(x, wr, lambda e: experts[e], None, 4, 1.0)
    y2, *_ = oracle.moe_forward(x, wr, lambda e: experts[e], None, 4, RSF)
    np.testing.assert_allclose(y2, RSF * y1, rtol=1e-12, atol=1e-14)
    ys, *_ = oracle.moe_forward(x, wr, lambda e: experts[e], shared, 4, RSF)
    np.testing.assert_allclose(ys - y2, oracle.swiglu_expert(x, *shared), rtol=1e-10, atol=1e-12)
    zero_shared = tuple(np.zeros_like(m) for m in shared)
    yz, *_ = oracle.moe_forward(x, wr, lambda e: experts[e], zero_shared, 4, RSF)
    np.testing.assert_allclose(yz, y2, rtol=0, atol=1e-15)


def test_zero_down_removes_expert():
    x, wr, experts, shared = _random_layer(7)
    ids, w, _, _ = oracle.route(x, wr, 4, RSF)
    e0 = int(ids[0, 0])
    killed = list(experts)
    killed[e0] = (experts[e0][0], experts[e0][1], np.zeros_like(experts[e0][2]))
    y, *_ = oracle.moe_forward(x, wr, lambda e: experts[e], shared, 4, RSF)
    yk, *_ = oracle.moe_forward(x, wr, lambda e: killed[e], shared, 4, RSF)
    for t in range(x.shape[0]):
        k = np.nonzero(ids[t] == e0)[0]
        contrib = w[t, k[0]] * oracle.swiglu_expert(x[t:t + 1], *experts[e0])[0] if k.size else 0.0
        np.testing.assert_allclose(y[t] - yk[t], contrib, rtol=1e-9, atol=1e-12)


# ----------------------------------------------------------------- brute force
def test_dense_masked_bruteforce_on_tiny_workload():
    """Evaluate all 16 experts on all 64 tokens of the tiny workload, gate them
    with a dense [T, E] matrix (w if selected else 0) built from a repeated-
    argmax top-2, and compare with the sparse dispatch path."""
    w = wl.WORKLOADS["tiny"]
    x = wl.host_x(w)
    wr = wl.host_router(w)
    experts = [wl.host_expert(w, e) for e in range(w.E)]
    shared = wl.host_shared(w)
    y, ids, wts, gap = oracle.moe_forward(x, wr, lambda e: experts[e], shared, w.K, w.rsf)

    logits = np.array([[float(np.dot(x[t], wr[e])) for e in range(w.E)] for t in range(w.T)])
    scores = 1.0 / (1.0 + np.exp(-logits))
    key = scores.astype(np.float32)
    G = np.zeros((w.T, w.E))
    for t in range(w.T):
        chosen = []
        for _ in range(w.K):
            cand = [e for e in range(w.E) if e not in chosen]
            best = max(cand, key=lambda e: (key[t, e], -e))
            chosen.append(best)
        tot = sum(scores[t, e] for e in chosen)
        for e in chosen:
            G[t, e] = w.rsf * scores[t, e] / tot
    dense = np.zeros_like(y)
    for e in range(w.E):
        Fe = oracle.swiglu_expert(x, *experts[e])
        dense += G[:, e:e + 1] * Fe
    dense += oracle.swiglu_expert(x, *shared)
    np.testing.assert_allclose(y, dense, rtol=1e-10, atol=1e-12)
    rel = np.linalg.norm(y - dense, axis=1) / np.linalg.norm(dense, axis=1)
    assert rel.max() < 1e-12


def test_permute_bruteforce():
    r = _rng(9)
    T, K, E = 37, 3, 11
    ids = np.stack([r.choice(E, size=K, replace=False) for _ in range(T)])
    offsets, row_token, pair_row = oracle.permute(ids, E)
    rows = []
    for e in range(E):
        seg = [(t, k) for t in range(T) for k in range(K) if ids[t, k] == e]
        assert offsets[e + 1] - offsets[e] == len(seg)
        rows.extend(seg)
    assert offsets[0] == 0 and offsets[E] == T * K
    for rix, (t, k) in enumerate(rows):
        assert row_token[rix] == t
        assert pair_row[t, k] == rix


def test_combine_equals_loop():
    r = _rng(10)
    T, K, H = 9, 3, 5
    O = r.standard_normal((T * K + 2, H))
    pair_row = r.permutation(T * K).reshape(T, K)
    wts = r.random((T, K))
    sh = r.standard_normal((T, H))
    y = oracle.combine(O, pair_row, wts, sh)
    for t in range(T):
        expect = sh[t].copy()
        for k in range(K):
            expect += wts[t, k] * O[pair_row[t, k]]
        np.testing.assert_allclose(y[t], expect, rtol=1e-14)


@pytest.mark.parametrize("name", ["tiny", "noshared"])
def test_combine_of_permuted_expert_rows_is_the_layer(name):
    """[DEEP] §10.2 Steps 5-7 as the GPU path runs them: rows grouped per expert by
    ``oracle.permute``, each row through its expert's SwiGLU, then ``oracle.combine`` with the
    routing weights and the shared expert.  That must equal ``moe_forward_given_routing`` (which the
    dense masked brute force above pins), so a wrong row index, a transposed pair_row, weights
    applied by row instead of by pair, or a dropped shared term in ``combine`` fails here."""
    w = wl.WORKLOADS["tiny"] if name == "tiny" else wl.custom("noshared", T=40, H=64, I=32, E=10, K=3,
                                                              dtype="f32", n_shared=0)
    x = wl.host_x(w)
    experts = [wl.host_expert(w, e) for e in range(w.E)]
    shared = wl.host_shared(w)
    ids, wts, _, _ = oracle.route(x, wl.host_router(w), w.K, w.rsf)
    offsets, row_token, pair_row = oracle.permute(ids, w.E)
    rows = np.zeros((w.T * w.K, w.H))
    for e in range(w.E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            rows[a:b] = oracle.swiglu_expert(x[row_token[a:b]], *experts[e])
    shared_out = oracle.swiglu_expert(x, *shared) if shared is not None else None
    y = oracle.combine(rows, pair_row, wts, shared_out)
    y_ref = oracle.moe_forward_given_routing(x, ids, wts, lambda e: experts[e], shared)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-14)
    # the pairing is not trivially the identity: rows are really reordered
    assert not np.array_equal(pair_row.ravel(), np.arange(w.T * w.K))


# ----------------------------------------------------------------- equivariance and poison
def test_token_permutation_and_expert_relabelling():
    x, wr, experts, shared = _random_layer(11, T=20, E=10)
    y, ids, w, _ = oracle.moe_forward(x, wr, lambda e: experts[e], shared, 3, RSF)
    perm = _rng(12).permutation(20)
    yp, *_ = oracle.moe_forward(x[perm], wr, lambda e: experts[e], shared, 3, RSF)
    np.testing.assert_allclose(yp, y[perm], rtol=1e-12, atol=1e-14)
    lab = _rng(13).permutation(10)          # new id j is old expert lab[j]
    wr2 = wr[lab]
    yr, ids2, w2, _ = oracle.moe_forward(x, wr2, lambda j: experts[lab[j]], shared, 3, RSF)
    np.testing.assert_allclose(yr, y, rtol=1e-12, atol=1e-14)
    assert [sorted(lab[r].tolist()) for r in ids2] == [sorted(r.tolist()) for r in ids]


def test_poison_in_unselected_experts_does_not_leak():
    x, wr, experts, shared = _random_layer(14, T=6, E=16)
    ids, _, _, _ = oracle.route(x, wr, 2, RSF)
    used = set(ids.ravel().tolist())
    nan = np.full_like(experts[0][0], np.nan)
    poisoned = [experts[e] if e in used else (nan, nan, np.full_like(experts[0][2], np.nan)) for e in range(16)]
    y, *_ = oracle.moe_forward(x, wr, lambda e: experts[e], shared, 2, RSF)
    yp, *_ = oracle.moe_forward(x, wr, lambda e: poisoned[e], shared, 2, RSF)
    assert np.all(np.isfinite(yp))
    np.testing.assert_array_equal(yp, y)


# ----------------------------------------------------------------- sizes
def test_expert_parameter_count():
    assert oracle.expert_param_count(7168, 2048) == 44_040_192
    per_expert_bytes_bf16 = 2 * oracle.expert_param_count(7168, 2048)
    assert per_expert_bytes_bf16 == 88_080_384
    assert 385 * per_expert_bytes_bf16 == pytest.approx(33.91e9, rel=1e-3)
    w = wl.WORKLOADS["decode"]
    g, u, d = w.I * w.H, w.I * w.H, w.H * w.I
    assert g + u + d == oracle.expert_param_count(w.H, w.I)


def test_real_shape_slice_invariants():
    """Two tokens of the decode workload at the real shape (H=7168, I=2048, E=384)."""
    w = wl.WORKLOADS["decode"]
    x = wl.host_x_rows(w, [0, 1])
    wr = wl.host_router(w)
    ids, wts, gap, s = oracle.route(x, wr, w.K, w.rsf)
    np.testing.assert_allclose(wts.sum(axis=1), 2.827, atol=2e-6)
    assert all(len(set(r.tolist())) == 8 for r in ids)
    # logits have the std the recipe implies: 0.02 * sqrt(7168) ~ 1.69
    lg = oracle.router_logits(wl.host_x_rows(w, np.arange(8)), wr)
    assert 1.3 < lg.std() < 2.1


# ----------------------------------------------------------------- 4-bit routed experts
def _golden_q4():
    words, qs, scale_bits, scale = [], [], None, None
    with open(os.path.join(GOLDEN, "q4_dequant.txt")) as fh:
        for line in fh:
            f = line.split()
            if not f or f[0].startswith("#") or f[0] == "words":
                continue
            if f[0] == "scale":
                scale_bits, scale = int(f[1], 16), float(f[2])
            else:
                words.append(int(f[0], 16))
                qs.extend(int(v) for v in f[1:])
    return np.array([words], dtype=np.uint32), np.array(qs), scale_bits, scale


def test_q4_dequant_golden():
    """Hand-worked decoding of packed 4-bit codes (tests/golden/q4_dequant.txt)."""
    codes, qs, scale_bits, scale = _golden_q4()
    w = oracle.dequant_q4(codes, np.array([[scale_bits]], dtype=np.uint16))
    np.testing.assert_array_equal(w[0], qs * scale)


def test_q4_quantizer_round_trip_bound():
    """Input preparation and the oracle's decoding agree: |dequant(quant(w)) - w| <= s/2 for every weight,
    the largest magnitude of a group is kept within s/2, and q stays in [-8, 7]."""
    from moe_layer_forward_amd import synth

    bits = synth.host_tensor(5, 3, 0, (64, 256), 0.02, "bf16")
    w = synth.bf16_bits_to_f32(bits).astype(np.float64)
    codes, scales = synth.host_quantize_q4(bits)
    deq = oracle.dequant_q4(codes, scales)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(deq - w) <= s / 2 + 1e-12)
    amax = np.abs(w).reshape(64, 8, 32).max(axis=2)
    dmax = np.abs(deq).reshape(64, 8, 32).max(axis=2)
    assert np.all(np.abs(dmax - amax) <= scales.view(np.float16).astype(np.float64) / 2 + 1e-12)
    assert np.all(np.abs(deq / np.where(s > 0, s, 1)) <= 8)
    # a zero group stays zero
    zc, zs = synth.host_quantize_q4(np.zeros((1, 32), dtype=np.uint16))
    assert zs[0, 0] == 0 and zc.sum() == 0 and np.all(oracle.dequant_q4(zc, zs) == 0)


# --------------------------------------------------------------------------- FP8 (E4M3) weights
def test_fp8_e4m3_matches_library_decoding():
    """Every one of the 256 codes decodes as PyTorch's float8_e4m3fn does (an independent
    implementation of the OCP E4M3 format), NaN codes included."""
    import torch

    c = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_value(c)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(v), np.isnan(ref))
    assert np.isnan(v[[0x7F, 0xFF]]).all()
    np.testing.assert_array_equal(v[~np.isnan(v)], ref[~np.isnan(ref)])


def test_fp8_e4m3_closed_forms():
    """The format's landmarks and spacing: smallest subnormal 2^-9, largest subnormal 7 * 2^-9,
    smallest normal 2^-6, one, largest 448; the positive codes increase strictly with a step of
    2^(max(e, 1) - 10) in binade e; the sign bit negates."""
    v = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x7E] == 448.0
    steps = np.diff(v[:0x7F])
    e = (np.arange(1, 0x7F) >> 3)
    np.testing.assert_array_equal(steps, 2.0 ** (np.maximum(e - ((np.arange(1, 0x7F) & 7) == 0), 1) - 10))
    np.testing.assert_array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def test_fp8_dequant_block_scales_brute_force():
    """dequant_fp8 against an element-by-element loop over a non-square grid of blocks with distinct
    scales (a transposed or misplaced block index fails)."""
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(256, 384), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    scales = rng.uniform(0.5, 2.0, size=(2, 3)).astype(np.float32)
    w = oracle.dequant_fp8(codes, scales)
    table = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    for i in range(0, 256, 7):
        for j in range(0, 384, 5):
            assert w[i, j] == table[codes[i, j]] * float(scales[i // 128, j // 128])


def test_fp8_quantizer_round_trip_bound():
    """Input preparation and the oracle's decoding agree: every weight is kept within half a step
    of E4M3 at its magnitude (times the block scale), each block's largest magnitude maps to 448,
    and an all-zero block stays zero."""
    import torch
    from moe_layer_forward_amd import synth

    bits = synth.host_tensor(6, 3, 0, (256, 384), 0.02, "bf16")
    w = synth.bf16_bits_to_f32(bits).astype(np.float64)
    codes, scales = synth.host_quantize_fp8(bits)
    deq = oracle.dequant_fp8(codes, scales)
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=0), 128, axis=1)
    t = np.abs(w) / s
    e = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
    half_step = 2.0 ** (e - 4)
    assert np.all(np.abs(deq - w) <= half_step * s * (1 + 1e-6))
    blocks = np.abs(codes.reshape(2, 128, 3, 128).transpose(0, 2, 1, 3).reshape(6, -1) & 0x7F)
    assert np.all(blocks.max(axis=1) == 0x7E)
    # the codes are the library's round-to-nearest-even of w / s (computed in fp32, as the quantizer does)
    t32 = torch.from_numpy(synth.bf16_bits_to_f32(bits)) / torch.from_numpy(np.repeat(np.repeat(scales, 128, 0), 128, 1))
    np.testing.assert_array_equal(t32.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), codes)
    zc, zs = synth.host_quantize_fp8(np.zeros((128, 128), dtype=np.uint16))
    assert zs[0, 0] == 0 and zc.sum() == 0 and np.all(oracle.dequant_fp8(zc, zs) == 0)


def test_logit_offsets_force_selection():
    """Offsets of +100 on exactly K experts select them whatever the router says, each with score
    sigma(l + 100) = 1 in float64, so each weight is rsf / K; offsets of -100 on every other expert
    leave the choice unchanged."""
    x = _rng(11).standard_normal((16, 64))
    wr = _rng(12).standard_normal((24, 64)) * 0.02
    forced = np.array([3, 7, 19, 22])
    off = np.zeros(24, np.float32)
    off[forced] = 100.0
    for rest in (0.0, -100.0):
        o = off.copy()
        o[np.setdiff1d(np.arange(24), forced)] = rest
        ids, w, gap, s = oracle.route(x, wr, 4, RSF, logit_offset=o)
        np.testing.assert_array_equal(np.sort(ids, axis=1), np.tile(forced, (16, 1)))
        np.testing.assert_array_equal(w, np.full((16, 4), RSF / 4))
