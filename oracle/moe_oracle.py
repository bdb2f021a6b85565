"""Plain, slow, float64 CPU oracle of the Kimi-K2 MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import or call this module.  It shares no
code with the GPU path (``moe_layer_forward_amd``) and imports nothing from it;
the two meet only through the seeded input generator module.

Sources (the pages this follows; "§" = the section on that page):

* [DEEP] "Kimi K2.5 模型架构深度拆解" (pillumina.github.io): §4.2 routing,
  §4.3 expert FFN, §10.2 the seven-step MoE data flow (Steps 1-7).
* [QA]   "Kimi K2.5 架构 QA" (cctoctofx.netlify.app): Q2.1 parameter count,
  Q2.3 routed scaling factor, Q7.2 bias as a non-learned buffer,
  Q8.3 routing dispatch (shared expert + index_add_ combine).
* [ZH-INFRA] Zhihu answer by a K2 inference engineer on why the K2 config
  looks the way it does: §2.4 n_group = 1 (router without expert groups).
* [ZH-PRETRAIN] Zhihu answer by a K2 pretraining author, "架构 / 异":
  routed experts' scaling factor changed from 2.5 to 2.827.

What is computed, per token t (rows are independent):

    l_e   = x_t . Wr_e  (+ o_e, an optional per-expert logit offset)
    s_e   = sigmoid(l_e)
    key_e = s_e + b_e   (b: optional e_score_correction_bias; selection only)
    S_t   = the K experts with the largest key (ties -> smaller expert id)
    w_te  = rsf * s_e / sum_{e' in S_t} s_e'
    F(x)  = W_down (SiLU(W_gate x) * (W_up x)),  SiLU(z) = z * sigmoid(z)
    y_t   = sum_{e in S_t} w_te F_e(x_t) + F_shared(x_t)

Readings where the pages are silent or garbled:

* Everything is float64 except the top-K *decision*, which compares fp32
  keys (fl32(fl32(s) + b)), the precision the GPU kernel decides in.
* The bias enters the selection only; weights use the unbiased scores
  ([QA] Q7.2 says the bias does not interfere with the main loss).  The
  literal listing in [DEEP] §4.2 would normalise biased scores; every
  workload passes no bias, so the two readings agree on them.
* The scaling factor multiplies the normalised routed weights only; the
  shared expert has weight exactly 1 ([DEEP] §10.2 Step 7).
* The routed output is the per-expert weighted sum ([DEEP] §10.2 Step 6);
  the product "weights * sum of expert outputs" in [DEEP] §4.2 does not
  type-check and is read as that sum.
* No epsilon in the normalisation (sigmoid scores are > 0).
* Selected ids are listed by key descending, then id ascending.

4-bit routed experts ([DEEP] §7.2: "pack-quantized", num_bits 4, strategy group, group_size 32,
symmetric, int; the shared expert and the dense MLP stay BF16): an expert weight is w = q * s, q a
signed 4-bit integer, s one scale per group of 32 consecutive inputs of an output row.  Readings
where the page is silent: q is stored as 4-bit two's complement, 8 per 32-bit word, input k in bits
4*(k % 8) of word k // 8; s is stored as IEEE binary16.  ``dequant_q4`` evaluates w exactly in
float64; the layer is then the same function of the dequantized weights.

FP8 routed experts (the Baidu developer article on K2-Instruct, developer.baidu.com article
8800668, §3.2 item 1: FP8 quantization halves the weight memory; the page names neither the
format nor the scaling).  Readings: the routed-expert weights are stored as OCP E4M3 codes (sign,
4 exponent bits with bias 7, 3 mantissa bits, exponent 0 subnormal, no infinities, S.1111.111 NaN)
with one fp32 scale per 128 x 128 block of each matrix, w = e4m3(c) * s[n // 128, k // 128]; only
the storage is quantized, as for the 4-bit weights ([QA] Q7.1).  ``dequant_fp8`` evaluates w
exactly in float64; the layer is then the same function of the dequantized weights.
"""
from __future__ import annotations

import numpy as np

RSF_K2 = 2.827


def sigmoid(z):
    """Logistic function in float64 ([DEEP] §10.2 Step 1; [QA] Q8.3)."""
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def silu(z):
    """SiLU(z) = z * sigmoid(z), the SwiGLU gate activation ([DEEP] §4.3)."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def router_logits(x, w_router, logit_offset=None):
    """Step 1 of [DEEP] §10.2: logits = x @ W_router^T (+ offset), float64 [T, E]."""
    logits = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if logit_offset is not None:
        logits = logits + np.asarray(logit_offset, np.float64)[None, :]
    return logits


def route(x, w_router, top_k, rsf=RSF_K2, score_bias=None, logit_offset=None):
    """Router of [DEEP] §10.2 Steps 1-4 with n_group = 1 ([ZH-INFRA] §2.4).

    Returns (ids int64 [T,K], weights float64 [T,K], gap float64 [T], scores float64 [T,E]).
    ``gap`` is key_(K) - key_(K+1) on the fp32 keys (inf when K == E): tokens
    whose gap is tiny are near-ties where either choice is correct.
    """
    s = sigmoid(router_logits(x, w_router, logit_offset))            # Step 1
    key = s.astype(np.float32)                                       # decision precision
    if score_bias is not None:                                       # Step 2
        key = (key + np.asarray(score_bias, np.float32)[None, :]).astype(np.float32)
    T, E = s.shape
    if not (1 <= top_k <= E):
        raise ValueError("top_k must be in [1, E]")
    order = np.argsort(-key, axis=1, kind="stable")                  # Step 3: key desc, id asc
    ids = order[:, :top_k]
    sel = np.take_along_axis(s, ids, axis=1)
    weights = rsf * sel / sel.sum(axis=1, keepdims=True)             # Step 4
    if top_k < E:
        kk = np.take_along_axis(key, order[:, top_k - 1:top_k + 1], axis=1).astype(np.float64)
        gap = kk[:, 0] - kk[:, 1]
    else:
        gap = np.full(T, np.inf)
    return ids, weights, gap, s


def swiglu_expert(x_rows, w_gate, w_up, w_down):
    """One SwiGLU expert ([DEEP] §4.3, §10.2 Step 5): W_down (SiLU(W_gate x) * W_up x).

    x_rows [m, H]; w_gate, w_up [I, H]; w_down [H, I] (nn.Linear [out, in]).
    """
    x_rows = np.asarray(x_rows, np.float64)
    g = x_rows @ np.asarray(w_gate, np.float64).T
    u = x_rows @ np.asarray(w_up, np.float64).T
    h = silu(g) * u
    return h @ np.asarray(w_down, np.float64).T


def permute(ids, n_experts):
    """Dispatch order of [DEEP] §10.2 Step 6: per-expert contiguous segments.

    Pairs (t, k) are grouped by expert; inside a segment they keep (t, k)
    order.  Returns (expert_offsets [E+1], row_token [T*K], pair_row [T,K]).
    """
    ids = np.asarray(ids, np.int64)
    T, K = ids.shape
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")          # row r holds pair order[r]
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row_token = order // K
    pair_row = np.empty(T * K, np.int64)
    pair_row[order] = np.arange(T * K)
    return offsets, row_token, pair_row.reshape(T, K)


def combine(expert_rows_out, pair_row, weights, shared_out=None):
    """Weighted combine ([DEEP] §10.2 Steps 6-7; [QA] Q8.3 index_add_):

    y_t = sum_k w_tk * O[pair_row[t, k]] (+ shared_out_t).
    """
    O = np.asarray(expert_rows_out, np.float64)
    T, K = pair_row.shape
    y = np.zeros((T, O.shape[1]), np.float64)
    for k in range(K):
        y += np.asarray(weights, np.float64)[:, k:k + 1] * O[pair_row[:, k]]
    if shared_out is not None:
        y += np.asarray(shared_out, np.float64)
    return y


def moe_forward_given_routing(x, ids, weights, expert, shared):
    """Steps 5-7 of [DEEP] §10.2 for already-routed tokens.

    ``expert(e)`` returns (W_gate, W_up, W_down) of routed expert e;
    ``shared`` is that triple for the shared expert, or None.
    The routed experts are visited one unique id at a time and their weighted
    outputs added into the token rows, as the pages' dispatch loop does.
    """
    x = np.asarray(x, np.float64)
    ids = np.asarray(ids, np.int64)
    weights = np.asarray(weights, np.float64)
    y = np.zeros_like(x)
    for e in np.unique(ids):                              # Step 6
        t_idx, k_idx = np.nonzero(ids == e)
        out = swiglu_expert(x[t_idx], *expert(int(e)))
        np.add.at(y, t_idx, weights[t_idx, k_idx][:, None] * out)
    if shared is not None:                                # Steps 5 and 7
        y += swiglu_expert(x, *shared)
    return y


def moe_forward(x, w_router, expert, shared, top_k, rsf=RSF_K2, score_bias=None, logit_offset=None):
    """The whole layer ([DEEP] §10.2 Steps 1-7).

    Returns (y float64 [T,H], ids [T,K], weights [T,K], gap [T]).
    """
    ids, weights, gap, _ = route(x, w_router, top_k, rsf, score_bias, logit_offset)
    y = moe_forward_given_routing(x, ids, weights, expert, shared)
    return y, ids, weights, gap


def expert_param_count(hidden, intermediate):
    """Parameters of one SwiGLU expert: gate, up and down each hold H*I ([QA] Q2.1)."""
    return 3 * hidden * intermediate


def dequant_q4(codes, scales):
    """4-bit group-quantised weight -> float64 ([DEEP] §7.2; readings in the module header).

    codes  uint32 [N, K/8]: q of input k in bits 4*(k % 8) of word k // 8, two's complement;
    scales IEEE binary16 (as uint16 bits or float16) [N, K/32]: one per 32 consecutive inputs.
    Returns w [N, K] = q * s.
    """
    codes = np.asarray(codes, dtype=np.uint32)
    n, words = codes.shape
    nib = ((codes[:, :, None] >> (4 * np.arange(8, dtype=np.uint32))) & np.uint32(0xF)).astype(np.uint8)
    # 4-bit two's complement: fields 0..7 are 0..7, fields 8..15 are -8..-1
    twos = np.array([0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1], dtype=np.float64)
    q = twos[nib].reshape(n, words * 8)
    sc = np.asarray(scales)
    if sc.dtype == np.uint16:
        sc = sc.view(np.float16)
    sc = sc.astype(np.float64)
    if sc.shape != (n, words * 8 // 32):
        raise ValueError("scales must be [N, K/32]")
    # group j of row r holds inputs 32j .. 32j+31, all times sc[r, j]
    return (q.reshape(n, words * 8 // 32, 32) * sc[:, :, None]).reshape(n, words * 8)


def e4m3_value(codes):
    """OCP E4M3 codes (uint8) -> float64 values: bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0
    mantissa m; e = 0 gives the subnormal 2^-6 * m/8, else 2^(e-7) * (1 + m/8); e = 15, m = 7 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def dequant_fp8(codes, scales, block=128):
    """FP8 block-scaled weight -> float64 (readings in the module header).

    codes  uint8 [N, K]: OCP E4M3;  scales float32 [N/block, K/block]: one per block x block tile.
    Returns w [N, K] = e4m3(code) * s[n // block, k // block].
    """
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    sc = np.asarray(scales, dtype=np.float64)
    if n % block or k % block or sc.shape != (n // block, k // block):
        raise ValueError("scales must be [N/block, K/block]")
    # every code's value, looked up in the 256 values e4m3_value gives; then weight (n, k) times the
    # scale of block (n // block, k // block)
    vals = e4m3_value(np.arange(256, dtype=np.uint8))[codes]
    w = vals.reshape(n // block, block, k // block, block) * sc[:, None, :, None]
    return w.reshape(n, k)
