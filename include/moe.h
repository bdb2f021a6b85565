/*
 * moe.h -- C ABI of the MI355X (gfx950) forward pass of the Kimi-K2 MoE FFN layer.
 *
 * Sources cited below (the section on the page):
 *   [DEEP]        "Kimi K2.5 模型架构深度拆解" (pillumina.github.io/posts/architecture/kimi-k2.5):
 *                 §4.2 routing, §4.3 expert FFN, §10.2 MoE data flow Steps 1-7.
 *   [QA]          "Kimi K2.5 架构 QA" (cctoctofx.netlify.app/posts/qa/kimi-k2.5-qa):
 *                 Q2.1 parameters, Q2.3 routed_scaling_factor, Q7.1 quantized storage,
 *                 Q7.2 bias buffer, Q8.3 dispatch.
 *   [ZH-INFRA]    Zhihu answer by a K2 inference engineer on the K2 config:
 *                 §2.1 num_experts = 384, §2.4 n_group = 1.
 *   [ZH-PRETRAIN] Zhihu answer by a K2 pretraining author, "架构 / 异": scaling factor 2.5 -> 2.827.
 *   [BAIDU]       Baidu developer article on K2-Instruct (developer.baidu.com, article 8800668):
 *                 §3.2 inference acceleration, item 1 (FP8 quantization).
 *
 * The layer, per token t (rows are independent):
 *   l_e = x_t . Wr_e (+ o_e);  s_e = sigmoid(l_e);  key_e = s_e + b_e
 *   S_t = top-K keys over all E experts (no groups), ties -> smaller id
 *   w_te = rsf * s_e / sum_{S_t} s          (the bias b selects only)
 *   F(x) = W_down (SiLU(W_gate x) * (W_up x))
 *   y_t  = sum_{e in S_t} w_te F_e(x_t) + F_shared(x_t)
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host".  The config struct
 *     is a host struct read during the call only.
 *   - Tensors are row-major and contiguous.  Weights use the nn.Linear
 *     [out, in] layout: w_gate/w_up [E, I, H], w_down [E, H, I].
 *   - Alignment: token rows, weights, 4-bit and FP8 codes, 4-bit scales and
 *     outputs start on a 16-byte boundary; id, offset, routing-weight, row-
 *     scale, bias and FP8-scale vectors on a 4-byte one (fresh allocations and
 *     slices along the first dimension of these tensors are).  A misaligned
 *     pointer returns MOE_ERR_INVALID_ARG.
 *   - dtype (config) is the element type of x, y, the router weight and the
 *     expert weights: MOE_BF16 (fp32 accumulation, the intermediate h rounded
 *     to bf16) or MOE_F32.  Routing scores/weights are always fp32, ids int32.
 *   - Ownership: the caller allocates every buffer; the library allocates and
 *     frees nothing and keeps no pointer after a call returns.  Scratch comes
 *     from the caller's `workspace` (device, 256-byte aligned), sized by
 *     moe_workspace_size().
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *     enqueued asynchronously; no call copies to the host or synchronises.
 *     Group sizes never leave the device.
 *   - Errors: arguments are checked synchronously before anything is
 *     launched.  On failure the call returns a moe_status, launches nothing and
 *     sets a thread-local message readable with moe_last_error().  T == 0 (or no
 *     rows) returns MOE_OK and launches nothing.  A failed launch returns
 *     MOE_ERR_DEVICE.  Faults during execution surface at the caller's next
 *     synchronisation.  Calls are reentrant; calls that share a workspace must
 *     be ordered on one stream.
 *   - Supported shapes: hidden_size and moe_intermediate_size multiples of 128;
 *     1 <= top_k <= min(64, n_routed_experts); n_routed_experts <= 512; n_group == topk_group == 1;
 *     n_shared_experts 0 or 1; norm_topk_prob == 1.  For MOE_BF16 every operand matrix the
 *     MFMA kernels read (x, the intermediate h of T*(top_k+n_shared) rows x I, one expert's
 *     weight, the router weight) must span less than 4 GiB (at H = 7168: T <= 299,593 for x and
 *     T*(K+1) <= 524,287 rows for h); larger calls return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* NULL where a pointer is required, negative size, K > E, ...      */
  MOE_ERR_UNSUPPORTED = 2, /* a valid configuration this library does not implement             */
  MOE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than moe_workspace_size()               */
  MOE_ERR_DEVICE = 4       /* a HIP launch failed                                               */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Which call a workspace is sized for (moe_workspace_size). */
typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_GROUPED_SWIGLU = 2,
  MOE_OP_COMBINE = 3,
  MOE_OP_FORWARD = 4,
  MOE_OP_FORWARD_ROUTED = 5,
  MOE_OP_FORWARD_Q4 = 6,
  MOE_OP_FORWARD_FP8 = 7
} moe_op;

/* The MoE config fields of the K2 layer ([DEEP] §4.2-§4.3; [ZH-INFRA] §2.4). Host struct. */
typedef struct moe_config {
  int32_t hidden_size;           /* H: 7168                                                */
  int32_t moe_intermediate_size; /* I: 2048                                                */
  int32_t n_routed_experts;      /* E: 384                                                 */
  int32_t top_k;                 /* K: 8                                                   */
  int32_t n_shared_experts;      /* 0 or 1 (K2: 1, weight 1, never scaled)                 */
  int32_t n_group;               /* must be 1: the router has no expert groups             */
  int32_t topk_group;            /* must be 1                                              */
  int32_t norm_topk_prob;        /* must be 1: weights are normalised to sum 1 ...         */
  float routed_scaling_factor;   /* ... then multiplied by this (K2: 2.827)                */
  int32_t dtype;                 /* moe_dtype of x, y, router and expert weights           */
} moe_config;

/* Bytes of workspace the call `op` needs.
 *   MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_COMBINE, MOE_OP_FORWARD, MOE_OP_FORWARD_ROUTED,
 *   MOE_OP_FORWARD_Q4, MOE_OP_FORWARD_FP8: rows = T (tokens), n_groups ignored.
 *   MOE_OP_GROUPED_SWIGLU: rows = max_rows, n_groups = number of groups.
 * Returns 0 for an invalid config (see moe_last_error()). */
size_t moe_workspace_size(const moe_config* cfg, int32_t op, int64_t rows, int32_t n_groups);

/* Router: [DEEP] §10.2 Steps 1-4, §4.2; n_group = 1 per [ZH-INFRA] §2.4; scale 2.827 per
 * [ZH-PRETRAIN] and [QA] Q2.3.
 *   x            [T, H]  dtype
 *   w_router     [E, H]  dtype
 *   score_bias   [E] fp32 or NULL: e_score_correction_bias ([QA] Q7.2), added to the
 *                scores for the top-K choice only; the weights use the unbiased scores.
 *   logit_offset [E] fp32 or NULL: added to the logits before the sigmoid (synthetic skew).
 *   topk_ids     [T, K] int32 out: the K experts with the largest key, key descending,
 *                ties to the smaller id.
 *   topk_weights [T, K] fp32 out: rsf * s / sum(s) over the selected experts.
 * Workspace: moe_workspace_size(cfg, MOE_OP_ROUTE, T, 0). */
int moe_route(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
              const float* score_bias, const float* logit_offset, int32_t* topk_ids,
              float* topk_weights, void* workspace, size_t workspace_bytes, void* stream);

/* Dispatch permutation: [DEEP] §10.2 Step 6 (tokens of each expert gathered together).
 * Pairs (t, k) are grouped into per-expert contiguous segments of a row space
 * [0, T*K); inside a segment they keep (t, k) order.
 *   topk_ids       [T, K] int32 in, each in [0, E)
 *   expert_offsets [E + 1] int32 out: segment e is rows [off[e], off[e+1]); off[E] = T*K
 *   row_token      [T * K] int32 out: token of row r
 *   pair_row       [T * K] int32 out: row of pair (t, k) at index t*K + k
 *   x, x_perm      both NULL, or x [T, H] dtype in and x_perm [T*K, H] out (x_perm[r] = x[row_token[r]])
 * Workspace: moe_workspace_size(cfg, MOE_OP_PERMUTE, T, 0). */
int moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_ids, int32_t* expert_offsets,
                int32_t* row_token, int32_t* pair_row, const void* x, void* x_perm, void* workspace,
                size_t workspace_bytes, void* stream);

/* Grouped SwiGLU experts: [DEEP] §4.3 and §10.2 Steps 5-6 (gate+up -> SiLU -> x -> down),
 * batched over groups as the grouped GEMM of [QA] Q8.3.
 * For every group g and row r in [group_offsets[g], group_offsets[g+1]):
 *     a = x[row_index ? row_index[r] : r]
 *     y_rows[r] = row_scale[r] (or 1) * W_down[g] (SiLU(W_gate[g] a) * (W_up[g] a))
 *   n_groups       G >= 1 (host)
 *   group_offsets  [G + 1] int32, non-decreasing, group_offsets[0] = 0, last <= max_rows
 *   max_rows       host upper bound on group_offsets[G]; rows at or beyond it are not computed
 *   x              [*, H] dtype; row_index [max_rows] int32 or NULL
 *   w_gate, w_up   [G, I, H] dtype; w_down [G, H, I] dtype
 *   row_scale      [max_rows] fp32 or NULL
 *   y_rows         [max_rows, H] of y_dtype (MOE_F32 or MOE_BF16; MOE_F32 when dtype is MOE_F32)
 * Workspace: moe_workspace_size(cfg, MOE_OP_GROUPED_SWIGLU, max_rows, G). */
int moe_grouped_swiglu(const moe_config* cfg, int32_t n_groups, const int32_t* group_offsets,
                       int64_t max_rows, const void* x, const int32_t* row_index, const void* w_gate,
                       const void* w_up, const void* w_down, const float* row_scale, void* y_rows,
                       int32_t y_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Weighted combine: [DEEP] §10.2 Steps 6-7; [QA] Q8.3 (index_add_ accumulation).
 *     y[t] = sum_k topk_weights[t,k] * y_rows[pair_row[t,k]]  (+ y_shared[t])
 * summed in fp32 in k order, the shared row last, rounded once to dtype.
 *   y_rows   [*, H] of y_dtype;  pair_row [T, K] int32;  topk_weights [T, K] fp32
 *   y_shared [T, H] of y_dtype or NULL;  y [T, H] dtype out
 * No workspace. */
int moe_combine(const moe_config* cfg, int64_t T, const void* y_rows, int32_t y_dtype,
                const int32_t* pair_row, const float* topk_weights, const void* y_shared, void* y,
                void* stream);

/* The whole layer: [DEEP] §10.2 Steps 1-7.
 *   x [T, H]; w_router [E, H]; score_bias, logit_offset as in moe_route
 *   w_gate, w_up [E, I, H]; w_down [E, H, I]            routed experts
 *   ws_gate, ws_up [I, H]; ws_down [H, I]                shared expert (required iff n_shared_experts = 1)
 *   y [T, H] dtype out
 *   topk_ids_out [T, K] int32, topk_weights_out [T, K] fp32: optional copies of the routing (or NULL)
 * Workspace: moe_workspace_size(cfg, MOE_OP_FORWARD, T, 0). */
int moe_forward(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                const float* score_bias, const float* logit_offset, const void* w_gate, const void* w_up,
                const void* w_down, const void* ws_gate, const void* ws_up, const void* ws_down, void* y,
                int32_t* topk_ids_out, float* topk_weights_out, void* workspace, size_t workspace_bytes,
                void* stream);

/* The whole layer, as moe_forward, with no workspace argument and no allocation: for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Scratch comes from a fixed array of MOE_NOALLOC_SCRATCH_BYTES in the library's
 * device code, one per GPU, held until the process ends; its address is looked up on the first call
 * on each device (the device current at the call; `stream` must belong to it).  The call allocates
 * nothing and frees nothing.
 *   Arguments, layouts and results: as moe_forward.
 *   Limit: the call's workspace (moe_workspace_size(cfg, MOE_OP_FORWARD, T, 0)) must fit the array,
 *   otherwise MOE_ERR_WORKSPACE and nothing is launched; at the K2 shape (H = 7168, I = 2048,
 *   E = 384, K = 8, one shared expert) that is T <= 176.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (concurrent streams,
 *   threads) race and give undefined results; calls ordered on one stream do not.  No part of the
 *   array needs to start at zero. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                        const float* score_bias, const float* logit_offset, const void* w_gate,
                        const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                        const void* ws_down, void* y, int32_t* topk_ids_out, float* topk_weights_out,
                        void* stream);

/* The layer for tokens that arrive already routed (one expert-parallel rank's share:
 * [ZH-INFRA] §2.1 places 3 routed + 1 shared expert per rank at EP = 128): Steps 5-7 of
 * [DEEP] §10.2 with topk_ids [T, K] int32 and topk_weights [T, K] fp32 given.
 * Workspace: moe_workspace_size(cfg, MOE_OP_FORWARD_ROUTED, T, 0). */
int moe_forward_routed(const moe_config* cfg, int64_t T, const void* x, const int32_t* topk_ids,
                       const float* topk_weights, const void* w_gate, const void* w_up,
                       const void* w_down, const void* ws_gate, const void* ws_up, const void* ws_down,
                       void* y, void* workspace, size_t workspace_bytes, void* stream);

/* The whole layer with 4-bit routed experts: [DEEP] §7.2 (INT4 weights for the routed experts,
 * symmetric, one scale per group of 32 inputs; shared expert excluded) and [QA] Q7.1 (only the
 * routed experts' storage is quantized, the arithmetic stays high-precision), Steps 1-7 of
 * [DEEP] §10.2.
 * As moe_forward, except that each routed-expert matrix W [E, N, K] comes as
 *   codes  [E, N, K/8] uint32: q[n, k] in bits 4*(k % 8) .. 4*(k % 8)+3 of word k/8, a 4-bit
 *          two's-complement integer in [-8, 7]
 *   scales [E, N, K/32] IEEE binary16 (uint16 bits): s[n, k/32]
 *   W[n, k] = q[n, k] * s[n, k/32]
 * i.e. gate_codes, up_codes [E, I, H/8], gate_scales, up_scales [E, I, H/32],
 *      down_codes [E, H, I/8], down_scales [E, H, I/32].
 * Precision: dtype must be MOE_BF16.  The routed experts multiply in binary16 with fp32
 * accumulation: x is rounded once to binary16 (|x| must stay below 65504); SiLU(g)*u is rounded to
 * binary16 between the two matmuls, y_rows to bf16.  On the weight-stream kernels every code enters
 * the matmul as an exact integer and each 32-input group's fp32 partial sum is multiplied by its
 * scale; on the tile kernels each decoded weight q*s is rounded once to binary16 (within 2^-11
 * relative).  The shared expert and the combine are as in moe_forward.
 * Shapes: as moe_forward, with hidden_size and moe_intermediate_size multiples of 256.
 * Kernels: with at most 4 rows per group on average (decode-sized T) every group streams its
 * codes and scales once per 4 of its rows.  Otherwise the groups run on tile GEMMs that read a
 * group's codes once per 192-row tile (the shared expert's rows too), except that in calls of 16 or
 * more groups those of at most 32 rows keep streaming.
 * Workspace: moe_workspace_size(cfg, MOE_OP_FORWARD_Q4, T, 0). */
int moe_forward_q4(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                   const float* score_bias, const float* logit_offset, const uint32_t* gate_codes,
                   const uint16_t* gate_scales, const uint32_t* up_codes, const uint16_t* up_scales,
                   const uint32_t* down_codes, const uint16_t* down_scales, const void* ws_gate,
                   const void* ws_up, const void* ws_down, void* y, int32_t* topk_ids_out,
                   float* topk_weights_out, void* workspace, size_t workspace_bytes, void* stream);

/* The whole layer with FP8 routed experts: the FP8 quantization of [BAIDU] §3.2 item 1 (weights
 * in 8 bits, half the bytes of bf16), which fixes neither the format nor the scaling.  Read here
 * as OCP E4M3 codes with one fp32 scale per 128 x 128 block of each routed-expert matrix; as for
 * the 4-bit weights ([QA] Q7.1) only the storage is quantized, the shared expert stays bf16, and
 * the layer is Steps 1-7 of [DEEP] §10.2.
 * As moe_forward, except that each routed-expert matrix W [E, N, K] comes as
 *   codes  [E, N, K] uint8: OCP E4M3 (bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0
 *          mantissa; exponent 0 = subnormal, 2^-6 * m/8; largest 448).  0x7f and 0xff (NaN) are
 *          not valid codes.
 *   scales [E, N/128, K/128] fp32: s[n/128, k/128]
 *   W[n, k] = e4m3(code[n, k]) * s[n/128, k/128]
 * i.e. gate_codes, up_codes [E, I, H], gate_scales, up_scales [E, I/128, H/128],
 *      down_codes [E, H, I], down_scales [E, H/128, I/128].
 * Precision: dtype must be MOE_BF16.  The routed experts multiply in binary16 with fp32
 * accumulation: x is rounded once to binary16 (|x| must stay below 65504); SiLU(g)*u is rounded to
 * binary16 between the two matmuls, y_rows to bf16.  On the weight-stream kernels every code enters
 * the matmul exactly (E4M3 values are binary16 values) and each 128-input block's partial sum is
 * multiplied by its scale in fp32; on the tile kernels each weight is decoded with its block scale
 * to binary16 (within 2^-10 relative).  The shared expert and the combine are as in moe_forward.
 * Shapes: as moe_forward, with hidden_size and moe_intermediate_size multiples of 128 and at
 * most 8192 (else MOE_ERR_UNSUPPORTED).
 * Kernels: with at most 4 rows per group on average (decode-sized T) every group streams its codes
 * once per 16 of its rows.  Otherwise the groups run on tile GEMMs that read a group's codes once
 * per 224-row tile (the shared expert's rows too), except that in calls of 16 or more groups those
 * of at most 32 rows keep streaming.
 * Workspace: moe_workspace_size(cfg, MOE_OP_FORWARD_FP8, T, 0). */
int moe_forward_fp8(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                    const float* score_bias, const float* logit_offset, const uint8_t* gate_codes,
                    const float* gate_scales, const uint8_t* up_codes, const float* up_scales,
                    const uint8_t* down_codes, const float* down_scales, const void* ws_gate,
                    const void* ws_up, const void* ws_down, void* y, int32_t* topk_ids_out,
                    float* topk_weights_out, void* workspace, size_t workspace_bytes, void* stream);

/* Message of the last failed call on this thread ("" if none); valid until the next call. */
const char* moe_last_error(void);

/* Per-kernel timing for profilers and benchmarks (not needed for normal use).
 *   events    host array of n_events hipEvent_t handles (as void*), created by the caller; the
 *             library only records them.  NULL / 0 switches timing off.
 * While set (per thread), each later call on this thread records events[2i] and events[2i+1] on
 * its stream right before and right after its i-th kernel launch, for up to min(n_events/2, 32)
 * launches.  moe_profile_count() and moe_profile_kernel(i) report what the last call on this
 * thread launched ("router_logits", "topk", "permute", "plan", "gateup_stream", "down_stream",
 * "gateup_tile", "down_tile", "combine", ...). */
int moe_profile_events(void* const* events, int32_t n_events);
int32_t moe_profile_count(void);
const char* moe_profile_kernel(int32_t i);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
