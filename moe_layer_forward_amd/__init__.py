"""MI355X-native forward of the Kimi-K2 MoE FFN layer.

Thin Python binding of ``libmoe.so`` (the C ABI declared in ``include/moe.h``):
the functions below carry the same names as the C entry points and only
marshal arguments -- torch supplies device memory and the current HIP stream,
every step of the layer runs in the library's gfx950 kernels.  There is no
fallback: if the library is missing, importing a call raises.

Layer (per token): sigmoid router over E experts without groups, top-K,
weights normalised to sum 1 and scaled by 2.827, SwiGLU experts plus one
always-on shared expert, weighted combine ("Kimi K2.5 模型架构深度拆解" §10.2).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16 = 0, 1
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_GROUPED_SWIGLU, MOE_OP_COMBINE, MOE_OP_FORWARD,
 MOE_OP_FORWARD_ROUTED, MOE_OP_FORWARD_Q4, MOE_OP_FORWARD_FP8) = range(8)

EXPORTED = ("moe_workspace_size", "moe_route", "moe_permute", "moe_grouped_swiglu", "moe_combine", "moe_forward",
            "moe_forward_noalloc", "moe_forward_routed", "moe_forward_q4", "moe_forward_fp8", "moe_last_error",
            "moe_profile_events", "moe_profile_count", "moe_profile_kernel")
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20  # the fixed scratch of moe_forward_noalloc (include/moe.h)


class MoeConfig(ctypes.Structure):
    """Mirror of ``moe_config`` in include/moe.h."""
    _fields_ = [
        ("hidden_size", ctypes.c_int32),
        ("moe_intermediate_size", ctypes.c_int32),
        ("n_routed_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_shared_experts", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("norm_topk_prob", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moe status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def load_library():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch first: its bundled HIP runtime (same soname) is then the one libmoe binds to, so
        # torch's streams and allocations are the library's own.
        import torch  # noqa: F401

        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -m moe_layer_forward_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(MoeConfig)
        lib.moe_workspace_size.argtypes = [cfgp, i32, i64, i32]
        lib.moe_workspace_size.restype = sz
        lib.moe_route.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.moe_permute.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.moe_grouped_swiglu.argtypes = [cfgp, i32, vp, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        lib.moe_combine.argtypes = [cfgp, i64, vp, i32, vp, vp, vp, vp, vp]
        lib.moe_forward.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.moe_forward_noalloc.argtypes = [cfgp, i64] + [vp] * 14
        lib.moe_forward_routed.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.moe_forward_q4.argtypes = [cfgp, i64] + [vp] * 17 + [sz, vp]
        lib.moe_forward_fp8.argtypes = [cfgp, i64] + [vp] * 17 + [sz, vp]
        for name in ("moe_route", "moe_permute", "moe_grouped_swiglu", "moe_combine", "moe_forward",
                     "moe_forward_routed", "moe_forward_q4", "moe_forward_fp8"):
            getattr(lib, name).restype = ctypes.c_int
        lib.moe_last_error.argtypes = []
        lib.moe_last_error.restype = ctypes.c_char_p
        lib.moe_profile_events.argtypes = [vp, i32]
        lib.moe_profile_events.restype = ctypes.c_int
        lib.moe_profile_count.argtypes = []
        lib.moe_profile_count.restype = ctypes.c_int32
        lib.moe_profile_kernel.argtypes = [i32]
        lib.moe_profile_kernel.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def moe_last_error() -> str:
    return load_library().moe_last_error().decode()


def make_config(hidden_size=7168, moe_intermediate_size=2048, n_routed_experts=384, top_k=8, n_shared_experts=1,
                routed_scaling_factor=2.827, dtype="bf16", n_group=1, topk_group=1, norm_topk_prob=1) -> MoeConfig:
    """The K2 layer's config by default ([ZH-INFRA] §2.1/§2.4, [DEEP] §4.2-§4.3)."""
    return MoeConfig(hidden_size, moe_intermediate_size, n_routed_experts, top_k, n_shared_experts, n_group,
                     topk_group, norm_topk_prob, routed_scaling_factor, MOE_BF16 if dtype == "bf16" else MOE_F32)


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, moe_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*tensors):
    import torch

    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("moe: every tensor must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("moe: tensors must be contiguous")
        dev = t.device
    return dev, torch.cuda.current_stream(dev).cuda_stream


def _elem(cfg):
    import torch

    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


def moe_workspace_size(cfg: MoeConfig, op: int, rows: int, n_groups: int = 0) -> int:
    n = load_library().moe_workspace_size(ctypes.byref(cfg), op, rows, n_groups)
    if n == 0 and moe_last_error():
        raise MoeError(MOE_ERR_INVALID_ARG, moe_last_error())
    return int(n)


def alloc_workspace(cfg: MoeConfig, op: int, rows: int, n_groups: int = 0, device="cuda"):
    import torch

    n = moe_workspace_size(cfg, op, rows, n_groups)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_route(cfg, x, w_router, score_bias=None, logit_offset=None, topk_ids=None, topk_weights=None,
              workspace=None):
    """Router: returns (topk_ids int32 [T,K], topk_weights fp32 [T,K])."""
    import torch

    T, K = x.shape[0], cfg.top_k
    dev, stream = _dev(x, w_router, score_bias, logit_offset)
    ids = topk_ids if topk_ids is not None else torch.empty((T, K), dtype=torch.int32, device=dev)
    wts = topk_weights if topk_weights is not None else torch.empty((T, K), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else alloc_workspace(cfg, MOE_OP_ROUTE, T, 0, dev)
    _check(load_library().moe_route(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(score_bias),
                                    _ptr(logit_offset), _ptr(ids), _ptr(wts), _ptr(ws), ws.numel(), stream))
    return ids, wts


def moe_permute(cfg, topk_ids, x=None, workspace=None):
    """Dispatch permutation: returns (expert_offsets [E+1], row_token [T*K], pair_row [T,K], x_perm or None)."""
    import torch

    T, K, E = topk_ids.shape[0], cfg.top_k, cfg.n_routed_experts
    dev, stream = _dev(topk_ids, x)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * K, dtype=torch.int32, device=dev)
    pair_row = torch.empty((T, K), dtype=torch.int32, device=dev)
    x_perm = torch.empty((T * K, cfg.hidden_size), dtype=x.dtype, device=dev) if x is not None else None
    ws = workspace if workspace is not None else alloc_workspace(cfg, MOE_OP_PERMUTE, T, 0, dev)
    _check(load_library().moe_permute(ctypes.byref(cfg), T, _ptr(topk_ids), _ptr(off), _ptr(row_token),
                                      _ptr(pair_row), _ptr(x), _ptr(x_perm), _ptr(ws), ws.numel(), stream))
    return off, row_token, pair_row, x_perm


def moe_grouped_swiglu(cfg, group_offsets, max_rows, x, w_gate, w_up, w_down, row_index=None, row_scale=None,
                       y_dtype=None, workspace=None, out=None):
    """Grouped SwiGLU experts: returns y_rows [max_rows, H]."""
    import torch

    G = group_offsets.numel() - 1
    ydt = y_dtype if y_dtype is not None else (MOE_F32 if cfg.dtype == MOE_F32 else MOE_BF16)
    dev, stream = _dev(group_offsets, x, w_gate, w_up, w_down, row_index, row_scale)
    y = out if out is not None else torch.empty(
        (max_rows, cfg.hidden_size), dtype=torch.bfloat16 if ydt == MOE_BF16 else torch.float32, device=dev)
    ws = workspace if workspace is not None else alloc_workspace(cfg, MOE_OP_GROUPED_SWIGLU, max_rows, G, dev)
    _check(load_library().moe_grouped_swiglu(ctypes.byref(cfg), G, _ptr(group_offsets), max_rows, _ptr(x),
                                             _ptr(row_index), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(row_scale),
                                             _ptr(y), ydt, _ptr(ws), ws.numel(), stream))
    return y


def moe_combine(cfg, y_rows, pair_row, topk_weights, y_shared=None, out=None):
    """Weighted combine: returns y [T, H] in the config dtype."""
    import torch

    T = pair_row.shape[0]
    if y_shared is not None and (y_shared.shape[0] < T or y_shared.shape[-1] != cfg.hidden_size):
        raise ValueError(f"y_shared must be [T={T}, H={cfg.hidden_size}], got {tuple(y_shared.shape)}")
    if y_rows.shape[-1] != cfg.hidden_size:
        raise ValueError(f"y_rows must have H={cfg.hidden_size} columns, got {tuple(y_rows.shape)}")
    ydt = MOE_BF16 if y_rows.dtype == torch.bfloat16 else MOE_F32
    dev, stream = _dev(y_rows, pair_row, topk_weights, y_shared)
    y = out if out is not None else torch.empty((T, cfg.hidden_size), dtype=_elem(cfg), device=dev)
    _check(load_library().moe_combine(ctypes.byref(cfg), T, _ptr(y_rows), ydt, _ptr(pair_row), _ptr(topk_weights),
                                      _ptr(y_shared), _ptr(y), stream))
    return y


def moe_forward(cfg, x, w_router, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None, score_bias=None,
                logit_offset=None, return_routing=False, workspace=None, out=None, routing_out=None):
    """The whole layer: returns y [T, H] (and (topk_ids, topk_weights) when return_routing).
    routing_out: caller-owned (topk_ids int32 [T, K], topk_weights fp32 [T, K]) to write the routing
    into (with out and workspace, a call that allocates nothing, e.g. inside a graph capture)."""
    import torch

    T = x.shape[0]
    dev, stream = _dev(x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, score_bias, logit_offset)
    y = out if out is not None else torch.empty((T, cfg.hidden_size), dtype=_elem(cfg), device=dev)
    ids = wts = None
    if routing_out is not None:
        ids, wts = routing_out
        if (ids.dtype != torch.int32 or wts.dtype != torch.float32 or tuple(ids.shape) != (T, cfg.top_k)
                or tuple(wts.shape) != (T, cfg.top_k) or not ids.is_contiguous() or not wts.is_contiguous()):
            raise ValueError("routing_out must be contiguous (int32 [T, K], float32 [T, K]) tensors")
    elif return_routing:
        ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else alloc_workspace(cfg, MOE_OP_FORWARD, T, 0, dev)
    _check(load_library().moe_forward(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(score_bias),
                                      _ptr(logit_offset), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate),
                                      _ptr(ws_up), _ptr(ws_down), _ptr(y), _ptr(ids), _ptr(wts), _ptr(ws),
                                      ws.numel(), stream))
    return (y, ids, wts) if (return_routing or routing_out is not None) else y


def moe_forward_noalloc(cfg, x, w_router, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None,
                        score_bias=None, logit_offset=None, out=None, routing_out=None):
    """The whole layer with the library's fixed per-GPU scratch instead of a workspace: the C call
    allocates nothing (with ``out`` given and ``routing_out`` for the routing, neither does this
    wrapper).  Returns y [T, H] (and the routing tensors when routing_out is given)."""
    import torch

    T = x.shape[0]
    dev, stream = _dev(x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, score_bias, logit_offset)
    y = out if out is not None else torch.empty((T, cfg.hidden_size), dtype=_elem(cfg), device=dev)
    ids = wts = None
    if routing_out is not None:
        ids, wts = routing_out
        if (ids.dtype != torch.int32 or wts.dtype != torch.float32 or tuple(ids.shape) != (T, cfg.top_k)
                or tuple(wts.shape) != (T, cfg.top_k) or not ids.is_contiguous() or not wts.is_contiguous()):
            raise ValueError("routing_out must be contiguous (int32 [T, K], float32 [T, K]) tensors")
    _check(load_library().moe_forward_noalloc(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(score_bias),
                                              _ptr(logit_offset), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                              _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(y), _ptr(ids),
                                              _ptr(wts), stream))
    return (y, ids, wts) if routing_out is not None else y


def moe_forward_routed(cfg, x, topk_ids, topk_weights, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None,
                       workspace=None, out=None):
    """The layer for pre-routed tokens (one expert-parallel rank's share): returns y [T, H]."""
    import torch

    T = x.shape[0]
    dev, stream = _dev(x, topk_ids, topk_weights, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    y = out if out is not None else torch.empty((T, cfg.hidden_size), dtype=_elem(cfg), device=dev)
    ws = workspace if workspace is not None else alloc_workspace(cfg, MOE_OP_FORWARD_ROUTED, T, 0, dev)
    _check(load_library().moe_forward_routed(ctypes.byref(cfg), T, _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                             _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up),
                                             _ptr(ws_down), _ptr(y), _ptr(ws), ws.numel(), stream))
    return y


QUANT_KEYS = ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")


def _forward_quant(entry, op, word_bytes, cfg, x, w_router, q, ws_gate, ws_up, ws_down, score_bias, logit_offset,
                   return_routing, workspace, out):
    import torch

    T = x.shape[0]
    qt = [q[n] for n in QUANT_KEYS]
    for n, t in zip(QUANT_KEYS, qt):
        want = word_bytes[0] if n.endswith("codes") else word_bytes[1]
        if t.element_size() != want:
            raise ValueError(f"{n} must hold {8 * want}-bit elements, got {t.dtype}")
    dev, stream = _dev(x, w_router, *qt, ws_gate, ws_up, ws_down, score_bias, logit_offset)
    y = out if out is not None else torch.empty((T, cfg.hidden_size), dtype=torch.bfloat16, device=dev)
    ids = wts = None
    if return_routing:
        ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else alloc_workspace(cfg, op, T, 0, dev)
    _check(getattr(load_library(), entry)(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(score_bias),
                                          _ptr(logit_offset), *[_ptr(t) for t in qt], _ptr(ws_gate), _ptr(ws_up),
                                          _ptr(ws_down), _ptr(y), _ptr(ids), _ptr(wts), _ptr(ws), ws.numel(),
                                          stream))
    return (y, ids, wts) if return_routing else y


def moe_forward_q4(cfg, x, w_router, q4, ws_gate=None, ws_up=None, ws_down=None, score_bias=None,
                   logit_offset=None, return_routing=False, workspace=None, out=None):
    """The layer with 4-bit routed experts: returns y [T, H] bf16 (and the routing when asked).

    q4 holds the routed experts' codes and scales: a mapping with keys gate_codes, gate_scales,
    up_codes, up_scales, down_codes, down_scales (codes int32/uint32 words, scales 16-bit words of
    binary16 values; layouts as in include/moe.h)."""
    return _forward_quant("moe_forward_q4", MOE_OP_FORWARD_Q4, (4, 2), cfg, x, w_router, q4, ws_gate, ws_up,
                          ws_down, score_bias, logit_offset, return_routing, workspace, out)


def moe_forward_fp8(cfg, x, w_router, f8, ws_gate=None, ws_up=None, ws_down=None, score_bias=None,
                    logit_offset=None, return_routing=False, workspace=None, out=None):
    """The layer with FP8 routed experts: returns y [T, H] bf16 (and the routing when asked).

    f8 holds the routed experts' codes and scales under the same keys as for moe_forward_q4 (codes
    uint8 OCP E4M3 [E, N, K], scales float32 [E, N/128, K/128]; layouts as in include/moe.h)."""
    return _forward_quant("moe_forward_fp8", MOE_OP_FORWARD_FP8, (1, 4), cfg, x, w_router, f8, ws_gate, ws_up,
                          ws_down, score_bias, logit_offset, return_routing, workspace, out)


def moe_profile_events(events_array, n_events: int):
    """Record per-kernel HIP events on this thread's later calls (events_array: ctypes array of
    hipEvent_t handles, or None to stop)."""
    _check(load_library().moe_profile_events(events_array, n_events))


def moe_profile_count() -> int:
    return int(load_library().moe_profile_count())


def moe_profile_kernel(i: int) -> str:
    return load_library().moe_profile_kernel(i).decode()


def config_for(workload) -> MoeConfig:
    """moe_config of a synthetic workload (see ``workloads``)."""
    return make_config(workload.H, workload.I, workload.E, workload.K, workload.n_shared, workload.rsf,
                       workload.dtype)
