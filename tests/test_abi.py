"""The C-ABI library without a GPU: it loads, exports every declared symbol, sizes workspaces and
rejects bad arguments before anything is launched (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import moe_layer_forward_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|size_t|const char\*)\s+(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    names = _declared_functions()
    assert set(names) == set(moe.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_config_struct_layout():
    assert ctypes.sizeof(moe.MoeConfig) == 40
    assert moe.MoeConfig.routed_scaling_factor.offset == 32


def test_workspace_sizes():
    cfg = moe.make_config()
    fwd = moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD, 8192)
    # h (73728 x 2048 bf16) + y_rows (73728 x 7168 bf16) dominate
    assert fwd > 73728 * (2048 + 7168) * 2
    assert moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD, 64) < fwd
    assert moe.moe_workspace_size(cfg, moe.MOE_OP_COMBINE, 64) == 0
    assert moe.moe_workspace_size(cfg, moe.MOE_OP_GROUPED_SWIGLU, 1000, 3) > 1000 * 2048 * 2
    assert moe.moe_workspace_size(cfg, moe.MOE_OP_ROUTE, 64) > 0
    assert moe.moe_workspace_size(cfg, moe.MOE_OP_PERMUTE, 64) > 0


def test_noalloc_scratch_limit_at_the_k2_shape():
    """The no-allocation forward's fixed scratch holds the K2 layer's forward workspace up to T = 176
    (the limit include/moe.h states), and its size matches the header's MOE_NOALLOC_SCRATCH_BYTES."""
    import re

    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == moe.MOE_NOALLOC_SCRATCH_BYTES
    cfg = moe.make_config()
    assert moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD, 176) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    assert moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD, 177) > moe.MOE_NOALLOC_SCRATCH_BYTES


def test_noalloc_checks_arguments_before_any_device_call():
    """Config errors come back synchronously from the no-allocation forward too (no GPU needed)."""
    cfg = moe.make_config()
    cfg.n_group = 8
    lib = moe.load_library()
    fake = ctypes.c_void_p(0x1000)
    rc = lib.moe_forward_noalloc(ctypes.byref(cfg), 64, fake, fake, None, None, fake, fake, fake, fake, fake, fake,
                                 fake, None, None, None)
    assert rc == moe.MOE_ERR_UNSUPPORTED and moe.moe_last_error()
    cfg = moe.make_config()
    rc = lib.moe_forward_noalloc(ctypes.byref(cfg), 100000, fake, fake, None, None, fake, fake, fake, fake, fake,
                                 fake, fake, None, None, None)
    assert rc == moe.MOE_ERR_WORKSPACE and "scratch" in moe.moe_last_error()


@pytest.mark.parametrize("field,value,status", [
    ("n_group", 8, moe.MOE_ERR_UNSUPPORTED),
    ("topk_group", 4, moe.MOE_ERR_UNSUPPORTED),
    ("norm_topk_prob", 0, moe.MOE_ERR_UNSUPPORTED),
    ("hidden_size", 7000, moe.MOE_ERR_UNSUPPORTED),
    ("moe_intermediate_size", 2000, moe.MOE_ERR_UNSUPPORTED),
    ("top_k", 400, moe.MOE_ERR_INVALID_ARG),
    ("top_k", 0, moe.MOE_ERR_INVALID_ARG),
    ("n_routed_experts", 600, moe.MOE_ERR_UNSUPPORTED),
    ("n_shared_experts", 2, moe.MOE_ERR_UNSUPPORTED),
    ("dtype", 7, moe.MOE_ERR_UNSUPPORTED),
])
def test_bad_config_is_rejected(field, value, status):
    cfg = moe.make_config()
    setattr(cfg, field, value)
    lib = moe.load_library()
    fake = ctypes.c_void_p(0x1000)
    rc = lib.moe_forward(ctypes.byref(cfg), 64, fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, 1 << 40, None)
    assert rc == status
    assert moe.moe_last_error()
    assert lib.moe_workspace_size(ctypes.byref(cfg), moe.MOE_OP_FORWARD, 64, 0) == 0


def test_null_pointers_and_small_workspace_are_rejected():
    cfg = moe.make_config()
    lib = moe.load_library()
    fake = ctypes.c_void_p(0x1000)
    rc = lib.moe_forward(ctypes.byref(cfg), 64, None, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, 1 << 40, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    rc = lib.moe_forward(ctypes.byref(cfg), 64, fake, fake, None, None, fake, fake, fake, None, fake, fake, fake,
                         None, None, fake, 1 << 40, None)
    assert rc == moe.MOE_ERR_INVALID_ARG and "shared" in moe.moe_last_error()
    rc = lib.moe_forward(ctypes.byref(cfg), 64, fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, 1024, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    rc = lib.moe_forward(ctypes.byref(cfg), 64, fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, None, None, 0, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    rc = lib.moe_forward(ctypes.byref(cfg), -1, fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, 1 << 40, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    rc = lib.moe_route(ctypes.byref(cfg), 64, fake, None, None, None, fake, fake, fake, 1 << 40, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    rc = lib.moe_permute(ctypes.byref(cfg), 64, fake, fake, fake, fake, fake, None, fake, 1 << 40, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    rc = lib.moe_grouped_swiglu(ctypes.byref(cfg), 0, fake, 10, fake, None, fake, fake, fake, None, fake,
                                moe.MOE_BF16, fake, 1 << 40, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    rc = lib.moe_combine(ctypes.byref(cfg), 64, fake, 9, fake, fake, None, fake, None)
    assert rc == moe.MOE_ERR_UNSUPPORTED


def test_operands_past_4_gib_are_unsupported():
    # bf16 operands are addressed with 32-bit byte offsets: h of T*(K+1) rows x I must stay < 4 GiB.
    cfg = moe.make_config()
    lib = moe.load_library()
    fake = ctypes.c_void_p(0x1000)
    T = (1 << 32) // (2 * 2048 * 9) + 1
    rc = lib.moe_forward(ctypes.byref(cfg), T, fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, 1 << 60, None)
    assert rc == moe.MOE_ERR_UNSUPPORTED and "4 GiB" in moe.moe_last_error()
    rc = lib.moe_forward(ctypes.byref(cfg), T - 1, fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, 16, None)
    assert rc == moe.MOE_ERR_WORKSPACE  # within the limit: the next check (workspace) fails instead
    rc = lib.moe_route(ctypes.byref(cfg), (1 << 31) // 7168 + 1, fake, fake, None, None, fake, fake, fake, 1 << 60,
                       None)
    assert rc == moe.MOE_ERR_UNSUPPORTED


def test_q4_forward_argument_checks():
    # the 4-bit forward checks its config, pointers and workspace before launching anything
    lib = moe.load_library()
    fake = ctypes.c_void_p(0x1000)

    def call(cfg, T=64, x=fake, codes=fake, shared=fake, ws=1 << 40):
        return lib.moe_forward_q4(ctypes.byref(cfg), T, x, fake, None, None, codes, fake, fake, fake, fake, fake,
                                  shared, fake, fake, fake, None, None, fake, ws, None)

    cfg = moe.make_config()
    need = moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD_Q4, 64)
    # x16 (64 x 7168 f16), h (576 x 2048) and y_rows (576 x 7168) at least
    assert need > 64 * 7168 * 2 + 576 * (2048 + 7168) * 2
    assert call(cfg, x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(cfg, codes=None) == moe.MOE_ERR_INVALID_ARG
    assert call(cfg, shared=None) == moe.MOE_ERR_INVALID_ARG and "shared" in moe.moe_last_error()
    assert call(cfg, ws=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(cfg, T=0, x=None, codes=None, shared=None, ws=0) == moe.MOE_OK
    for bad in (moe.make_config(hidden_size=7168 + 128), moe.make_config(dtype="f32")):
        assert call(bad) == moe.MOE_ERR_UNSUPPORTED
        assert lib.moe_workspace_size(ctypes.byref(bad), moe.MOE_OP_FORWARD_Q4, 64, 0) == 0


def test_fp8_forward_argument_checks():
    # the FP8 forward checks its config, pointers and workspace before launching anything
    lib = moe.load_library()
    fake = ctypes.c_void_p(0x1000)

    def call(cfg, T=64, x=fake, codes=fake, scales=fake, shared=fake, ws=1 << 40):
        return lib.moe_forward_fp8(ctypes.byref(cfg), T, x, fake, None, None, codes, scales, fake, fake, fake, fake,
                                   shared, fake, fake, fake, None, None, fake, ws, None)

    cfg = moe.make_config()
    need = moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD_FP8, 64)
    assert need == moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD_Q4, 64)  # the same buffers
    assert call(cfg, x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(cfg, codes=None) == moe.MOE_ERR_INVALID_ARG
    assert call(cfg, scales=None) == moe.MOE_ERR_INVALID_ARG
    assert call(cfg, shared=None) == moe.MOE_ERR_INVALID_ARG and "shared" in moe.moe_last_error()
    assert call(cfg, ws=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(cfg, T=0, x=None, codes=None, shared=None, ws=0) == moe.MOE_OK
    # multiples of 128 up to 8192 (7296 is not a multiple of 256, so the 4-bit path refuses it)
    assert moe.moe_workspace_size(moe.make_config(hidden_size=7296), moe.MOE_OP_FORWARD_FP8, 64, 0) > 0
    for bad in (moe.make_config(hidden_size=7168 + 64), moe.make_config(hidden_size=8192 + 128),
                moe.make_config(moe_intermediate_size=8192 + 128), moe.make_config(dtype="f32")):
        assert call(bad) == moe.MOE_ERR_UNSUPPORTED
        assert lib.moe_workspace_size(ctypes.byref(bad), moe.MOE_OP_FORWARD_FP8, 64, 0) == 0


def test_misaligned_pointers_are_refused():
    # checked on the host before anything is launched
    lib = moe.load_library()
    cfg = moe.make_config()
    fake, odd8, odd2 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1002)
    ws = 1 << 40
    rc = lib.moe_forward(ctypes.byref(cfg), 64, odd8, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, ws, None)
    assert rc == moe.MOE_ERR_INVALID_ARG and "x must be 16-byte aligned" in moe.moe_last_error()
    rc = lib.moe_forward(ctypes.byref(cfg), 64, fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake,
                         odd2, None, fake, ws, None)
    assert rc == moe.MOE_ERR_INVALID_ARG and "topk_ids_out must be 4-byte aligned" in moe.moe_last_error()

    def fp8(codes=fake, scales=fake, ws=ws):
        return lib.moe_forward_fp8(ctypes.byref(cfg), 64, fake, fake, None, None, codes, scales, fake, fake, fake,
                                   fake, fake, fake, fake, fake, None, None, fake, ws, None)

    assert fp8(codes=odd8) == moe.MOE_ERR_INVALID_ARG and "gate_codes" in moe.moe_last_error()
    assert fp8(scales=odd2) == moe.MOE_ERR_INVALID_ARG and "gate_scales" in moe.moe_last_error()
    # FP8 scales need 4 bytes only: with too small a workspace the call then stops at that check
    assert fp8(scales=ctypes.c_void_p(0x1004), ws=16) == moe.MOE_ERR_WORKSPACE
    rc = lib.moe_combine(ctypes.byref(cfg), 8, fake, 1, fake, fake, None, odd8, None)
    assert rc == moe.MOE_ERR_INVALID_ARG and "y must be 16-byte aligned" in moe.moe_last_error()


def test_zero_tokens_is_a_no_op():
    cfg = moe.make_config()
    lib = moe.load_library()
    rc = lib.moe_forward(ctypes.byref(cfg), 0, None, None, None, None, None, None, None, None, None, None, None,
                         None, None, None, 0, None)
    assert rc == moe.MOE_OK
    assert lib.moe_route(ctypes.byref(cfg), 0, None, None, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert lib.moe_combine(ctypes.byref(cfg), 0, None, 1, None, None, None, None, None) == moe.MOE_OK


def test_python_binding_refuses_host_tensors():
    import torch

    cfg = moe.make_config(hidden_size=256, moe_intermediate_size=128, n_routed_experts=4, top_k=2)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_route(cfg, x, torch.zeros((4, 256), dtype=torch.bfloat16))
