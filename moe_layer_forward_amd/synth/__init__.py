"""Seeded synthetic inputs for the MoE layer workloads.

One element definition, two independent implementations:

* ``synth_host.c``  (gcc, OpenMP)  -> numpy arrays on the host, used by the
  oracle to regenerate exactly the rows / experts it needs;
* ``synth_dev.hip`` (hipcc, gfx950) -> tensors filled directly in HBM, used
  by the GPU path and the benchmark.

Element ``i`` of tensor ``(seed, stream, index)`` is an Irwin-Hall(8)
approximately-normal variate built from one Philox4x32-10 call (see the
header of ``synth_host.c``), scaled to the requested standard deviation with
one fp32 multiply, and optionally rounded to bf16 (nearest-even).  Nothing of
the MoE layer's arithmetic lives in this module.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# Standard deviation of c = 2*d - 524280, d a sum of eight uniform 16-bit integers.
_C_STD = math.sqrt(8.0 / 3.0 * (2.0**32 - 1.0))


def scale_for(sigma: float) -> float:
    """fp32 multiplier that maps the integer variate to standard deviation sigma."""
    return float(np.float32(sigma / _C_STD))


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(HOST_LIB)
        u32, i64, u64, f32, vp = (ctypes.c_uint32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                                  ctypes.c_void_p)
        lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
        lib.synth_philox4x32_10.restype = None
        for name in ("synth_fill_f32", "synth_fill_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u32, u32, u32, u64, i64, f32, vp]
            fn.restype = None
        for name in ("synth_fill_rows_f32", "synth_fill_rows_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u32, u32, u32, i64, vp, i64, f32, vp]
            fn.restype = None
        lib.synth_quantize_q4.argtypes = [vp, i64, vp, vp]
        lib.synth_quantize_q4.restype = None
        lib.synth_quantize_fp8.argtypes = [vp, i64, i64, i64, vp, vp]
        lib.synth_quantize_fp8.restype = None
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (bind to the HIP runtime torch has loaded)

        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_dev_fill.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                       ctypes.c_void_p]
        lib.synth_dev_fill.restype = ctypes.c_int
        lib.synth_dev_quantize_q4.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]
        lib.synth_dev_quantize_q4.restype = ctypes.c_int
        lib.synth_dev_quantize_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_dev_quantize_fp8.restype = ctypes.c_int
        _dev = lib
    return _dev


def philox4x32_10(counter, key):
    """Raw generator call (4 x uint32 counter, 2 x uint32 key) -> 4 x uint32."""
    c = np.asarray(counter, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    _host_lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32: the pattern becomes the upper 16 bits
    of the float32 (little-endian, so the second uint16 of each pair), the lower 16 bits are zero."""
    bits = np.asarray(bits, dtype=np.uint16)
    pairs = np.zeros(bits.shape + (2,), dtype=np.uint16)
    pairs[..., 1] = bits
    return pairs.view(np.float32)[..., 0]


def host_tensor(seed: int, stream: int, index: int, shape, sigma: float, dtype: str,
                elem0: int = 0) -> np.ndarray:
    """Elements [elem0, elem0 + prod(shape)) of tensor (seed, stream, index).

    dtype 'bf16' returns uint16 bit patterns, 'f32' returns float32.
    """
    n = int(np.prod(shape))
    lib = _host_lib()
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.synth_fill_bf16(seed, stream, index, elem0, n, scale_for(sigma), out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.synth_fill_f32(seed, stream, index, elem0, n, scale_for(sigma), out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def host_rows(seed: int, stream: int, index: int, cols: int, rows, sigma: float, dtype: str) -> np.ndarray:
    """Selected rows of the [*, cols] tensor (seed, stream, index)."""
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    lib = _host_lib()
    if dtype == "bf16":
        out = np.empty((rows.size, cols), dtype=np.uint16)
        lib.synth_fill_rows_bf16(seed, stream, index, cols, rows.ctypes.data, rows.size, scale_for(sigma),
                                 out.ctypes.data)
    elif dtype == "f32":
        out = np.empty((rows.size, cols), dtype=np.float32)
        lib.synth_fill_rows_f32(seed, stream, index, cols, rows.ctypes.data, rows.size, scale_for(sigma),
                                out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def device_fill(tensor, seed: int, stream: int, index0: int, n_index: int, per_index: int, sigma: float):
    """Fill a contiguous torch tensor on the GPU with n_index stacked tensors of
    per_index elements, tensor j being (seed, stream, index0 + j)."""
    import torch

    if not tensor.is_contiguous() or tensor.numel() != n_index * per_index:
        raise ValueError("device_fill: tensor must be contiguous with n_index*per_index elements")
    if tensor.dtype == torch.bfloat16:
        is_bf16 = 1
    elif tensor.dtype == torch.float32:
        is_bf16 = 0
    else:
        raise ValueError(f"device_fill: unsupported dtype {tensor.dtype}")
    stream_ptr = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _dev_lib().synth_dev_fill(tensor.data_ptr(), is_bf16, seed, stream, index0, n_index, per_index,
                                   scale_for(sigma), stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill failed with status {rc}")
    return tensor


# --------------------------------------------------------------------------- 4-bit weight storage
# Input preparation (an offline checkpoint conversion), identical on host and device: per group of 32
# consecutive inputs of a row, s = f16(max|w| / 7), q = clamp(rint(w / s), -8, 7); codes 8 per
# uint32 (input k at bits 4*(k % 8), two's complement), scales as f16 bits.

def host_quantize_q4(w_bits: np.ndarray):
    """bf16 bits [rows, cols] (cols % 32 == 0) -> (codes uint32 [rows, cols/8], scales uint16 [rows, cols/32])."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows, cols = w.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    codes = np.empty((rows, cols // 8), dtype=np.uint32)
    scales = np.empty((rows, cols // 32), dtype=np.uint16)
    _host_lib().synth_quantize_q4(w.ctypes.data, rows * cols // 32, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def device_quantize_q4(w, codes, scales):
    """bf16 tensor [..., cols] -> fills int32 codes [..., cols/8] and 16-bit scales [..., cols/32] on the GPU."""
    import torch

    for t in (w, codes, scales):
        if not t.is_contiguous():
            raise ValueError("device_quantize_q4: tensors must be contiguous")
    if w.dtype != torch.bfloat16 or codes.dtype != torch.int32 or scales.element_size() != 2:
        raise ValueError("device_quantize_q4: w bf16, codes int32, scales 16-bit")
    n_groups = w.numel() // 32
    if w.numel() % 32 or codes.numel() != n_groups * 4 or scales.numel() != n_groups:
        raise ValueError("device_quantize_q4: shapes do not match")
    rc = _dev_lib().synth_dev_quantize_q4(w.data_ptr(), n_groups, codes.data_ptr(), scales.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
    if rc:
        raise RuntimeError(f"synth_dev_quantize_q4 failed ({rc})")
    return codes, scales


# --------------------------------------------------------------------------- 8-bit weight storage
# Input preparation of the same kind, identical on host and device: per 128 x 128 block of a matrix,
# s = max|w| / 448 (fp32), c = OCP E4M3 code of w / s, rounded to nearest even and saturating at
# +-448 (0 when s == 0); codes one byte per weight, scales fp32 [rows/128, cols/128].

def host_quantize_fp8(w_bits: np.ndarray):
    """bf16 bits [rows, cols] (multiples of 128) -> (codes uint8 [rows, cols], scales float32
    [rows/128, cols/128])."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows, cols = w.shape
    if rows % 128 or cols % 128:
        raise ValueError("rows and cols must be multiples of 128")
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows // 128, cols // 128), dtype=np.float32)
    _host_lib().synth_quantize_fp8(w.ctypes.data, 1, rows, cols, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def device_quantize_fp8(w, codes, scales):
    """bf16 tensor [..., rows, cols] -> fills uint8 codes of the same shape and float32 scales
    [..., rows/128, cols/128] on the GPU."""
    import torch

    for t in (w, codes, scales):
        if not t.is_contiguous():
            raise ValueError("device_quantize_fp8: tensors must be contiguous")
    if w.dtype != torch.bfloat16 or codes.dtype != torch.uint8 or scales.dtype != torch.float32:
        raise ValueError("device_quantize_fp8: w bf16, codes uint8, scales float32")
    if w.dim() < 2:
        raise ValueError("device_quantize_fp8: w must be [..., rows, cols]")
    rows, cols = w.shape[-2], w.shape[-1]
    n_mats = w.numel() // (rows * cols) if rows * cols else 0
    if (rows % 128 or cols % 128 or tuple(codes.shape) != tuple(w.shape)
            or scales.numel() != n_mats * (rows // 128) * (cols // 128)):
        raise ValueError("device_quantize_fp8: shapes do not match")
    rc = _dev_lib().synth_dev_quantize_fp8(w.data_ptr(), n_mats, rows, cols, codes.data_ptr(), scales.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    if rc:
        raise RuntimeError(f"synth_dev_quantize_fp8 failed ({rc})")
    return codes, scales
