"""Thin ctypes binding of libfp4.so: the C ABI functions under the same names.

Argument marshalling only: tensors are checked for device, dtype, shape and contiguity,
outputs are allocated with torch when the caller passes none, and the raw device
pointers go to the C entry points on torch's current HIP stream.  Every arithmetic step
runs in the HIP kernels; there is no fallback.  A missing library raises at first use.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4.so")

FP4_NVFP4, FP4_MXFP4 = 0, 1
FP4_F32, FP4_BF16 = 0, 1
FP4_SCALE_COMPUTE, FP4_SCALE_GIVEN = 0, 1
_STATUS = {0: "FP4_OK", 1: "FP4_E_NULL", 2: "FP4_E_SHAPE", 3: "FP4_E_ALIGN",
           4: "FP4_E_UNSUPPORTED", 5: "FP4_E_HIP"}
#: every symbol include/fp4.h declares
EXPORTED = ("fp4_quantize", "fp4_dequantize", "fp4_residual_quantize", "fp4_residual_quantize_mx", "fp4_pack_bytes",
            "fp4_pack", "fp4_unpack", "fp4_gemm", "fp4_status_str", "fp4_last_error")

_lib = None


class Fp4Error(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


def library_path():
    return _LIB_PATH


def lib():
    """Load libfp4.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library missing: {_LIB_PATH} (run microscaled_fp4_quantization_block_amd.build)")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.fp4_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, i32, vp, vp]
        L.fp4_dequantize.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, i32, vp]
        L.fp4_residual_quantize.argtypes = [vp, i64, i64, vp, f32, vp, i64, vp, vp, vp, i32, vp, vp]
        L.fp4_residual_quantize_mx.argtypes = [vp, i64, i64, vp, f32, vp, i64, vp, vp, vp, vp]
        L.fp4_pack_bytes.argtypes = [i64, i64]
        L.fp4_pack_bytes.restype = ctypes.c_size_t
        L.fp4_pack.argtypes = [vp, i64, i64, vp, vp, vp]
        L.fp4_unpack.argtypes = [vp, i64, i64, vp, vp]
        L.fp4_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, vp]
        L.fp4_status_str.argtypes = [i32]
        L.fp4_status_str.restype = ctypes.c_char_p
        L.fp4_last_error.argtypes = []
        L.fp4_last_error.restype = ctypes.c_char_p
        for name in ("fp4_quantize", "fp4_dequantize", "fp4_residual_quantize", "fp4_residual_quantize_mx", "fp4_pack",
                     "fp4_unpack", "fp4_gemm"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise Fp4Error(status, lib().fp4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t


def _arg(t, name, device, shape=None, dtype=None, numel=None):
    """Check a tensor argument the kernels will read or write through a raw pointer:
    contiguous, on `device`, and of the given shape / dtype / minimum element count.  The
    C ABI cannot see sizes, so a short buffer must be refused here."""
    if t is None:
        return None
    _dev(t, name)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {numel}")
    return t


def _dtype_code(dt):
    if dt == torch.float32:
        return FP4_F32
    if dt == torch.bfloat16:
        return FP4_BF16
    raise ValueError(f"unsupported dtype {dt}")


def _fmt_code(fmt):
    return {"nvfp4": FP4_NVFP4, "mxfp4": FP4_MXFP4}[fmt] if isinstance(fmt, str) else int(fmt)


def fp4_quantize(x, fmt="mxfp4", hadamard=0, codes=None, scales=None, tensor_scale=None,
                 mode="compute", dbg_rotated=None, stream=None):
    """Quantize x [M, K] (fp32 or bf16) to packed E2M1 codes [M, K/2] and block scales.

    Returns (codes, scales, tensor_scale); tensor_scale is a 1-element fp32 tensor for
    NVFP4 (written in mode "compute", read in mode "given") and None for MXFP4.
    """
    _dev(x, "x")
    M, K = x.shape
    f = _fmt_code(fmt)
    block = 16 if f == FP4_NVFP4 else 32
    dev = x.device
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, K // block), dtype=torch.uint8, device=dev)
    if f == FP4_NVFP4 and tensor_scale is None:
        tensor_scale = torch.zeros(1, dtype=torch.float32, device=dev)
    _arg(codes, "codes", dev, (M, K // 2), torch.uint8)
    _arg(scales, "scales", dev, (M, K // block), torch.uint8)
    if f == FP4_NVFP4:
        _arg(tensor_scale, "tensor_scale", dev, dtype=torch.float32, numel=1)
    _arg(dbg_rotated, "dbg_rotated", dev, (M, K), torch.float32)
    m = FP4_SCALE_COMPUTE if mode == "compute" else FP4_SCALE_GIVEN
    _check(lib().fp4_quantize(_ptr(x), _dtype_code(x.dtype), M, K, f, int(hadamard), _ptr(codes),
                              _ptr(scales), _ptr(tensor_scale) if f == FP4_NVFP4 else None, m,
                              _ptr(dbg_rotated), _stream(stream)))
    return codes, scales, (tensor_scale if f == FP4_NVFP4 else None)


def fp4_dequantize(codes, scales, tensor_scale=None, fmt="mxfp4", inverse_hadamard=0,
                   out_dtype=torch.float32, y=None, stream=None):
    """Values [M, K] of packed codes [M, K/2] and scales, optional inverse rotation."""
    _dev(codes, "codes")
    M, K = codes.shape[0], codes.shape[1] * 2
    dev = codes.device
    f = _fmt_code(fmt)
    _arg(codes, "codes", dev, dtype=torch.uint8)
    _arg(scales, "scales", dev, (M, K // (16 if f == FP4_NVFP4 else 32)), torch.uint8)
    if f == FP4_NVFP4:
        if tensor_scale is None:
            raise ValueError("NVFP4 dequantization needs tensor_scale")
        _arg(tensor_scale, "tensor_scale", dev, dtype=torch.float32, numel=1)
    if y is None:
        y = torch.empty((M, K), dtype=out_dtype, device=dev)
    _arg(y, "y", dev, (M, K))
    _check(lib().fp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tensor_scale), M, K, _fmt_code(fmt),
                                int(inverse_hadamard), _ptr(y), _dtype_code(y.dtype), _stream(stream)))
    return y


def _residual_args(x, perm, gamma, dbg_normed, codes, scales, S, block):
    M, K = x.shape
    dev = x.device
    _arg(x, "x", dev, dtype=torch.bfloat16)
    _arg(perm, "perm", dev, (K,), torch.int32)
    _arg(gamma, "gamma", dev, (K,), torch.float32)
    _arg(dbg_normed, "dbg_normed", dev, (M, K), torch.float32)
    _arg(codes, "codes", dev, (M, (K + S) // 2), torch.uint8)
    _arg(scales, "scales", dev, (M, (K + S) // block), torch.uint8)


def fp4_residual_quantize(x, perm, S, gamma=None, eps=1e-6, codes=None, scales=None,
                          tensor_scale=None, mode="compute", dbg_normed=None, stream=None):
    """ARCQuant fused RMSNorm + reorder + primary/residual NVFP4 of bf16 x [M, K].

    Returns (codes [M, (K+S)/2], scales [M, (K+S)/16], tensor_scale [1])."""
    _dev(x, "x")
    M, K = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((M, (K + S) // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, (K + S) // 16), dtype=torch.uint8, device=dev)
    if tensor_scale is None:
        tensor_scale = torch.zeros(1, dtype=torch.float32, device=dev)
    _residual_args(x, perm, gamma, dbg_normed, codes, scales, S, 16)
    _arg(tensor_scale, "tensor_scale", dev, dtype=torch.float32, numel=1)
    m = FP4_SCALE_COMPUTE if mode == "compute" else FP4_SCALE_GIVEN
    _check(lib().fp4_residual_quantize(_ptr(x), M, K, _ptr(gamma), float(eps), _ptr(perm), int(S),
                                       _ptr(codes), _ptr(scales), _ptr(tensor_scale), m,
                                       _ptr(dbg_normed), _stream(stream)))
    return codes, scales, tensor_scale


def fp4_residual_quantize_mx(x, perm, S, gamma=None, eps=1e-6, codes=None, scales=None,
                             dbg_normed=None, stream=None):
    """MXFP4 flavour of the ARCQuant fused kernel on bf16 x [M, K].

    Returns (codes [M, (K+S)/2], scales [M, (K+S)/32] E8M0)."""
    _dev(x, "x")
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, (K + S) // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, (K + S) // 32), dtype=torch.uint8, device=x.device)
    _residual_args(x, perm, gamma, dbg_normed, codes, scales, S, 32)
    _check(lib().fp4_residual_quantize_mx(_ptr(x), M, K, _ptr(gamma), float(eps), _ptr(perm), int(S),
                                          _ptr(codes), _ptr(scales), _ptr(dbg_normed), _stream(stream)))
    return codes, scales


def fp4_pack_bytes(M, K):
    return int(lib().fp4_pack_bytes(int(M), int(K)))


def fp4_pack(x, packed=None, dbg_rotated=None, stream=None):
    """Dual-scale FP4 message (uint8 [fp4_pack_bytes(M, K)]) of bf16 x [M, K]."""
    _dev(x, "x")
    M, K = x.shape
    n = fp4_pack_bytes(M, K)
    if packed is None:
        packed = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
    _arg(packed, "packed", x.device, dtype=torch.uint8, numel=n)
    _arg(dbg_rotated, "dbg_rotated", x.device, (M, K), torch.float32)
    _check(lib().fp4_pack(_ptr(x), M, K, _ptr(packed), _ptr(dbg_rotated), _stream(stream)))
    return packed


def fp4_unpack(packed, M, K, y=None, stream=None):
    """bf16 [M, K] reconstruction of a dual-scale FP4 message."""
    _dev(packed, "packed")
    _arg(packed, "packed", packed.device, dtype=torch.uint8, numel=fp4_pack_bytes(M, K))
    if y is None:
        y = torch.empty((M, K), dtype=torch.bfloat16, device=packed.device)
    _arg(y, "y", packed.device, (M, K), torch.bfloat16)
    _check(lib().fp4_unpack(_ptr(packed), M, K, _ptr(y), _stream(stream)))
    return y


def fp4_gemm(a_codes, a_scales, b_codes, b_scales, out_dtype=torch.bfloat16, c=None, stream=None):
    """C [M, N] = A [M, K] B [N, K]^T of MXFP4 operands (codes [rows, K/2], E8M0 [rows, K/32])."""
    for t, n in ((a_codes, "a_codes"), (a_scales, "a_scales"), (b_codes, "b_codes"), (b_scales, "b_scales")):
        _dev(t, n)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[0]
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B disagree on K")
    dev = a_codes.device
    _arg(a_codes, "a_codes", dev, dtype=torch.uint8)
    _arg(b_codes, "b_codes", dev, dtype=torch.uint8)
    _arg(a_scales, "a_scales", dev, (M, K // 32), torch.uint8)
    _arg(b_scales, "b_scales", dev, (N, K // 32), torch.uint8)
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=dev)
    _arg(c, "c", dev, (M, N))
    _check(lib().fp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K,
                          _ptr(c), _dtype_code(c.dtype), _stream(stream)))
    return c
