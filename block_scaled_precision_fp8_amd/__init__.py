"""Block-scaled FP8 / MXFP4 quantisation and GEMM on AMD MI355X (gfx950).

A thin ctypes binding over ``libbsfp8.so`` (C ABI in ``include/bsfp8.h``).
It only marshals arguments: PyTorch provides the device memory and the
stream, every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing, importing the functions
raises, and a non-OK status raises ``RuntimeError``.

Functions (same names as the C ABI):
  fp8_quantize(x, fmt="e4m3", tile_rows=128) -> (codes, scales)
  fp8_quantize_pair(a, b, a_fmt="e4m3", b_fmt="e4m3") -> (a_codes, a_scales, b_codes, b_scales)
  fp8_quantize_transposed(x, fmt="e4m3", tile_rows=128) -> (codes of x^T, scales)
  fp8_quantize_granular(x, fmt="e4m3", granularity="tile"|"row"|"tensor") -> (codes, scales)
  mxfp4_quantize(x) -> (packed, scales)
  mx_quantize(x, block=32|16|8, scale="e8m0"|"f16"|"bf16") -> (packed, scales)
  scaled_gemm(a, a_scales, b, b_scales, a_fmt, b_fmt, out="bf16", d=None) -> d
  scaled_gemm_ex(a, a_scales, b, b_scales, a_fmt, b_fmt, out="bf16", alpha=1.0,
                 c=None, beta=0.0, d=None) -> d = alpha A B + beta C
  scaled_gemm_granular(..., a_gran, b_gran, ...) -> d (scales per tile, row or tensor)
  scaled_gemm_mx(a, a_scales, b, b_scales, block, scale, out="bf16", ...) -> d
  scaled_gemm_quantize_a(x, b, b_scales, ...) -> d (A quantised inside the GEMM;
                 optionally also its codes and scales)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BSFP8_LIB", os.path.join(_HERE, "libbsfp8.so"))

FORMATS = {"e4m3": 0, "e5m2": 1, "mxfp4": 2}
OUTS = {"f32": 0, "bf16": 1, "f16": 2}
GRANULARITIES = {"tile": 0, "row": 1, "tensor": 2, "mx32": 3}
MX_SCALES = {"e8m0": 0, "f16": 1, "bf16": 2}
STATUS = {0: "BSFP8_OK", 1: "BSFP8_ERR_INVALID_ARG", 2: "BSFP8_ERR_UNSUPPORTED",
          3: "BSFP8_ERR_HIP"}
FP8_TILE_ROWS = 128

_lib = None


def lib() -> ctypes.CDLL:
    """Load libbsfp8.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libbsfp8.so not found at {LIB_PATH}; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python block_scaled_precision_fp8_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.fp8_quantize.argtypes = [vp, i64, i64, i64, c_int, c_int, vp, vp, vp]
    L.fp8_quantize.restype = c_int
    L.fp8_quantize_pair.argtypes = [vp, i64, i64, c_int, vp, vp, vp, i64, i64, c_int, vp, vp, i64, vp]
    L.fp8_quantize_pair.restype = c_int
    L.fp8_quantize_transposed.argtypes = [vp, i64, i64, i64, c_int, c_int, vp, vp, vp]
    L.fp8_quantize_transposed.restype = c_int
    L.mxfp4_quantize.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    L.mxfp4_quantize.restype = c_int
    L.scaled_gemm.argtypes = [i64, i64, i64, c_int, vp, vp, c_int, vp, vp, c_int, vp, i64, vp]
    L.scaled_gemm.restype = c_int
    L.scaled_gemm_ex.argtypes = [i64, i64, i64, c_int, vp, vp, c_int, vp, vp, ctypes.c_float, vp,
                                 i64, ctypes.c_float, c_int, vp, i64, vp]
    L.scaled_gemm_ex.restype = c_int
    L.fp8_quantize_granular.argtypes = [vp, i64, i64, i64, c_int, c_int, vp, vp, vp]
    L.fp8_quantize_granular.restype = c_int
    L.scaled_gemm_granular.argtypes = [i64, i64, i64, c_int, vp, vp, c_int, c_int, vp, vp, c_int,
                                       ctypes.c_float, vp, i64, ctypes.c_float, c_int, vp, i64, vp]
    L.scaled_gemm_granular.restype = c_int
    L.scaled_gemm_quantize_a.argtypes = [i64, i64, i64, vp, i64, c_int, c_int, vp, vp, c_int,
                                         ctypes.c_float, vp, i64, ctypes.c_float, c_int, vp, i64,
                                         vp, vp, vp]
    L.scaled_gemm_quantize_a.restype = c_int
    L.mx_quantize.argtypes = [vp, i64, i64, i64, c_int, c_int, vp, vp, vp]
    L.mx_quantize.restype = c_int
    L.scaled_gemm_mx.argtypes = [i64, i64, i64, c_int, c_int, vp, vp, vp, vp, ctypes.c_float, vp, i64,
                                 ctypes.c_float, c_int, vp, i64, vp]
    L.scaled_gemm_mx.restype = c_int
    L.bsfp8_status_string.argtypes = [c_int]
    L.bsfp8_status_string.restype = ctypes.c_char_p
    L.bsfp8_version.argtypes = []
    L.bsfp8_version.restype = c_int
    _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        name = lib().bsfp8_status_string(status).decode()
        raise RuntimeError(f"{what} failed: {name}")


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev_ptr(t) -> int:
    return t.data_ptr() if t.numel() > 0 else 0


def fp8_quantize(x, fmt: str = "e4m3", tile_rows: int = FP8_TILE_ROWS,
                 codes=None, scales=None):
    """Quantise a rows x k FP32 CUDA tensor (row-major, unit column stride)
    to FP8 codes with one FP32 scale per tile_rows x 32 tile."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 CUDA tensor with unit column stride")
    rows, k = x.shape
    if codes is None:
        codes = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(((rows + tile_rows - 1) // tile_rows, (k + 31) // 32),
                             dtype=torch.float32, device=x.device)
    st = lib().fp8_quantize(_dev_ptr(x), rows, k, x.stride(0) if rows > 1 else k, tile_rows,
                            FORMATS[fmt], _dev_ptr(codes), _dev_ptr(scales), _stream(x))
    _check(st, "fp8_quantize")
    return codes, scales


def fp8_quantize_pair(a, b, a_fmt: str = "e4m3", b_fmt: str = "e4m3", a_codes=None, a_scales=None,
                      b_codes=None, b_scales=None):
    """fp8_quantize of A (M x K) and B (N x K, the N x K storage of a K x N
    operand) in one launch; returns (a_codes, a_scales, b_codes, b_scales),
    byte-for-byte what two fp8_quantize calls give."""
    import torch
    for t in (a, b):
        if t.dtype != torch.float32 or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("a and b must be 2-D float32 CUDA tensors with unit column stride")
    if a.shape[1] != b.shape[1] or a.device != b.device:
        raise ValueError("a and b must have the same K and device")
    k = a.shape[1]

    def outs(x, codes, scales):
        rows = x.shape[0]
        if codes is None:
            codes = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
        if scales is None:
            scales = torch.empty(((rows + FP8_TILE_ROWS - 1) // FP8_TILE_ROWS, (k + 31) // 32),
                                 dtype=torch.float32, device=x.device)
        return codes, scales

    a_codes, a_scales = outs(a, a_codes, a_scales)
    b_codes, b_scales = outs(b, b_codes, b_scales)
    ld = lambda x: x.stride(0) if x.shape[0] > 1 else k
    st = lib().fp8_quantize_pair(_dev_ptr(a), a.shape[0], ld(a), FORMATS[a_fmt], _dev_ptr(a_codes),
                                 _dev_ptr(a_scales), _dev_ptr(b), b.shape[0], ld(b), FORMATS[b_fmt],
                                 _dev_ptr(b_codes), _dev_ptr(b_scales), k, _stream(a))
    _check(st, "fp8_quantize_pair")
    return a_codes, a_scales, b_codes, b_scales



def fp8_quantize_transposed(x, fmt: str = "e4m3", tile_rows: int = FP8_TILE_ROWS,
                            codes=None, scales=None):
    """Quantise the transpose of a k x rows FP32 CUDA tensor (row-major, unit
    column stride): returns rows x k codes and FP32 scales per tile_rows x 32
    tile of x^T, identical to fp8_quantize(x.t().contiguous())."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 CUDA tensor with unit column stride")
    k, rows = x.shape
    if codes is None:
        codes = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(((rows + tile_rows - 1) // tile_rows, (k + 31) // 32),
                             dtype=torch.float32, device=x.device)
    st = lib().fp8_quantize_transposed(_dev_ptr(x), k, rows, x.stride(0) if k > 1 else rows,
                                       tile_rows, FORMATS[fmt], _dev_ptr(codes),
                                       _dev_ptr(scales), _stream(x))
    _check(st, "fp8_quantize_transposed")
    return codes, scales

def fp8_quantize_granular(x, fmt: str = "e4m3", granularity: str = "tile", codes=None, scales=None):
    """Quantise a rows x k FP32 CUDA tensor to FP8 with one scale per 128 x 32
    tile ("tile"), per row ("row"; per column for a B operand stored N x K) or
    for the whole tensor ("tensor").  Scales: [ceil(rows/128)][k/32], [rows]
    or [1] float32."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 CUDA tensor with unit column stride")
    rows, k = x.shape
    if codes is None:
        codes = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        shape = {"tile": ((rows + FP8_TILE_ROWS - 1) // FP8_TILE_ROWS, (k + 31) // 32),
                 "row": (rows,), "tensor": (1,)}[granularity]
        scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    st = lib().fp8_quantize_granular(_dev_ptr(x), rows, k, x.stride(0) if rows > 1 else k,
                                     GRANULARITIES[granularity], FORMATS[fmt], _dev_ptr(codes),
                                     _dev_ptr(scales), _stream(x))
    _check(st, "fp8_quantize_granular")
    return codes, scales


def mxfp4_quantize(x, packed=None, scales=None):
    """Quantise a rows x k FP32 CUDA tensor to packed E2M1 (two per byte)
    with one E8M0 scale byte per 32-element block of a row."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 CUDA tensor with unit column stride")
    rows, k = x.shape
    if packed is None:
        packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, (k + 31) // 32), dtype=torch.uint8, device=x.device)
    st = lib().mxfp4_quantize(_dev_ptr(x), rows, k, x.stride(0) if rows > 1 else k,
                              _dev_ptr(packed), _dev_ptr(scales), _stream(x))
    _check(st, "mxfp4_quantize")
    return packed, scales


_OUT_DTYPES = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def scaled_gemm(a, a_scales, b, b_scales, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                out: str = "bf16", d=None, K: Optional[int] = None):
    """D = deq(A) deq(B): A is M x K codes (M x K/2 packed for MXFP4), B is
    N x K codes (a K x N column-major matrix).  Returns D (M x N, float32,
    bfloat16 or float16)."""
    import torch
    M = a.shape[0]
    N = b.shape[0]
    if K is None:
        K = a.shape[1] * (2 if a_fmt == "mxfp4" else 1)
    if d is None:
        d = torch.empty((M, N), dtype=getattr(torch, _OUT_DTYPES[out]), device=a.device)
    ldd = d.stride(0) if M > 1 else N
    st = lib().scaled_gemm(M, N, K, FORMATS[a_fmt], _dev_ptr(a), _dev_ptr(a_scales),
                           FORMATS[b_fmt], _dev_ptr(b), _dev_ptr(b_scales), OUTS[out],
                           _dev_ptr(d), ldd, _stream(a))
    _check(st, "scaled_gemm")
    return d


def scaled_gemm_ex(a, a_scales, b, b_scales, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                   out: str = "bf16", alpha: float = 1.0, c=None, beta: float = 0.0, d=None,
                   K: Optional[int] = None):
    """D = alpha deq(A) deq(B) + beta C.  C (M x N, the output dtype) is read
    only when beta != 0; it may be d itself to accumulate in place."""
    import torch
    M = a.shape[0]
    N = b.shape[0]
    if K is None:
        K = a.shape[1] * (2 if a_fmt == "mxfp4" else 1)
    if d is None:
        d = torch.empty((M, N), dtype=getattr(torch, _OUT_DTYPES[out]), device=a.device)
    ldd = d.stride(0) if M > 1 else N
    if c is None:
        cptr, ldc = 0, 0
    else:
        cptr, ldc = _dev_ptr(c), (c.stride(0) if M > 1 else N)
    st = lib().scaled_gemm_ex(M, N, K, FORMATS[a_fmt], _dev_ptr(a), _dev_ptr(a_scales),
                              FORMATS[b_fmt], _dev_ptr(b), _dev_ptr(b_scales), float(alpha), cptr,
                              ldc, float(beta), OUTS[out], _dev_ptr(d), ldd, _stream(a))
    _check(st, "scaled_gemm_ex")
    return d


def scaled_gemm_granular(a, a_scales, b, b_scales, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                         a_gran: str = "tile", b_gran: str = "tile", out: str = "bf16",
                         alpha: float = 1.0, c=None, beta: float = 0.0, d=None,
                         K: Optional[int] = None):
    """scaled_gemm_ex with a scale granularity per operand ("tile", "row",
    "tensor" for FP8; "mx32" for MXFP4)."""
    import torch
    M = a.shape[0]
    N = b.shape[0]
    if K is None:
        K = a.shape[1] * (2 if a_fmt == "mxfp4" else 1)
    if d is None:
        d = torch.empty((M, N), dtype=getattr(torch, _OUT_DTYPES[out]), device=a.device)
    ldd = d.stride(0) if M > 1 else N
    if c is None:
        cptr, ldc = 0, 0
    else:
        cptr, ldc = _dev_ptr(c), (c.stride(0) if M > 1 else N)
    st = lib().scaled_gemm_granular(M, N, K, FORMATS[a_fmt], _dev_ptr(a), _dev_ptr(a_scales),
                                    GRANULARITIES[a_gran], FORMATS[b_fmt], _dev_ptr(b),
                                    _dev_ptr(b_scales), GRANULARITIES[b_gran], float(alpha), cptr,
                                    ldc, float(beta), OUTS[out], _dev_ptr(d), ldd, _stream(a))
    _check(st, "scaled_gemm_granular")
    return d


def scaled_gemm_quantize_a(x, b, b_scales, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                           b_gran: str = "tile", out: str = "bf16", alpha: float = 1.0, c=None,
                           beta: float = 0.0, d=None, a_codes=None, a_scales=None,
                           return_a: bool = False):
    """D = alpha * deq(Q(x)) deq(B) + beta * C with the FP32 A operand x
    quantised per 128 x 32 tile inside the GEMM.  With return_a (or given
    a_codes / a_scales buffers) A's codes and scales are written as well and
    (d, a_codes, a_scales) is returned; otherwise d."""
    import torch
    M, K = x.shape
    N = b.shape[0]
    ldx = x.stride(0) if M > 1 else K
    if d is None:
        d = torch.empty((M, N), dtype=getattr(torch, _OUT_DTYPES[out]), device=x.device)
    ldd = d.stride(0) if M > 1 else N
    if c is None:
        cptr, ldc = 0, 0
    else:
        cptr, ldc = _dev_ptr(c), (c.stride(0) if M > 1 else N)
    if return_a and a_codes is None:
        a_codes = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        a_scales = torch.empty(((M + FP8_TILE_ROWS - 1) // FP8_TILE_ROWS, K // 32),
                               dtype=torch.float32, device=x.device)
    st = lib().scaled_gemm_quantize_a(M, N, K, _dev_ptr(x), ldx, FORMATS[a_fmt], FORMATS[b_fmt],
                                      _dev_ptr(b), _dev_ptr(b_scales), GRANULARITIES[b_gran],
                                      float(alpha), cptr, ldc, float(beta), OUTS[out], _dev_ptr(d),
                                      ldd, _dev_ptr(a_codes) if a_codes is not None else 0,
                                      _dev_ptr(a_scales) if a_scales is not None else 0, _stream(x))
    _check(st, "scaled_gemm_quantize_a")
    if a_codes is not None:
        return d, a_codes, a_scales
    return d


def mx_quantize(x, block: int = 32, scale: str = "e8m0", packed=None, scales=None):
    """E2M1 quantisation with blocks of `block` (32, 16, 8) K elements and
    block scales of format `scale` ("e8m0" bytes, "f16" / "bf16" 16-bit
    patterns).  Returns (packed rows x k/2 uint8, scales [rows][k/block])."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 CUDA tensor with unit column stride")
    rows, k = x.shape
    if packed is None:
        packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        sdt = torch.uint8 if scale == "e8m0" else torch.int16
        scales = torch.empty((rows, k // block), dtype=sdt, device=x.device)
    st = lib().mx_quantize(_dev_ptr(x), rows, k, x.stride(0) if rows > 1 else k, block,
                           MX_SCALES[scale], _dev_ptr(packed), _dev_ptr(scales), _stream(x))
    _check(st, "mx_quantize")
    return packed, scales


def scaled_gemm_mx(a, a_scales, b, b_scales, block: int = 32, scale: str = "e8m0",
                   out: str = "bf16", alpha: float = 1.0, c=None, beta: float = 0.0, d=None,
                   K: Optional[int] = None):
    """D = alpha * deq(A) deq(B) + beta * C for mx_quantize operands (A: M x K/2,
    B: N x K/2 packed, scales [rows][K/block])."""
    import torch
    M = a.shape[0]
    N = b.shape[0]
    if K is None:
        K = a.shape[1] * 2
    if d is None:
        d = torch.empty((M, N), dtype=getattr(torch, _OUT_DTYPES[out]), device=a.device)
    ldd = d.stride(0) if M > 1 else N
    if c is None:
        cptr, ldc = 0, 0
    else:
        cptr, ldc = _dev_ptr(c), (c.stride(0) if M > 1 else N)
    st = lib().scaled_gemm_mx(M, N, K, block, MX_SCALES[scale], _dev_ptr(a), _dev_ptr(a_scales),
                              _dev_ptr(b), _dev_ptr(b_scales), float(alpha), cptr, ldc, float(beta),
                              OUTS[out], _dev_ptr(d), ldd, _stream(a))
    _check(st, "scaled_gemm_mx")
    return d
