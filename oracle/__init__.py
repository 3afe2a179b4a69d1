"""CPU oracle for block-scaled FP8 / MXFP4 quantisation and GEMM (Python side).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import this package.  It
shares no code with the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, explicit format tables);
this module only marshals numpy arrays through ctypes.  Formats are named
"e4m3", "e5m2", "e2m1", "e8m0" and "mxfp4".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB points the pins at another build of oracle.c (the mutation tests
# build copies with planted mistakes and check that some pin fails).
_LIB_PATH = os.environ.get("ORACLE_LIB", os.path.join(_HERE, "liboracle.so"))

_FMT = {"e4m3": 0, "e5m2": 1, "e2m1": 2, "e8m0": 3, "mxfp4": 2}
FP8_TILE_ROWS = 128

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.oracle_decode_table.argtypes = [c_int, vp]
        L.oracle_decode_table.restype = c_int
        L.oracle_decode.argtypes = [c_int, ctypes.c_uint]
        L.oracle_decode.restype = ctypes.c_double
        L.oracle_encode.argtypes = [c_int, ctypes.c_double]
        L.oracle_encode.restype = ctypes.c_uint
        L.oracle_encode_array.argtypes = [c_int, vp, i64, vp]
        L.oracle_encode_array.restype = None
        L.oracle_mx_exponent.argtypes = [ctypes.c_double]
        L.oracle_mx_exponent.restype = c_int
        L.oracle_fp8_quantize.argtypes = [vp, i64, i64, i64, i64, c_int, vp, vp]
        L.oracle_fp8_quantize.restype = c_int
        L.oracle_fp8_quantize_groups.argtypes = [vp, i64, i64, i64, i64, i64, c_int, vp, vp]
        L.oracle_fp8_quantize_groups.restype = c_int
        L.oracle_mxfp4_quantize.argtypes = [vp, i64, i64, i64, vp, vp]
        L.oracle_mxfp4_quantize.restype = c_int
        L.oracle_mx_quantize.argtypes = [vp, i64, i64, i64, i64, c_int, vp, vp]
        L.oracle_mx_quantize.restype = c_int
        L.oracle_gemm_rows.argtypes = [i64, i64, i64, i64, c_int, vp, vp, c_int, vp, vp,
                                       i64, i64, vp, vp]
        L.oracle_gemm_rows.restype = c_int
        L.oracle_gemm_points.argtypes = [i64, i64, i64, i64, c_int, vp, vp, c_int, vp, vp,
                                         i64, vp, vp, vp, vp]
        L.oracle_gemm_points.restype = c_int
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = c_int
        L.oracle_set_threads.argtypes = [c_int]
        L.oracle_set_threads.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def threads() -> int:
    return lib().oracle_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def decode_table(fmt: str) -> np.ndarray:
    n = 16 if fmt == "e2m1" else 256
    out = np.empty(n, dtype=np.float64)
    got = lib().oracle_decode_table(_FMT[fmt], _ptr(out))
    assert got == n
    return out


def encode(fmt: str, values) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64).reshape(-1))
    out = np.empty(v.size, dtype=np.uint8)
    lib().oracle_encode_array(_FMT[fmt], _ptr(v), v.size, _ptr(out))
    return out.reshape(np.shape(values))


def mx_exponent(amax: float) -> int:
    return lib().oracle_mx_exponent(float(amax))


def fp8_quantize(x: np.ndarray, fmt: str = "e4m3", tile_rows: int = FP8_TILE_ROWS):
    """x: rows x k float32.  Returns (codes uint8 rows x k,
    scales float32 [ceil(rows/tile_rows)][ceil(k/32)])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, k = x.shape
    codes = np.zeros((rows, k), dtype=np.uint8)
    scales = np.zeros(((rows + tile_rows - 1) // tile_rows, (k + 31) // 32), dtype=np.float32)
    rc = lib().oracle_fp8_quantize(_ptr(x), rows, k, k, tile_rows, _FMT[fmt],
                                   _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_fp8_quantize rc={rc}")
    return codes, scales


GRANULARITIES = ("tile", "row", "tensor")


def _group_shape(granularity: str, rows: int, k: int):
    """(group_rows, group_k) of one scale: tile 128 x 32, row 1 x k, tensor rows x k."""
    if granularity == "tile":
        return FP8_TILE_ROWS, 32
    if granularity == "row":
        return 1, max(k, 1)
    if granularity == "tensor":
        return max(rows, 1), max(k, 1)
    raise ValueError(f"unknown granularity {granularity!r}")


def fp8_quantize_granular(x: np.ndarray, fmt: str = "e4m3", granularity: str = "tile"):
    """FP8 quantisation with one scale per 128 x 32 tile ("tile"), per row of x
    ("row": per row of an A operand, per column of a B operand stored N x K)
    or for all of x ("tensor").  Returns (codes uint8 rows x k, scales float32:
    [ceil(rows/128)][ceil(k/32)], [rows] or [1])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, k = x.shape
    gr, gk = _group_shape(granularity, rows, k)
    codes = np.zeros((rows, k), dtype=np.uint8)
    scales = np.zeros(((rows + gr - 1) // gr, (k + gk - 1) // gk), dtype=np.float32)
    rc = lib().oracle_fp8_quantize_groups(_ptr(x), rows, k, k, gr, gk, _FMT[fmt],
                                          _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_fp8_quantize_groups rc={rc}")
    if granularity == "row":
        scales = scales.reshape(rows)
    elif granularity == "tensor":
        scales = np.ones(1, dtype=np.float32) if rows * k == 0 else scales.reshape(1)
    return codes, scales


def dequantize_granular(fmt: str, q: np.ndarray, scales: np.ndarray, granularity: str):
    """Dequantised FP8 operand in fp64 (rows x K) for any granularity."""
    if granularity == "tile":
        return dequantize(fmt, q, scales)
    t = decode_table(fmt)
    vals = t[np.asarray(q).astype(np.int64)]
    s = np.asarray(scales, dtype=np.float64)
    if granularity == "row":
        return vals * s.reshape(-1, 1)
    if granularity == "tensor":
        return vals * s.reshape(1)[0]
    raise ValueError(f"unknown granularity {granularity!r}")


def gemm_granular(a_fmt, a, a_scales, a_gran, b_fmt, b, b_scales, b_gran):
    """D = deq(A) deq(B)^T and S = |deq(A)| |deq(B)|^T in fp64, for FP8 operands of
    any granularity (A: M x K codes, B: N x K codes).  The fp64 products of the
    dequantised operands are exact; the sums round at most K 2^-53 S."""
    ad = dequantize_granular(a_fmt, a, a_scales, a_gran)
    bd = dequantize_granular(b_fmt, b, b_scales, b_gran)
    return ad @ bd.T, np.abs(ad) @ np.abs(bd).T


MX_BLOCKS = (32, 16, 8)
MX_SCALES = {"e8m0": 0, "f16": 1, "bf16": 2}


def mx_quantize(x: np.ndarray, block: int = 32, scale: str = "e8m0"):
    """E2M1 block quantisation with blocks of `block` (32, 16 or 8) consecutive
    K elements and block scales of format `scale` ("e8m0", "f16", "bf16").
    x: rows x k float32, k a multiple of block.  Returns (packed uint8
    rows x k/2, low nibble first; scales [rows][k/block]: uint8 E8M0 codes or
    uint16 FP16 / BF16 bit patterns)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, k = x.shape
    packed = np.zeros((rows, k // 2), dtype=np.uint8)
    sdt = np.uint8 if scale == "e8m0" else np.uint16
    scales = np.zeros((rows, k // block), dtype=sdt)
    rc = lib().oracle_mx_quantize(_ptr(x), rows, k, k, block, MX_SCALES[scale], _ptr(packed),
                                  _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_mx_quantize rc={rc}")
    return packed, scales


def mx_scale_values(scales: np.ndarray, scale: str) -> np.ndarray:
    """Block scale values in fp64: E8M0 by the oracle's table, FP16 by numpy's
    binary16, BF16 as the upper half of a binary32."""
    scales = np.asarray(scales)
    if scale == "e8m0":
        return decode_table("e8m0")[scales.astype(np.int64)]
    if scale == "f16":
        return scales.astype(np.uint16).view(np.float16).astype(np.float64)
    return (scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequantize_mx(packed: np.ndarray, scales: np.ndarray, block: int = 32, scale: str = "e8m0"):
    """rows x k fp64 values code * scale of an MX-variant operand."""
    packed = np.asarray(packed)
    rows, kh = packed.shape
    nib = np.empty((rows, 2 * kh), dtype=np.int64)
    nib[:, 0::2] = packed & 0xF
    nib[:, 1::2] = packed >> 4
    sv = np.repeat(mx_scale_values(scales, scale), block, axis=1)
    return decode_table("e2m1")[nib] * sv


def gemm_mx(a, a_scales, b, b_scales, block: int = 32, scale: str = "e8m0"):
    """D = deq(A) deq(B)^T and S = |deq(A)| |deq(B)|^T in fp64 for MX-variant
    operands (A: M x K/2 packed, B: N x K/2 packed)."""
    ad = dequantize_mx(a, a_scales, block, scale)
    bd = dequantize_mx(b, b_scales, block, scale)
    return ad @ bd.T, np.abs(ad) @ np.abs(bd).T


def mxfp4_quantize(x: np.ndarray):
    """x: rows x k float32, k even.  Returns (packed uint8 rows x k/2,
    E8M0 scales uint8 [rows][ceil(k/32)])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, k = x.shape
    packed = np.zeros((rows, k // 2), dtype=np.uint8)
    scales = np.zeros((rows, (k + 31) // 32), dtype=np.uint8)
    rc = lib().oracle_mxfp4_quantize(_ptr(x), rows, k, k, _ptr(packed), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_mxfp4_quantize rc={rc}")
    return packed, scales


def _gemm_args(a_fmt, a, a_scales, b_fmt, b, b_scales):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    a_scales = np.ascontiguousarray(a_scales)
    b_scales = np.ascontiguousarray(b_scales)
    M = a.shape[0]
    N = b.shape[0]
    K = a.shape[1] * (2 if a_fmt == "mxfp4" else 1)
    return M, N, K, a, a_scales, b, b_scales


def gemm_rows(a_fmt, a, a_scales, b_fmt, b, b_scales, row0=0, row1=None,
              tile_rows: int = FP8_TILE_ROWS):
    """Rows [row0, row1) of D = deq(A) deq(B)^T and S = sum |a b| (fp64).
    A: M x K codes (M x K/2 packed for MXFP4); B: N x K codes (a K x N
    column-major matrix)."""
    M, N, K, a, a_scales, b, b_scales = _gemm_args(a_fmt, a, a_scales, b_fmt, b, b_scales)
    row1 = M if row1 is None else row1
    d = np.empty((row1 - row0, N), dtype=np.float64)
    s = np.empty((row1 - row0, N), dtype=np.float64)
    rc = lib().oracle_gemm_rows(M, N, K, tile_rows, _FMT[a_fmt], _ptr(a), _ptr(a_scales),
                                _FMT[b_fmt], _ptr(b), _ptr(b_scales), row0, row1,
                                _ptr(d), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_gemm_rows rc={rc}")
    return d, s


def gemm_points(a_fmt, a, a_scales, b_fmt, b, b_scales, ii, jj,
                tile_rows: int = FP8_TILE_ROWS):
    """D and S at the output positions (ii[p], jj[p])."""
    M, N, K, a, a_scales, b, b_scales = _gemm_args(a_fmt, a, a_scales, b_fmt, b, b_scales)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    d = np.empty(ii.size, dtype=np.float64)
    s = np.empty(ii.size, dtype=np.float64)
    rc = lib().oracle_gemm_points(M, N, K, tile_rows, _FMT[a_fmt], _ptr(a), _ptr(a_scales),
                                  _FMT[b_fmt], _ptr(b), _ptr(b_scales), ii.size,
                                  _ptr(ii), _ptr(jj), _ptr(d), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_gemm_points rc={rc}")
    return d, s


def dequantize(fmt: str, q: np.ndarray, scales: np.ndarray, tile_rows: int = FP8_TILE_ROWS):
    """Dequantised operand in fp64 (rows x K), by the oracle's tables."""
    q = np.asarray(q)
    if fmt == "mxfp4":
        rows, kh = q.shape
        lo = (q & 0xF).astype(np.int64)
        hi = (q >> 4).astype(np.int64)
        nib = np.empty((rows, 2 * kh), dtype=np.int64)
        nib[:, 0::2] = lo
        nib[:, 1::2] = hi
        t4 = decode_table("e2m1")
        t8 = decode_table("e8m0")
        sc = np.repeat(t8[np.asarray(scales, dtype=np.int64)], 32, axis=1)[:, : 2 * kh]
        return t4[nib] * sc
    t = decode_table(fmt)
    rows, k = q.shape
    s = np.asarray(scales, dtype=np.float64)
    sfull = np.repeat(np.repeat(s, tile_rows, axis=0)[:rows], 32, axis=1)[:, :k]
    return t[q.astype(np.int64)] * sfull
