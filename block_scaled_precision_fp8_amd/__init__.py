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


# ---------------------------------------------------------------------------
# Argument checks.  The C ABI takes plain pointers and sizes; these checks make
# sure the tensors behind them hold what the sizes say, so that a wrong tensor
# raises ValueError here instead of reaching a kernel as an out-of-bounds
# access.  Nothing is launched when a check fails.
# ---------------------------------------------------------------------------
def _key(table: dict, value, what: str):
    if value not in table:
        raise ValueError(f"unknown {what} {value!r}; expected one of {sorted(table)}")
    return table[value]


def _tensor(t, name: str, dtypes, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    return t


def _rows_input(x, name: str, device=None):
    """A 2-D float32 CUDA matrix with unit column stride (any row stride >= its width)."""
    import torch
    _tensor(x, name, (torch.float32,), device)
    if x.dim() != 2 or (x.numel() > 0 and x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    if x.shape[0] > 1 and x.stride(0) < x.shape[1]:
        raise ValueError(f"{name} rows overlap (row stride {x.stride(0)} < {x.shape[1]})")
    return x


def _packed(t, name: str, shape, dtypes, device):
    """A contiguous buffer of exactly `shape` (codes rows x K, row stride K)."""
    _tensor(t, name, dtypes, device)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor of shape {tuple(shape)}, "
                         f"got {tuple(t.shape)} (contiguous: {t.is_contiguous()})")
    return t


def _flat(t, name: str, count: int, dtypes, device):
    """A contiguous buffer of at least `count` elements (scale arrays)."""
    _tensor(t, name, dtypes, device)
    if not t.is_contiguous() or t.numel() < count:
        raise ValueError(f"{name} must be contiguous with at least {count} elements, "
                         f"got {t.numel()} (contiguous: {t.is_contiguous()})")
    return t


def _matrix_out(t, name: str, M: int, N: int, dtype, device):
    """An M x N output (or C input) of the given dtype: unit column stride, row stride >= N."""
    _tensor(t, name, (dtype,), device)
    if t.dim() != 2 or tuple(t.shape) != (M, N):
        raise ValueError(f"{name} must be {M} x {N}, got {tuple(t.shape)}")
    if M * N > 0 and ((N > 1 and t.stride(1) != 1) or (M > 1 and t.stride(0) < N)):
        raise ValueError(f"{name} must have unit column stride and row stride >= {N}")
    return t


def _ld(t, rows: int, width: int) -> int:
    return t.stride(0) if rows > 1 else width


def _fp8_scale_count(gran: str, rows: int, K: int) -> int:
    return {"tile": ((rows + FP8_TILE_ROWS - 1) // FP8_TILE_ROWS) * (K // 32), "row": rows,
            "tensor": 1}[gran]


def _fp8_operands(a, a_scales, b, b_scales, a_fmt, b_fmt, K, a_gran="tile", b_gran="tile"):
    """Checks of a GEMM's A and B (codes and scales); returns (M, N, K)."""
    import torch
    u8 = (torch.uint8,)
    _tensor(a, "a", u8)
    dev = a.device
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    mx = a_fmt == "mxfp4"
    per_byte = 2 if mx else 1
    kk = a.shape[1] * per_byte
    if K is None:
        K = kk
    if K != kk or b.shape[1] * per_byte != K:
        raise ValueError(f"K = {K} does not match a ({tuple(a.shape)}) and b ({tuple(b.shape)}); "
                         f"codes are stored with row stride K{' / 2' if mx else ''}")
    M, N = a.shape[0], b.shape[0]
    _packed(a, "a", (M, K // per_byte), u8, dev)
    _packed(b, "b", (N, K // per_byte), u8, dev)
    for sc, name, rows, gran in ((a_scales, "a_scales", M, a_gran), (b_scales, "b_scales", N, b_gran)):
        if mx:
            _flat(sc, name, rows * (K // 32), u8, dev)
        else:
            _flat(sc, name, _fp8_scale_count(gran, rows, K), (torch.float32,), dev)
    return M, N, K


def _epilogue_tensors(d, c, beta, M, N, out, device):
    import torch
    _key(OUTS, out, "output type")
    dt = getattr(torch, _OUT_DTYPES[out])
    if d is None:
        d = torch.empty((M, N), dtype=dt, device=device)
    _matrix_out(d, "d", M, N, dt, device)
    if c is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs c")
        return d, 0, 0
    _matrix_out(c, "c", M, N, dt, device)
    return d, _dev_ptr(c), _ld(c, M, N)


def _fp8_fmt(fmt: str) -> int:
    if fmt not in ("e4m3", "e5m2"):
        raise ValueError(f"unknown FP8 format {fmt!r}; expected 'e4m3' or 'e5m2'")
    return FORMATS[fmt]


def _quant_outputs(rows, k, codes, scales, device, scale_count):
    """Allocate codes (rows x k) when not given, and check codes and the FP32
    scales (allocated by the caller when not given)."""
    import torch
    if codes is None:
        codes = torch.empty((rows, k), dtype=torch.uint8, device=device)
    _packed(codes, "codes", (rows, k), (torch.uint8,), device)
    _flat(scales, "scales", scale_count, (torch.float32,), device)
    return codes, scales


def fp8_quantize(x, fmt: str = "e4m3", tile_rows: int = FP8_TILE_ROWS,
                 codes=None, scales=None):
    """Quantise a rows x k FP32 CUDA tensor (row-major, unit column stride)
    to FP8 codes with one FP32 scale per tile_rows x 32 tile."""
    import torch
    _rows_input(x, "x")
    f = _fp8_fmt(fmt)
    rows, k = x.shape
    if scales is None:
        scales = torch.empty(((rows + tile_rows - 1) // tile_rows, (k + 31) // 32),
                             dtype=torch.float32, device=x.device)
    codes, scales = _quant_outputs(rows, k, codes, scales, x.device,
                                   ((rows + tile_rows - 1) // tile_rows) * (k // 32) if tile_rows > 0 else 0)
    st = lib().fp8_quantize(_dev_ptr(x), rows, k, _ld(x, rows, k), tile_rows, f,
                            _dev_ptr(codes), _dev_ptr(scales), _stream(x))
    _check(st, "fp8_quantize")
    return codes, scales


def fp8_quantize_pair(a, b, a_fmt: str = "e4m3", b_fmt: str = "e4m3", a_codes=None, a_scales=None,
                      b_codes=None, b_scales=None):
    """fp8_quantize of A (M x K) and B (N x K, the N x K storage of a K x N
    operand) in one launch; returns (a_codes, a_scales, b_codes, b_scales),
    byte-for-byte what two fp8_quantize calls give."""
    import torch
    _rows_input(a, "a")
    _rows_input(b, "b", a.device)
    fa, fb = _fp8_fmt(a_fmt), _fp8_fmt(b_fmt)
    if a.shape[1] != b.shape[1]:
        raise ValueError("a and b must have the same K")
    k = a.shape[1]

    def outs(x, codes, scales):
        rows = x.shape[0]
        n = ((rows + FP8_TILE_ROWS - 1) // FP8_TILE_ROWS) * (k // 32)
        if scales is None:
            scales = torch.empty(((rows + FP8_TILE_ROWS - 1) // FP8_TILE_ROWS, (k + 31) // 32),
                                 dtype=torch.float32, device=x.device)
        return _quant_outputs(rows, k, codes, scales, x.device, n)

    a_codes, a_scales = outs(a, a_codes, a_scales)
    b_codes, b_scales = outs(b, b_codes, b_scales)
    st = lib().fp8_quantize_pair(_dev_ptr(a), a.shape[0], _ld(a, a.shape[0], k), fa, _dev_ptr(a_codes),
                                 _dev_ptr(a_scales), _dev_ptr(b), b.shape[0], _ld(b, b.shape[0], k), fb,
                                 _dev_ptr(b_codes), _dev_ptr(b_scales), k, _stream(a))
    _check(st, "fp8_quantize_pair")
    return a_codes, a_scales, b_codes, b_scales


def fp8_quantize_transposed(x, fmt: str = "e4m3", tile_rows: int = FP8_TILE_ROWS,
                            codes=None, scales=None):
    """Quantise the transpose of a k x rows FP32 CUDA tensor (row-major, unit
    column stride): returns rows x k codes and FP32 scales per tile_rows x 32
    tile of x^T, identical to fp8_quantize(x.t().contiguous())."""
    import torch
    _rows_input(x, "x")
    f = _fp8_fmt(fmt)
    k, rows = x.shape
    if scales is None:
        scales = torch.empty(((rows + tile_rows - 1) // tile_rows, (k + 31) // 32),
                             dtype=torch.float32, device=x.device)
    codes, scales = _quant_outputs(rows, k, codes, scales, x.device,
                                   ((rows + tile_rows - 1) // tile_rows) * (k // 32) if tile_rows > 0 else 0)
    st = lib().fp8_quantize_transposed(_dev_ptr(x), k, rows, _ld(x, k, rows), tile_rows, f,
                                       _dev_ptr(codes), _dev_ptr(scales), _stream(x))
    _check(st, "fp8_quantize_transposed")
    return codes, scales


def fp8_quantize_granular(x, fmt: str = "e4m3", granularity: str = "tile", codes=None, scales=None):
    """Quantise a rows x k FP32 CUDA tensor to FP8 with one scale per 128 x 32
    tile ("tile"), per row ("row"; per column for a B operand stored N x K) or
    for the whole tensor ("tensor").  Scales: [ceil(rows/128)][k/32], [rows]
    or [1] float32."""
    import torch
    _rows_input(x, "x")
    f = _fp8_fmt(fmt)
    if granularity not in ("tile", "row", "tensor"):
        raise ValueError(f"unknown FP8 granularity {granularity!r}")
    rows, k = x.shape
    if scales is None:
        shape = {"tile": ((rows + FP8_TILE_ROWS - 1) // FP8_TILE_ROWS, (k + 31) // 32),
                 "row": (rows,), "tensor": (1,)}[granularity]
        scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    codes, scales = _quant_outputs(rows, k, codes, scales, x.device,
                                   _fp8_scale_count(granularity, rows, k))
    st = lib().fp8_quantize_granular(_dev_ptr(x), rows, k, _ld(x, rows, k),
                                     GRANULARITIES[granularity], f, _dev_ptr(codes),
                                     _dev_ptr(scales), _stream(x))
    _check(st, "fp8_quantize_granular")
    return codes, scales


def mxfp4_quantize(x, packed=None, scales=None):
    """Quantise a rows x k FP32 CUDA tensor to packed E2M1 (two per byte)
    with one E8M0 scale byte per 32-element block of a row."""
    import torch
    _rows_input(x, "x")
    rows, k = x.shape
    if packed is None:
        packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, (k + 31) // 32), dtype=torch.uint8, device=x.device)
    _packed(packed, "packed", (rows, k // 2), (torch.uint8,), x.device)
    _flat(scales, "scales", rows * (k // 32), (torch.uint8,), x.device)
    st = lib().mxfp4_quantize(_dev_ptr(x), rows, k, _ld(x, rows, k),
                              _dev_ptr(packed), _dev_ptr(scales), _stream(x))
    _check(st, "mxfp4_quantize")
    return packed, scales


_OUT_DTYPES = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def _gemm_formats(a_fmt, b_fmt):
    fa = _key(FORMATS, a_fmt, "format")
    fb = _key(FORMATS, b_fmt, "format")
    if (a_fmt == "mxfp4") != (b_fmt == "mxfp4"):
        raise ValueError("MXFP4 operands cannot be mixed with FP8 ones")
    return fa, fb


def scaled_gemm(a, a_scales, b, b_scales, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                out: str = "bf16", d=None, K: Optional[int] = None):
    """D = deq(A) deq(B): A is M x K codes (M x K/2 packed for MXFP4), B is
    N x K codes (a K x N column-major matrix).  Returns D (M x N, float32,
    bfloat16 or float16)."""
    fa, fb = _gemm_formats(a_fmt, b_fmt)
    M, N, K = _fp8_operands(a, a_scales, b, b_scales, a_fmt, b_fmt, K,
                            "mx32" if a_fmt == "mxfp4" else "tile", "mx32" if b_fmt == "mxfp4" else "tile")
    d, _, _ = _epilogue_tensors(d, None, 0.0, M, N, out, a.device)
    st = lib().scaled_gemm(M, N, K, fa, _dev_ptr(a), _dev_ptr(a_scales), fb, _dev_ptr(b),
                           _dev_ptr(b_scales), OUTS[out], _dev_ptr(d), _ld(d, M, N), _stream(a))
    _check(st, "scaled_gemm")
    return d


def scaled_gemm_ex(a, a_scales, b, b_scales, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                   out: str = "bf16", alpha: float = 1.0, c=None, beta: float = 0.0, d=None,
                   K: Optional[int] = None):
    """D = alpha deq(A) deq(B) + beta C.  C (M x N, the output dtype) is read
    only when beta != 0; it may be d itself to accumulate in place."""
    fa, fb = _gemm_formats(a_fmt, b_fmt)
    M, N, K = _fp8_operands(a, a_scales, b, b_scales, a_fmt, b_fmt, K,
                            "mx32" if a_fmt == "mxfp4" else "tile", "mx32" if b_fmt == "mxfp4" else "tile")
    d, cptr, ldc = _epilogue_tensors(d, c, beta, M, N, out, a.device)
    st = lib().scaled_gemm_ex(M, N, K, fa, _dev_ptr(a), _dev_ptr(a_scales), fb, _dev_ptr(b),
                              _dev_ptr(b_scales), float(alpha), cptr, ldc, float(beta), OUTS[out],
                              _dev_ptr(d), _ld(d, M, N), _stream(a))
    _check(st, "scaled_gemm_ex")
    return d


def scaled_gemm_granular(a, a_scales, b, b_scales, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                         a_gran: str = "tile", b_gran: str = "tile", out: str = "bf16",
                         alpha: float = 1.0, c=None, beta: float = 0.0, d=None,
                         K: Optional[int] = None):
    """scaled_gemm_ex with a scale granularity per operand ("tile", "row",
    "tensor" for FP8; "mx32" for MXFP4)."""
    fa, fb = _gemm_formats(a_fmt, b_fmt)
    ga = _key(GRANULARITIES, a_gran, "granularity")
    gb = _key(GRANULARITIES, b_gran, "granularity")
    if (a_gran == "mx32") != (a_fmt == "mxfp4") or (b_gran == "mx32") != (b_fmt == "mxfp4"):
        raise ValueError("granularity mx32 goes with MXFP4 operands, tile/row/tensor with FP8 ones")
    M, N, K = _fp8_operands(a, a_scales, b, b_scales, a_fmt, b_fmt, K, a_gran, b_gran)
    d, cptr, ldc = _epilogue_tensors(d, c, beta, M, N, out, a.device)
    st = lib().scaled_gemm_granular(M, N, K, fa, _dev_ptr(a), _dev_ptr(a_scales), ga, fb, _dev_ptr(b),
                                    _dev_ptr(b_scales), gb, float(alpha), cptr, ldc, float(beta),
                                    OUTS[out], _dev_ptr(d), _ld(d, M, N), _stream(a))
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
    _rows_input(x, "x")
    fa, fb = _fp8_fmt(a_fmt), _fp8_fmt(b_fmt)
    if b_gran not in ("tile", "tensor"):
        raise ValueError("b_gran must be 'tile' or 'tensor'")
    M, K = x.shape
    dev = x.device
    _tensor(b, "b", (torch.uint8,), dev)
    if b.dim() != 2:
        raise ValueError("b must be 2-D")
    N = b.shape[0]
    _packed(b, "b", (N, K), (torch.uint8,), dev)
    _flat(b_scales, "b_scales", _fp8_scale_count(b_gran, N, K), (torch.float32,), dev)
    d, cptr, ldc = _epilogue_tensors(d, c, beta, M, N, out, dev)
    if return_a and a_codes is None and a_scales is None:
        a_codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
        a_scales = torch.empty(((M + FP8_TILE_ROWS - 1) // FP8_TILE_ROWS, K // 32),
                               dtype=torch.float32, device=dev)
    if (a_codes is None) != (a_scales is None):
        raise ValueError("a_codes and a_scales go together")
    if a_codes is not None:
        _packed(a_codes, "a_codes", (M, K), (torch.uint8,), dev)
        _flat(a_scales, "a_scales", _fp8_scale_count("tile", M, K), (torch.float32,), dev)
    st = lib().scaled_gemm_quantize_a(M, N, K, _dev_ptr(x), _ld(x, M, K), fa, fb,
                                      _dev_ptr(b), _dev_ptr(b_scales), GRANULARITIES[b_gran],
                                      float(alpha), cptr, ldc, float(beta), OUTS[out], _dev_ptr(d),
                                      _ld(d, M, N), _dev_ptr(a_codes) if a_codes is not None else 0,
                                      _dev_ptr(a_scales) if a_scales is not None else 0, _stream(x))
    _check(st, "scaled_gemm_quantize_a")
    if a_codes is not None:
        return d, a_codes, a_scales
    return d


_MX_SCALE_DTYPES = {"e8m0": ("uint8",), "f16": ("int16", "uint16", "float16"),
                    "bf16": ("int16", "uint16", "bfloat16")}


def _mx_scale_dtypes(scale):
    import torch
    _key(MX_SCALES, scale, "MX scale format")
    return tuple(getattr(torch, n) for n in _MX_SCALE_DTYPES[scale] if hasattr(torch, n))


def mx_quantize(x, block: int = 32, scale: str = "e8m0", packed=None, scales=None):
    """E2M1 quantisation with blocks of `block` (32, 16, 8) K elements and
    block scales of format `scale` ("e8m0" bytes, "f16" / "bf16" 16-bit
    patterns).  Returns (packed rows x k/2 uint8, scales [rows][k/block])."""
    import torch
    _rows_input(x, "x")
    sdts = _mx_scale_dtypes(scale)
    if block not in (32, 16, 8):
        raise ValueError("block must be 32, 16 or 8")
    rows, k = x.shape
    if packed is None:
        packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        sdt = torch.uint8 if scale == "e8m0" else torch.int16
        scales = torch.empty((rows, k // block), dtype=sdt, device=x.device)
    _packed(packed, "packed", (rows, k // 2), (torch.uint8,), x.device)
    _flat(scales, "scales", rows * (k // block), sdts, x.device)
    st = lib().mx_quantize(_dev_ptr(x), rows, k, _ld(x, rows, k), block,
                           MX_SCALES[scale], _dev_ptr(packed), _dev_ptr(scales), _stream(x))
    _check(st, "mx_quantize")
    return packed, scales


def scaled_gemm_mx(a, a_scales, b, b_scales, block: int = 32, scale: str = "e8m0",
                   out: str = "bf16", alpha: float = 1.0, c=None, beta: float = 0.0, d=None,
                   K: Optional[int] = None):
    """D = alpha * deq(A) deq(B) + beta * C for mx_quantize operands (A: M x K/2,
    B: N x K/2 packed, scales [rows][K/block])."""
    import torch
    sdts = _mx_scale_dtypes(scale)
    if block not in (32, 16, 8):
        raise ValueError("block must be 32, 16 or 8")
    _tensor(a, "a", (torch.uint8,))
    dev = a.device
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, N = a.shape[0], b.shape[0]
    if K is None:
        K = a.shape[1] * 2
    if K != a.shape[1] * 2 or K != b.shape[1] * 2:
        raise ValueError(f"K = {K} does not match a ({tuple(a.shape)}) and b ({tuple(b.shape)})")
    _packed(a, "a", (M, K // 2), (torch.uint8,), dev)
    _packed(b, "b", (N, K // 2), (torch.uint8,), dev)
    _flat(a_scales, "a_scales", M * (K // block), sdts, dev)
    _flat(b_scales, "b_scales", N * (K // block), sdts, dev)
    d, cptr, ldc = _epilogue_tensors(d, c, beta, M, N, out, dev)
    st = lib().scaled_gemm_mx(M, N, K, block, MX_SCALES[scale], _dev_ptr(a), _dev_ptr(a_scales),
                              _dev_ptr(b), _dev_ptr(b_scales), float(alpha), cptr, ldc, float(beta),
                              OUTS[out], _dev_ptr(d), _ld(d, M, N), _stream(a))
    _check(st, "scaled_gemm_mx")
    return d
