"""Python side of the matrix-core probe (test instrument).

`dot(instr, a, b, c, sa=None, sb=None)` evaluates one dot product per row of the
numpy arrays `a` and `b` (operand storage as described for `mfma_probe_dot` in
mfma_probe.hip) with a single gfx950 MFMA instruction and returns the FP32
results.  `encode_*` turn exactly representable values into operand bit
patterns; they reject anything that would need rounding, so every probe input
is the value the test states.
"""
import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmfmaprobe.so")

FP8_FP8, FP8_BF8, BF8_FP8, BF8_BF8, BF16, SCALE_FP4, SCALE_E4M3, SCALE_E5M2, K64_E4M3, K64_E5M2 = range(10)
# instruction -> (A element format, B element format, K)
INSTR = {
    FP8_FP8: ("e4m3", "e4m3", 16), FP8_BF8: ("e4m3", "e5m2", 16),
    BF8_FP8: ("e5m2", "e4m3", 16), BF8_BF8: ("e5m2", "e5m2", 16),
    BF16: ("bf16", "bf16", 16), SCALE_FP4: ("e2m1", "e2m1", 64),
    SCALE_E4M3: ("e4m3", "e4m3", 64), SCALE_E5M2: ("e5m2", "e5m2", 64),
    K64_E4M3: ("e4m3", "e4m3", 64), K64_E5M2: ("e5m2", "e5m2", 64),
}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built; run tests/mfma_probe/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.mfma_probe_dot.argtypes = [ctypes.c_int, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp]
        L.mfma_probe_dot.restype = ctypes.c_int
        L.mfma_probe_k.argtypes = [ctypes.c_int]
        L.mfma_probe_k.restype = ctypes.c_int
        _lib = L
    return _lib


# ---------------------------------------------------------------- encoders
def _minifloat_values(ebits, mbits, bias, has_inf_nan_exp):
    """code -> value for the non-negative codes of a small float format."""
    vals = {}
    for e in range(1 << ebits):
        for m in range(1 << mbits):
            code = (e << mbits) | m
            if has_inf_nan_exp == "ieee" and e == (1 << ebits) - 1:
                continue
            if has_inf_nan_exp == "fn" and e == (1 << ebits) - 1 and m == (1 << mbits) - 1:
                continue
            if e == 0:
                v = math.ldexp(m, 1 - bias - mbits)
            else:
                v = math.ldexp((1 << mbits) | m, e - bias - mbits)
            vals[code] = v
    return vals


_TABLES = {
    "e4m3": (_minifloat_values(4, 3, 7, "fn"), 0x80),
    "e5m2": (_minifloat_values(5, 2, 15, "ieee"), 0x80),
    "e2m1": (_minifloat_values(2, 1, 1, "none"), 0x8),
}
_REVERSE = {f: {v: c for c, v in t.items()} for f, (t, _) in _TABLES.items()}


def encode(fmt, v):
    """Exact code of value v in fmt ('e4m3', 'e5m2', 'e2m1', 'bf16')."""
    v = float(v)
    if fmt == "bf16":
        u = int(np.array([v], dtype=np.float32).view(np.uint32)[0])
        if float(np.float32(v)) != v or (u & 0xFFFF):
            raise ValueError(f"{v!r} is not a bf16 value")
        return u >> 16
    table, sign = _REVERSE[fmt], _TABLES[fmt][1]
    mag = abs(v)
    if mag not in table:
        raise ValueError(f"{v!r} is not an {fmt} value")
    code = table[mag]
    return code | sign if math.copysign(1.0, v) < 0 else code


def representable(fmt, v):
    try:
        encode(fmt, v)
        return True
    except ValueError:
        return False


def pack_operand(fmt, rows, K):
    """rows: list of length-K value lists -> operand storage for one side."""
    n = len(rows)
    if fmt == "bf16":
        out = np.zeros((n, K), dtype=np.uint16)
        for i, r in enumerate(rows):
            for k, v in enumerate(r):
                out[i, k] = encode(fmt, v)
        return out
    if fmt == "e2m1":
        out = np.zeros((n, K // 2), dtype=np.uint8)
        for i, r in enumerate(rows):
            for k, v in enumerate(r):
                out[i, k // 2] |= encode(fmt, v) << (4 * (k & 1))
        return out
    out = np.zeros((n, K), dtype=np.uint8)
    for i, r in enumerate(rows):
        for k, v in enumerate(r):
            out[i, k] = encode(fmt, v)
    return out


# ---------------------------------------------------------------- evaluation
def dot(instr, a, b, c, sa=None, sb=None, device="cuda:0"):
    """Run the instruction on every case; a, b: operand storage (numpy), c: FP32 per case."""
    import torch

    n = a.shape[0]
    c = np.ascontiguousarray(np.asarray(c, dtype=np.float32).reshape(n))
    dev = torch.device(device)
    ta = torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to(dev)
    tb = torch.from_numpy(np.ascontiguousarray(b).view(np.uint8).reshape(-1).copy()).to(dev)
    tc = torch.from_numpy(c.copy()).to(dev)
    td = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    if SCALE_FP4 <= instr <= SCALE_E5M2:
        if sa is None or sb is None:
            raise ValueError("scaled instructions need E8M0 scales for both operands")
        tsa = torch.from_numpy(np.ascontiguousarray(sa, dtype=np.uint8).reshape(-1).copy()).to(dev)
        tsb = torch.from_numpy(np.ascontiguousarray(sb, dtype=np.uint8).reshape(-1).copy()).to(dev)
        psa, psb = tsa.data_ptr(), tsb.data_ptr()
    else:
        psa = psb = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().mfma_probe_dot(instr, n, ta.data_ptr(), tb.data_ptr(), psa, psb, tc.data_ptr(),
                              td.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError(f"mfma_probe_dot returned {rc}")
    torch.cuda.synchronize(dev)
    return td.cpu().numpy()


def dot_values(instr, xs, ys, cs, sa=None, sb=None):
    """Like dot() but from lists of exactly representable values (zero-padded to K)."""
    fa, fb, K = INSTR[instr]
    pad = lambda rows: [list(r) + [0.0] * (K - len(r)) for r in rows]
    return dot(instr, pack_operand(fa, pad(xs), K), pack_operand(fb, pad(ys), K), cs, sa, sb)


# ---------------------------------------------------------------- issue rates
# rate_probe.hip: instruction and pattern selectors of mfma_rate_launch
R_FP8_K16, R_SCALE_FP8_K64, R_SCALE_FP4_K64, R_BF16_K16, R_FP8_16X16X32 = range(5)
RATE_NAMES = {
    R_FP8_K16: "v_mfma_f32_32x32x16_fp8_fp8",
    R_SCALE_FP8_K64: "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)",
    R_SCALE_FP4_K64: "v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1)",
    R_BF16_K16: "v_mfma_f32_32x32x16_bf16",
    R_FP8_16X16X32: "v_mfma_f32_16x16x32_fp8_fp8",
}
P_CHAINS, P_PROMOTE, P_INTERLEAVE = 0, 1, 2
PATTERN_NAMES = {P_CHAINS: "independent chains", P_PROMOTE: "per-block promotion",
                 P_INTERLEAVE: "per-block promotion, interleaved"}


def _rate_lib():
    L = lib()
    if not hasattr(L, "_rate_declared"):
        vp = ctypes.c_void_p
        L.mfma_rate_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_float, vp, vp, vp, vp]
        L.mfma_rate_launch.restype = ctypes.c_int
        L.mfma_rate_flops_per_iter.argtypes = [ctypes.c_int, ctypes.c_int]
        L.mfma_rate_flops_per_iter.restype = ctypes.c_double
        L._rate_declared = True
    return L


RATE_SRC_DWORDS = 9216


def rate_operands(instr, data, seed=7):
    """RATE_SRC_DWORDS dwords of operand registers: random valid codes of the
    instruction's element format, or zeros."""
    n = RATE_SRC_DWORDS
    if data == "zero":
        return np.zeros(n, dtype=np.uint32)
    g = np.random.Generator(np.random.PCG64(seed))
    if instr == R_BF16_K16:
        v = g.standard_normal(2 * n).astype(np.float32).view(np.uint32) >> 16
        return (v[0::2] | (v[1::2] << 16)).astype(np.uint32)
    if instr == R_SCALE_FP4_K64:
        return g.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    codes = g.integers(0, 256, size=4 * n, dtype=np.int64)
    codes[(codes & 0x7F) == 0x7F] = 0x7E      # no E4M3 NaN
    return codes.astype(np.uint8).view(np.uint32).copy()


def rate(instr, pattern=P_CHAINS, data="random", waves_per_simd=2, iters=20000, cus=None,
         repeats=3, device="cuda:0"):
    """Sustained rate of one pattern over the whole chip.

    Launches cus * waves_per_simd workgroups of four waves (one per SIMD) and
    returns a dict: TFLOP/s of the matrix work from the kernel's HIP-event time
    (median of `repeats` launches after one warm-up), the shader clock from the
    waves' s_memtime / s_memrealtime ratio (median over waves, GHz), and the
    shader cycles per instruction that ratio implies."""
    import torch

    dev = torch.device(device)
    if cus is None:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nwg = cus * waves_per_simd
    src = torch.from_numpy(rate_operands(instr, data).view(np.int32).copy()).to(dev)
    times = torch.zeros(2 * nwg * 4, dtype=torch.int64, device=dev)
    sink = torch.zeros(nwg * 4 * 64, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    L = _rate_lib()
    fl = L.mfma_rate_flops_per_iter(instr, pattern)
    if fl <= 0:
        raise ValueError("unknown instruction or pattern")
    ms = []
    for r in range(repeats + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = L.mfma_rate_launch(instr, pattern, nwg, iters, 1.0, src.data_ptr(), times.data_ptr(),
                                sink.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"mfma_rate_launch returned {rc}")
        torch.cuda.synchronize(dev)
        if r > 0:
            ms.append(e0.elapsed_time(e1))
    t = times.cpu().numpy().reshape(-1, 2).astype(np.float64)
    ghz = float(np.median(t[:, 0] / np.maximum(t[:, 1], 1) * 0.1))
    ms_med = float(np.median(ms))
    total = fl * iters * nwg * 4
    instr_per_iter = 4 if pattern == P_CHAINS else 4 * (4 if instr == R_FP8_16X16X32 else
                                                       2 if instr in (R_FP8_K16, R_BF16_K16) else 1)
    # shader cycles per instruction per SIMD, from the chip-wide rate at the
    # measured clock (the waves of one SIMD do not start and end together, so
    # their own loop times overstate the overlap)
    tflops = total / (ms_med * 1e-3) / 1e12
    flop_per_instr = fl / instr_per_iter
    cyc_per_instr = flop_per_instr / (tflops * 1e12 / (cus * 4 * ghz * 1e9)) if tflops > 0 else 0.0
    return {
        "instr": RATE_NAMES[instr], "pattern": PATTERN_NAMES[pattern], "data": data,
        "waves_per_simd": waves_per_simd, "workgroups": nwg, "iters": iters,
        "ms": round(ms_med, 4), "tflops": round(tflops, 1),
        "sclk_ghz": round(ghz, 3), "shader_cycles_per_instr_per_simd": round(cyc_per_instr, 2),
    }
