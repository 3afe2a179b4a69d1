"""Pins of the oracle's MX variants ("Rubin FP4 GEMM deep dive": blocks of 16
or 8 elements, section 5.3; FP16 or BF16 block scales, section 3.2) against
what the page and the number formats fix, independently of the oracle's C:

* blocks of 32 with E8M0 scales are exactly the pinned MXFP4 quantiser;
* brute force on small inputs: the block exponent by exact search over the
  integers, every code by exhaustive nearest-value search over the E2M1
  values (ties to the even code), FP16 / BF16 scales by exhaustive search
  over all positive bit patterns of the format, in exact rational arithmetic;
* invariants: every nonzero block's largest element lands on the top codes;
* the page's claim that smaller blocks and wider scales lose less;
* the GEMM of the dequantised operands against exact rational sums.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # codes 0..7 by the format's bit fields


def e2m1_code(v):
    """Exhaustive nearest E2M1 code of a real v, ties to the even code,
    saturating at 6, sign bit 8 (also for -0)."""
    v = Fraction(v) if not isinstance(v, Fraction) else v
    neg = v < 0
    a = abs(v)
    best = None
    for code, val in enumerate(E2M1):
        d = abs(a - Fraction(val))
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | (8 if neg else 0)


def sign_code(x, code):
    """Apply the sign of a float x (including -0) to a magnitude code."""
    return (code & 7) | (8 if np.signbit(x) else 0)


def smallest_exponent(amax):
    """Smallest integer e with 6 2^e >= amax, by search, clamped to [-127, 127]."""
    a = Fraction(float(amax))
    for e in range(-200, 200):
        if 6 * Fraction(2) ** e >= a:
            return max(-127, min(127, e))
    raise AssertionError


def positive_values(fmt):
    """(bit pattern, value) of every positive finite value of FP16 or BF16,
    in increasing order (the bit patterns of positive values are monotonic)."""
    if fmt == "f16":
        bits = np.arange(1, 0x7C00, dtype=np.uint16)
        vals = bits.view(np.float16).astype(np.float64)
    else:
        bits = np.arange(1, 0x7F80, dtype=np.uint32)
        vals = (bits << 16).view(np.float32).astype(np.float64)
    return bits, vals


_POS = {f: positive_values(f) for f in ("f16", "bf16")}


def nearest_scale(amax, fmt):
    """The format value nearest to amax / 6 (ties to the even bit pattern);
    the largest finite value beyond it; 1 when it is zero."""
    q = Fraction(float(amax)) / 6
    bits, vals = _POS[fmt]
    if q == 0:
        return 1.0
    i = int(np.searchsorted(vals, float(q)))   # vals[i-1] < ~q <= vals[i]
    cands = [j for j in (i - 2, i - 1, i, i + 1) if 0 <= j < len(vals)]
    best = None
    for j in cands:
        d = abs(Fraction(vals[j]) - q)
        if best is None or d < best[0] or (d == best[0] and int(bits[j]) % 2 == 0):
            best = (d, j)
    # below the smallest subnormal: zero if nearer to 0 (tie to 0, the even pattern)
    if q <= Fraction(vals[0]) / 2:
        return 1.0
    if q > Fraction(vals[-1]):
        return float(vals[-1])
    return float(vals[best[1]])


def scale_value(bits16, fmt):
    if fmt == "f16":
        return float(np.array([bits16], dtype=np.uint16).view(np.float16)[0])
    return float((np.array([bits16], dtype=np.uint32) << 16).view(np.float32)[0])


def nibbles(packed):
    rows, kh = packed.shape
    out = np.empty((rows, 2 * kh), dtype=np.int64)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def sample(seed, rows, k):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)) * np.exp2(rng.integers(-20, 20, size=(rows, 1)))
    x[0, :8] = [6.0, -3.0, 0.25, -0.0, 2.5, 1.25, 5.0, 0.75]      # ties and exact values
    x[1, :] = 0.0                                                 # all-zero blocks
    x[2, :4] = [1e-42, -2e-44, 0.0, 3e-45]                        # subnormal block maxima
    return x.astype(np.float32)


def test_block32_e8m0_is_the_mxfp4_quantiser():
    x = sample(1, 40, 256)
    p0, s0 = oracle.mxfp4_quantize(x)
    p1, s1 = oracle.mx_quantize(x, 32, "e8m0")
    assert np.array_equal(p0, p1) and np.array_equal(s0, s1)


@pytest.mark.parametrize("block", [16, 8])
def test_e8m0_blocks_by_brute_force(block):
    x = sample(2 + block, 6, 64)
    packed, scales = oracle.mx_quantize(x, block, "e8m0")
    codes = nibbles(packed)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // block):
            blk = x[r, b * block:(b + 1) * block]
            amax = float(np.max(np.abs(blk)))
            e = 0 if amax == 0 else smallest_exponent(amax)
            assert int(scales[r, b]) == e + 127, (r, b)
            for j, v in enumerate(blk):
                want = sign_code(v, e2m1_code(Fraction(float(v)) / Fraction(2) ** e))
                assert codes[r, b * block + j] == want, (r, b, j, float(v))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("block", [32, 16, 8])
def test_wide_scales_by_brute_force(fmt, block):
    x = sample(3 + block, 5, 64)
    x[3, :] *= np.float32(2.0 ** 20)          # FP16 scales saturate at 65504 here
    packed, scales = oracle.mx_quantize(x, block, fmt)
    assert scales.dtype == np.uint16
    codes = nibbles(packed)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // block):
            blk = x[r, b * block:(b + 1) * block]
            s = nearest_scale(float(np.max(np.abs(blk))), fmt)
            assert scale_value(int(scales[r, b]), fmt) == s, (fmt, r, b)
            for j, v in enumerate(blk):
                y = np.float32(v) / np.float32(s)              # IEEE binary32 division
                want = sign_code(y, e2m1_code(Fraction(float(y))))
                assert codes[r, b * block + j] == want, (fmt, r, b, j, float(v))


def midpoint_rows(fmt):
    """Blocks of 8 whose maximum is 6 s for every scale value s of one binade of
    the format (so the scale is s exactly) and whose other elements are s times
    the seven E2M1 midpoints (so x / s is exactly a midpoint); then blocks whose
    amax / 6 lies exactly halfway between two neighbouring scale values, with
    an even and with an odd lower neighbour."""
    mant = 10 if fmt == "f16" else 7
    ulp = 2.0 ** -mant
    rows = []
    for j in range(2 ** mant):
        sv = 1.0 + j * ulp
        rows.append([6 * sv] + [m * sv for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)])
    for j in (0, 1, 2, 3, 2 ** mant - 2):
        half = 1.0 + (j + 0.5) * ulp
        rows.append([6 * half, -half, 2 * half, 0.0, -3 * half, half / 4, 5 * half, -0.0])
    x = np.array(rows, dtype=np.float64)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)   # all exact in FP32
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_exact_midpoints_and_scale_ties(fmt):
    """Ties at both roundings go to the even neighbour: codes of x / s exactly
    on an E2M1 midpoint, and scales of amax / 6 exactly halfway between two
    scale values."""
    x = midpoint_rows(fmt)
    packed, scales = oracle.mx_quantize(x, 8, fmt)
    codes = nibbles(packed)
    for r in range(x.shape[0]):
        s = nearest_scale(float(np.max(np.abs(x[r]))), fmt)
        assert scale_value(int(scales[r, 0]), fmt) == s, (fmt, r)
        for j, v in enumerate(x[r]):
            y = np.float32(v) / np.float32(s)
            assert codes[r, j] == sign_code(y, e2m1_code(Fraction(float(y)))), (fmt, r, j)


@pytest.mark.parametrize("block", [32, 16, 8])
def test_block_maximum_lands_on_the_top_codes(block):
    x = sample(7, 64, 512)
    for fmt in ("e8m0", "f16", "bf16"):
        packed, scales = oracle.mx_quantize(x, block, fmt)
        codes = nibbles(packed) & 7
        a = np.abs(x).reshape(64, -1, block)
        c = codes.reshape(64, -1, block)
        nz = a.max(axis=2) > 2.0 ** -120
        top = np.take_along_axis(c, a.argmax(axis=2)[..., None], axis=2)[..., 0]
        # E8M0: amax 2^-e in (3, 6] -> code 3 (value 3), 6 (4) or 7 (6); wide scales: 6
        lo = 5 if fmt == "e8m0" else 7
        if fmt == "f16":   # outside FP16's normal range the scale loses precision or saturates
            nz &= (a.max(axis=2) >= 6 * 2.0 ** -14) & (a.max(axis=2) < 6 * 65504)
        assert np.all(top[nz] >= lo), fmt


def test_smaller_blocks_and_wider_scales_lose_less():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((256, 1024)) * rng.lognormal(0, 1, size=(256, 1024))).astype(np.float32)
    err = {}
    for block in (32, 16, 8):
        for fmt in ("e8m0", "f16", "bf16"):
            p, s = oracle.mx_quantize(x, block, fmt)
            err[block, fmt] = float(np.mean(np.abs(oracle.dequantize_mx(p, s, block, fmt) - x)))
    for fmt in ("e8m0", "f16", "bf16"):
        assert err[8, fmt] < err[16, fmt] < err[32, fmt]
    for block in (32, 16, 8):
        assert err[block, "f16"] < err[block, "e8m0"]
        assert err[block, "bf16"] < err[block, "e8m0"]


@pytest.mark.parametrize("block,fmt", [(16, "e8m0"), (8, "bf16"), (32, "f16")])
def test_gemm_of_the_dequantised_operands_is_exact(block, fmt):
    a = sample(21, 5, 64)
    b = sample(22, 3, 64)
    qa, sa = oracle.mx_quantize(a, block, fmt)
    qb, sb = oracle.mx_quantize(b, block, fmt)
    d, s = oracle.gemm_mx(qa, sa, qb, sb, block, fmt)
    ca, cb = nibbles(qa), nibbles(qb)

    def val(codes, scales, r, k):
        c = int(codes[r, k])
        v = Fraction(E2M1[c & 7]) * (-1 if c & 8 else 1)
        sc = int(scales[r, k // block])
        return v * (Fraction(2) ** (sc - 127) if fmt == "e8m0" else Fraction(scale_value(sc, fmt)))

    for i in range(5):
        for j in range(3):
            terms = [val(ca, sa, i, k) * val(cb, sb, j, k) for k in range(64)]
            exact = sum(terms)
            mag = sum(abs(t) for t in terms)
            assert abs(Fraction(d[i, j]) - exact) <= mag * Fraction(1, 2 ** 50)
            assert abs(Fraction(s[i, j]) - mag) <= mag * Fraction(1, 2 ** 50)
