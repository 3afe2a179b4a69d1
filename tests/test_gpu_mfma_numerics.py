"""The matrix-core dot-product model against the hardware, bit for bit (gfx950).

Every case runs ONE MFMA instruction through the test probe (tests/mfma_probe)
and compares its FP32 result with oracle/mfma_model.py:
  1. the hand-derived feature vectors (tests/mfma_features.py), against both
     the derived value and the model;
  2. feature sweeps for every instruction the GEMM kernels use: the distance of
     a small product below a large one at several K positions, the accumulator
     above or below the products, cancellations within and across groups;
  3. seeded random dot products (uniform codes including subnormals, sparse
     vectors, exact cancellations, random block scales and accumulators).
This is the randomised test-and-refine loop of "Exact models of AMD matrix
cores" (section 3), run here as a regression check.
"""
import math
import zlib

import numpy as np
import pytest

from gpu_common import say
from mfma_features import VECTORS
import mfma_probe as P
from oracle import mfma_model as M

pytestmark = pytest.mark.gpu

SELECTOR = {
    "v_mfma_f32_32x32x16_fp8_fp8": P.FP8_FP8,
    "v_mfma_f32_32x32x16_fp8_bf8": P.FP8_BF8,
    "v_mfma_f32_32x32x16_bf8_fp8": P.BF8_FP8,
    "v_mfma_f32_32x32x16_bf8_bf8": P.BF8_BF8,
    "v_mfma_f32_32x32x16_bf16": P.BF16,
    "v_mfma_scale_f32_32x32x64_f8f6f4.e2m1": P.SCALE_FP4,
    "v_mfma_scale_f32_32x32x64_f8f6f4.e4m3": P.SCALE_E4M3,
    "v_mfma_scale_f32_32x32x64_f8f6f4.e5m2": P.SCALE_E5M2,
    "v_mfma_f32_32x32x64_f8f6f4.e4m3": P.K64_E4M3,
    "v_mfma_f32_32x32x64_f8f6f4.e5m2": P.K64_E5M2,
}
NAMES = list(SELECTOR)


def bits(v):
    return np.asarray(v, dtype=np.float32).view(np.uint32)


def pack(fmt, codes):
    """K codes per row -> probe operand storage."""
    codes = np.asarray(codes)
    if fmt == "e2m1":
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    if fmt == "bf16":
        return codes.astype(np.uint16)
    return codes.astype(np.uint8)


def run_both(instr, a_codes, b_codes, c, sa=None, sb=None, label=""):
    """Hardware and model results for rows of K codes; returns (hw, model) FP32 arrays."""
    a_fmt, b_fmt, K, scaled, _ = M.INSTRUCTIONS[instr]
    a_codes = np.asarray(a_codes, dtype=np.int64)
    b_codes = np.asarray(b_codes, dtype=np.int64)
    c = np.asarray(c, dtype=np.float32)
    say(f"mfma probe {instr} {label}: {len(c)} dot products")
    hw = P.dot(SELECTOR[instr], pack(a_fmt, a_codes), pack(b_fmt, b_codes), c,
               None if sa is None else np.asarray(sa, np.uint8), None if sb is None else np.asarray(sb, np.uint8))
    model = np.empty(len(c), dtype=np.float32)
    for i in range(len(c)):
        model[i] = M.mfma_dot(instr, a_codes[i].tolist(), b_codes[i].tolist(), float(c[i]),
                              None if sa is None else list(sa[i]), None if sb is None else list(sb[i]))
    return hw, model


def assert_same(instr, hw, model, a, b, c, label):
    bad = np.nonzero(bits(hw) != bits(model))[0]
    if len(bad):
        i = int(bad[0])
        raise AssertionError(
            f"{instr} {label}: {len(bad)}/{len(hw)} results differ from the model; first case {i}: "
            f"hw {hw[i]!r} ({bits(hw[i]):08x}) model {model[i]!r} ({bits(model[i]):08x}) "
            f"a={list(a[i])} b={list(b[i])} c={c[i]!r}")


# ---------------------------------------------------------------- 1. derived vectors
def vector_codes(instr, prods):
    a_fmt, b_fmt, K, _, _ = M.INSTRUCTIONS[instr]
    a, b = [0] * K, [0] * K
    for k, (x, y) in prods.items():
        a[k], b[k] = P.encode(a_fmt, x), P.encode(b_fmt, y)
    return a, b


@pytest.mark.parametrize("instr", sorted({v[1] for v in VECTORS}))
def test_derived_feature_vectors_on_hardware(instr):
    vecs = [v for v in VECTORS if v[1] == instr]
    a, b = zip(*[vector_codes(instr, v[2]) for v in vecs])
    c = [v[3] for v in vecs]
    sa = sb = None
    if M.INSTRUCTIONS[instr][3]:
        sa = [v[4][0] for v in vecs]
        sb = [v[4][1] for v in vecs]
    hw, model = run_both(instr, a, b, c, sa, sb, "derived vectors")
    for v, h, m in zip(vecs, hw, model):
        assert bits(h) == bits(np.float32(v[5])), f"{v[0]}: hardware {h!r}, derived {v[5]!r}"
        assert bits(h) == bits(m), f"{v[0]}: hardware {h!r}, model {m!r}"


# ---------------------------------------------------------------- 2. sweeps
_BF16_SIGNIFICANDS = (1.0, 1.25, 1.5, 1.75)


def values_of(fmt):
    if fmt == "bf16":
        return sorted(m * 2.0 ** e for m in _BF16_SIGNIFICANDS for e in range(-60, 60))
    table, _ = P._TABLES[fmt]
    return sorted(v for v in table.values() if v > 0)


def factor(a_fmt, b_fmt, v):
    """Exact operands x (a_fmt) and y (b_fmt) with x y = v, or None."""
    if v == 0:
        return 0.0, 0.0
    best = None
    for x in values_of(a_fmt):
        y = abs(v) / x
        if P.representable(b_fmt, y):
            score = abs(math.log2(x) - math.log2(abs(v)) / 2)
            if best is None or score < best[0]:
                best = (score, x, y)
    if best is None:
        return None
    return math.copysign(best[1], v), best[2]


def sweep_cases(instr):
    """(products {k: value}, c) cases probing alignment, groups, passes and c."""
    a_fmt, b_fmt, K, _, _ = M.INSTRUCTIONS[instr]
    E = 4 if a_fmt == "e2m1" else 16
    big = 2.0 ** E
    cases = []
    positions = [1, 7, 8, 15] + ([16, 31, 32, 40, 63] if K == 64 else [])
    for k in positions:
        for g in range(1, 41):
            for sgn in (1.0, -1.0):
                cases.append(({0: big, k: sgn * 2.0 ** (E - g)}, 0.0))
    for k in positions:                      # cancellation of two large products, small third term
        cases.append(({0: big, 1: -big, k: 2.0 ** (E - 30)}, 0.0))
        cases.append(({0: big, k: -big, 2 if k != 2 else 3: 2.0 ** (E - 30)}, 0.0))
    for g in range(-30, 31, 3):              # accumulator above and below the products
        for sgn in (1.0, -1.0):
            cases.append(({0: big}, sgn * 2.0 ** (E - g)))
            cases.append(({0: big, 1: 1.5 * 2.0 ** (E - 9)}, sgn * 1.75 * 2.0 ** (E - g)))
            cases.append(({0: -big, 8 % K: 2.0 ** (E - 20)}, sgn * big * (1 + 2.0 ** -g if g > 0 else 1)))
    return cases


def e2m1_sweep_cases():
    """E2M1 products span few binades, so the sweeps move the block scales:
    (operands {k: (a, b)}, c, a scale bytes, b scale bytes)."""
    cases = []
    pairs = [((1.0, 1.0), (1.0, 1.0)), ((6.0, 6.0), (0.5, 0.5)), ((4.0, 1.0), (-0.5, 0.5)),
             ((-6.0, 4.0), (1.5, 3.0))]
    for u in range(-26, 27, 2):               # block 0 scale 2^u against block 1 at 2^0
        for (p0, p1) in pairs:
            for k1 in (1, 8, 31, 32, 40, 63):
                for c in (0.0, 1.0, -(2.0 ** (u - 12)), 2.0 ** (u + 3), -0.375):
                    cases.append(({0: p0, k1: p1}, c, (127 + u, 127), (127, 127)))
        cases.append(({0: (4.0, 1.0), 1: (-4.0, 1.0), 32: (0.5, 0.5)}, 2.0 ** (u - 30), (127 + u, 127), (127, 127)))
        cases.append(({0: (1.0, 1.0), 32: (-1.0, 1.0), 33: (0.5, 0.5)}, 0.0, (127 + u, 127 + u), (127, 120)))
    return cases


@pytest.mark.parametrize("instr", NAMES)
def test_feature_sweeps_match_model(instr):
    a_fmt, b_fmt, K, scaled, _ = M.INSTRUCTIONS[instr]
    A, B, C, SA, SB = [], [], [], [], []
    if a_fmt == "e2m1":
        for ops, c, sa, sb in e2m1_sweep_cases():
            a, b = vector_codes(instr, ops)
            A.append(a)
            B.append(b)
            C.append(np.float32(c))
            SA.append(sa)
            SB.append(sb)
    else:
        for prods, c in sweep_cases(instr):
            a, b, ok = [0] * K, [0] * K, True
            for k, v in prods.items():
                f = factor(a_fmt, b_fmt, v)
                if f is None:
                    ok = False
                    break
                a[k], b[k] = P.encode(a_fmt, f[0]), P.encode(b_fmt, f[1])
            if ok:
                A.append(a)
                B.append(b)
                C.append(np.float32(c))
                SA.append((127, 127))
                SB.append((127, 127))
    assert len(A) > 200, f"only {len(A)} sweep cases are representable for {instr}"
    sa = np.asarray(SA, np.uint8) if scaled else None
    sb = np.asarray(SB, np.uint8) if scaled else None
    hw, model = run_both(instr, A, B, C, sa, sb, "sweeps")
    assert_same(instr, hw, model, np.asarray(A), np.asarray(B), C, "sweeps")


# ---------------------------------------------------------------- 3. random
def random_codes(rng, fmt, n, K):
    if fmt == "e4m3":
        c = rng.integers(0, 256, (n, K))
        c[(c & 0x7F) == 0x7F] ^= 1
    elif fmt == "e5m2":
        c = rng.integers(0, 256, (n, K))
        bad = (c & 0x7C) == 0x7C
        c[bad] &= 0xF3
    elif fmt == "e2m1":
        c = rng.integers(0, 16, (n, K))
    else:                                      # bf16 within 2^+-24
        c = (rng.integers(0, 2, (n, K)) << 15) | (rng.integers(127 - 24, 127 + 24, (n, K)) << 7) \
            | rng.integers(0, 128, (n, K))
    return c


def negate(fmt, codes):
    return codes ^ {"e4m3": 0x80, "e5m2": 0x80, "e2m1": 0x8, "bf16": 0x8000}[fmt]


@pytest.mark.parametrize("instr", NAMES)
def test_random_dot_products_match_model(instr):
    a_fmt, b_fmt, K, scaled, _ = M.INSTRUCTIONS[instr]
    rng = np.random.default_rng(zlib.crc32(instr.encode()))
    n = 6000
    a = random_codes(rng, a_fmt, n, K)
    b = random_codes(rng, b_fmt, n, K)
    third = n // 3
    sparse = rng.random((third, K)) < 0.6      # rows third..2 third: 60 % zero products
    a[third:2 * third][sparse] = 0
    # last third: exact cancellations -- product k + K/2 is minus product k
    h = K // 2
    a[2 * third:, h:] = negate(a_fmt, a[2 * third:, :h])
    b[2 * third:, h:] = b[2 * third:, :h]
    keep = rng.random((n - 2 * third, h)) < 0.3
    a[2 * third:, h:][keep] = random_codes(rng, a_fmt, int(keep.sum()), 1)[:, 0]
    cexp = rng.integers(-30, 31, n)
    c = ((rng.random(n) + 0.5) * np.exp2(cexp) * np.where(rng.random(n) < 0.5, -1, 1)).astype(np.float32)
    c[rng.random(n) < 0.25] = 0
    sa = sb = None
    if scaled:
        spread = 20 if a_fmt == "e2m1" else 12
        sa = rng.integers(127 - spread, 127 + spread, (n, 2)).astype(np.uint8)
        sb = rng.integers(127 - spread, 127 + spread, (n, 2)).astype(np.uint8)
    hw, model = run_both(instr, a, b, c, sa, sb, "random")
    assert not np.any(np.isnan(hw)), "probe left results unwritten"
    assert_same(instr, hw, model, a, b, c, "random")
