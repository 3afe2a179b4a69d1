"""Pins of the oracle's FP8 scale granularities (per row, per tensor) and of the
granular GEMM, CPU only.  "Why grind FP8 GEMM on CDNA4" (section 3.3) weighs
per-row, per-column, per-tile and per-matrix scales; the per-row scale of a B
operand stored N x K is its per-column scale.

The pins are fixed outside the granular code: a hand-worked example, the
already pinned per-tile quantiser in the cases where the mathematics forces
the same result, exact invariances, and exact rational brute force with
operands decoded by torch."""
import fractions
import math

import numpy as np
import pytest
import torch

import oracle

F = fractions.Fraction
TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def torch_decode(fmt, codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(TORCH_FP8[fmt])
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- worked example
def test_worked_example_per_row_and_per_tensor():
    """Row 0 has amax 448 (s = 1), row 1 amax 896 (s = 2); per tensor s = 2.
    Codes worked by hand from the E4M3 fields (bias 7, three mantissa bits):
    448 = 0x7E, 224 = 1.75 2^7 = 0x76, 112 = 0x6E, 1.5 = 0x3C, 0.75 = 0x34,
    0.25 = 0x28, 2^-7 = subnormal 4 2^-9 = 0x04, 2^-8 = 0x02, sign bit 0x80."""
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, :4] = [448.0, -224.0, 1.5, 2.0 ** -7]
    x[1, :3] = [896.0, 3.0, -0.5]
    q, s = oracle.fp8_quantize_granular(x, "e4m3", "row")
    assert s.tolist() == [1.0, 2.0]
    assert q[0, :4].tolist() == [0x7E, 0xF6, 0x3C, 0x04]
    assert q[1, :3].tolist() == [0x7E, 0x3C, 0xA8]
    assert not q[0, 4:].any() and not q[1, 3:].any()
    q, s = oracle.fp8_quantize_granular(x, "e4m3", "tensor")
    assert s.tolist() == [2.0]
    assert q[0, :4].tolist() == [0x76, 0xEE, 0x34, 0x02]
    assert q[1, :3].tolist() == [0x7E, 0x3C, 0xA8]


def test_all_zero_operand_has_unit_scale():
    for g in ("row", "tensor"):
        q, s = oracle.fp8_quantize_granular(np.zeros((3, 32), np.float32), "e5m2", g)
        assert not q.any() and np.all(s == 1.0)


# ---------------------------------------------------------------- agreement with the tile quantiser
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_per_tensor_of_one_tile_is_the_tile_quantiser(fmt):
    rng = np.random.default_rng(3)
    for rows in (1, 7, 128):
        x = (rng.standard_normal((rows, 32)) * 10.0 ** rng.integers(-3, 4)).astype(np.float32)
        qt, st = oracle.fp8_quantize(x, fmt)
        qg, sg = oracle.fp8_quantize_granular(x, fmt, "tensor")
        assert np.array_equal(qt, qg) and st.reshape(1)[0] == sg[0]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_per_row_with_k_32_is_a_tile_of_copies(fmt):
    """A tile made of 128 copies of one 32-wide row has that row's amax, so the
    tile quantiser gives the row's per-row codes in every copy."""
    rng = np.random.default_rng(4)
    x = (rng.laplace(size=(16, 32)) * 0.01).astype(np.float32)
    qr, sr = oracle.fp8_quantize_granular(x, fmt, "row")
    for i in range(x.shape[0]):
        qt, st = oracle.fp8_quantize(np.tile(x[i:i + 1], (128, 1)), fmt)
        assert np.all(qt == qr[i]) and st[0, 0] == sr[i]


# ---------------------------------------------------------------- invariances
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_power_of_two_row_scaling(fmt):
    """Multiplying a row by 2^j leaves its codes alone and multiplies its scale
    by 2^j (all values stay normal FP32); other rows are untouched."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 96)).astype(np.float32)
    q0, s0 = oracle.fp8_quantize_granular(x, fmt, "row")
    j = rng.integers(-20, 21, size=9)
    q1, s1 = oracle.fp8_quantize_granular((x * np.exp2(j)[:, None]).astype(np.float32), fmt, "row")
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, (s0 * np.exp2(j)).astype(np.float32))
    qt0, st0 = oracle.fp8_quantize_granular(x, fmt, "tensor")
    qt1, st1 = oracle.fp8_quantize_granular((x * np.float32(2.0 ** -13)).astype(np.float32), fmt, "tensor")
    assert np.array_equal(qt0, qt1) and st1[0] == np.float32(st0[0] * 2.0 ** -13)


def test_rows_are_independent_and_permutable():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((12, 64)).astype(np.float32)
    q, s = oracle.fp8_quantize_granular(x, "e4m3", "row")
    perm = rng.permutation(12)
    qp, sp = oracle.fp8_quantize_granular(x[perm], "e4m3", "row")
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])
    y = x.copy()
    y[3] *= 1000.0
    qy, sy = oracle.fp8_quantize_granular(y, "e4m3", "row")
    keep = np.arange(12) != 3
    assert np.array_equal(qy[keep], q[keep]) and np.array_equal(sy[keep], s[keep])
    qt, st = oracle.fp8_quantize_granular(x, "e4m3", "tensor")
    cols = rng.permutation(64)
    qtp, stp = oracle.fp8_quantize_granular(x[perm][:, cols], "e4m3", "tensor")
    assert np.array_equal(qtp, qt[perm][:, cols]) and stp[0] == st[0]


@pytest.mark.parametrize("g", ["row", "tensor"])
def test_the_largest_magnitude_codes_to_the_format_maximum(g):
    rng = np.random.default_rng(8)
    for fmt, top in (("e4m3", 448.0), ("e5m2", 57344.0)):
        x = (rng.standard_normal((6, 160)) * 3.0).astype(np.float32)
        q, s = oracle.fp8_quantize_granular(x, fmt, g)
        vals = torch_decode(fmt, q)
        if g == "row":
            for i in range(6):
                j = int(np.argmax(np.abs(x[i])))
                assert abs(vals[i, j]) == top
        else:
            i, j = np.unravel_index(int(np.argmax(np.abs(x))), x.shape)
            assert abs(vals[i, j]) == top


# ---------------------------------------------------------------- the granular GEMM
def exact_dot(fmt_a, qa_row, sa, fmt_b, qb_row, sb):
    av = torch_decode(fmt_a, qa_row)
    bv = torch_decode(fmt_b, qb_row)
    tot = sum((F(float(x)) * F(float(y)) for x, y in zip(av, bv)), F(0))
    return tot * F(float(sa)) * F(float(sb))


def scale_of(g, s, i, k):
    s = np.asarray(s)
    if g == "row":
        return s[i]
    if g == "tensor":
        return s[0]
    return s[i // 128, k // 32]


@pytest.mark.parametrize("ga,gb", [("row", "row"), ("row", "tensor"), ("tensor", "tensor"), ("tensor", "row")])
def test_granular_gemm_brute_force(ga, gb):
    rng = np.random.default_rng(9)
    M, N, K = 40, 24, 96
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = (rng.laplace(size=(N, K)) * 1e-3).astype(np.float32)
    qa, sa = oracle.fp8_quantize_granular(a, "e4m3", ga)
    qb, sb = oracle.fp8_quantize_granular(b, "e5m2", gb)
    d, smag = oracle.gemm_granular("e4m3", qa, sa, ga, "e5m2", qb, sb, gb)
    for i, j in [(0, 0), (39, 23), (17, 5), (3, 19), (25, 11), (38, 1)]:
        ex = exact_dot("e4m3", qa[i], scale_of(ga, sa, i, 0), "e5m2", qb[j], scale_of(gb, sb, j, 0))
        assert abs(F(float(d[i, j])) - ex) <= F(2) ** -45 * F(float(smag[i, j]))


def test_tile_granularity_matches_the_pinned_tile_gemm():
    rng = np.random.default_rng(10)
    a = rng.standard_normal((200, 96)).astype(np.float32)
    b = rng.standard_normal((150, 96)).astype(np.float32)
    qa, sa = oracle.fp8_quantize(a, "e4m3")
    qb, sb = oracle.fp8_quantize(b, "e4m3")
    d1, s1 = oracle.gemm_rows("e4m3", qa, sa, "e4m3", qb, sb)
    d2, s2 = oracle.gemm_granular("e4m3", qa, sa, "tile", "e4m3", qb, sb, "tile")
    assert np.all(np.abs(d1 - d2) <= 2.0 ** -45 * s1) and np.allclose(s1, s2, rtol=2.0 ** -45, atol=0)
