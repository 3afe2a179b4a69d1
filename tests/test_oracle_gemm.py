"""Pins of the oracle's GEMM: the pages' two FP8 dot examples (exact values),
exact rational brute force with operands decoded by an independent library
(torch) rather than the oracle's tables, and a closed form.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_dot_examples():
    out = []
    with open(os.path.join(GOLDEN, "dot_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            a, b, exact, bits, h100 = [p.strip() for p in line.split("|")]
            out.append(([float(v) for v in a.split()], [float(v) for v in b.split()],
                        float(exact), int(bits, 16), int(h100, 16)))
    return out


def torch_codes(vals, dtype=torch.float8_e4m3fn):
    t = torch.tensor(np.asarray(vals, dtype=np.float32))
    c = t.to(dtype)
    assert torch.equal(c.to(torch.float32), t), "value not exactly representable"
    return c.view(torch.uint8).numpy()


def test_dot_examples_exact():
    for a, b, exact, bits, _ in load_dot_examples():
        A = np.zeros((128, 32), dtype=np.uint8)
        B = np.zeros((128, 32), dtype=np.uint8)
        A[0, : len(a)] = torch_codes(a)
        B[0, : len(b)] = torch_codes(b)
        one = np.ones((1, 1), dtype=np.float32)
        d, s = oracle.gemm_rows("e4m3", A, one, "e4m3", B, one, 0, 1)
        assert d[0, 0] == exact
        assert np.float32(d[0, 0]).view(np.uint32) == bits
        assert s[0, 0] == sum(abs(x * y) for x, y in zip(a, b))
        assert np.all(d[0, 1:] == 0)


def _torch_table(fmt):
    dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]
    return torch.arange(256, dtype=torch.uint8).view(dt).to(torch.float64).numpy()


def _finite_codes(rng, fmt, shape):
    t = _torch_table(fmt)
    ok = np.nonzero(np.isfinite(t))[0].astype(np.uint8)
    return ok[rng.integers(0, ok.size, size=shape)]


def _rand_scales(rng, shape):
    # random positive FP32 with full 24-bit significands over a wide range
    return (rng.uniform(1, 2, shape) * np.exp2(rng.integers(-20, 10, shape))).astype(np.float32)


def _exact_fp8_dot(ta, tb, A, sa, B, sb, i, j, K):
    acc = Fraction(0)
    mag = Fraction(0)
    for k in range(K):
        x = Fraction(ta[A[i, k]]) * Fraction(float(sa[i // 128, k // 32]))
        y = Fraction(tb[B[j, k]]) * Fraction(float(sb[j // 128, k // 32]))
        acc += x * y
        mag += abs(x * y)
    return acc, mag


def test_fp8_gemm_brute_force_exact_rationals():
    rng = np.random.default_rng(5)
    for a_fmt, b_fmt in (("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")):
        M, N, K = 260, 200, 96
        A = _finite_codes(rng, a_fmt, (M, K))
        B = _finite_codes(rng, b_fmt, (N, K))
        sa = _rand_scales(rng, ((M + 127) // 128, K // 32))
        sb = _rand_scales(rng, ((N + 127) // 128, K // 32))
        ii = np.array([0, 1, 127, 128, 129, 255, 256, 259, 77, 200])
        jj = np.array([0, 199, 128, 127, 5, 130, 199, 0, 64, 3])
        d, s = oracle.gemm_points(a_fmt, A, sa, b_fmt, B, sb, ii, jj)
        ta, tb = _torch_table(a_fmt), _torch_table(b_fmt)
        for p in range(ii.size):
            ex, mag = _exact_fp8_dot(ta, tb, A, sa, B, sb, ii[p], jj[p], K)
            assert abs(Fraction(d[p]) - ex) <= Fraction(2) ** -40 * mag
            assert abs(Fraction(s[p]) - mag) <= Fraction(2) ** -40 * mag
        # the row routine agrees with the point routine
        dr, sr = oracle.gemm_rows(a_fmt, A, sa, b_fmt, B, sb, 0, M)
        assert np.array_equal(dr[ii, jj], d) and np.array_equal(sr[ii, jj], s)


def test_fp8_gemm_constant_tiles_closed_form():
    # every A code is 1.5 (0x3C), every B code is 2.0 (0x40): D = sum_kb 32*1.5*2*sa*sb
    rng = np.random.default_rng(9)
    M, N, K = 256, 128, 128
    A = np.full((M, K), 0x3C, dtype=np.uint8)
    B = np.full((N, K), 0x40, dtype=np.uint8)
    sa = _rand_scales(rng, (2, 4))
    sb = _rand_scales(rng, (1, 4))
    d, s = oracle.gemm_rows("e4m3", A, sa, "e4m3", B, sb)
    for ti in range(2):
        want = sum(32 * 1.5 * 2.0 * float(sa[ti, kb]) * float(sb[0, kb]) for kb in range(4))
        assert np.allclose(d[ti * 128:(ti + 1) * 128], want, rtol=2 ** -44, atol=0)   # K * 2^-53 rounding of fp64 sums
        assert np.array_equal(d[ti * 128:(ti + 1) * 128], s[ti * 128:(ti + 1) * 128])


def test_mxfp4_gemm_brute_force_exact_rationals():
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        mags = [Fraction(v) for line in f if not line.startswith("#") for v in line.split()]
    e2m1 = mags + [-m for m in mags]                 # codes 8..15 are the negatives
    rng = np.random.default_rng(17)
    M, N, K = 40, 24, 96
    A = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    B = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sa = rng.integers(110, 145, size=(M, K // 32), dtype=np.uint8)
    sb = rng.integers(110, 145, size=(N, K // 32), dtype=np.uint8)
    d, s = oracle.gemm_rows("mxfp4", A, sa, "mxfp4", B, sb)

    def elem(P, S, r, k):
        byte = int(P[r, k // 2])
        nib = byte & 0xF if k % 2 == 0 else byte >> 4
        return e2m1[nib] * Fraction(2) ** (int(S[r, k // 32]) - 127)

    for i in range(0, M, 7):
        for j in range(0, N, 5):
            terms = [elem(A, sa, i, k) * elem(B, sb, j, k) for k in range(K)]
            ex = sum(terms)
            mag = sum(abs(t) for t in terms)
            assert abs(Fraction(d[i, j]) - ex) <= Fraction(2) ** -40 * mag
            assert abs(Fraction(s[i, j]) - mag) <= Fraction(2) ** -40 * mag
