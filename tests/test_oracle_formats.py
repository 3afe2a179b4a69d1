"""Pins of the oracle's number formats against facts fixed outside the oracle:
values the pages print, independent library decodes/casts (torch CPU), closed
forms and exhaustive enumeration.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode(dtype):
    return torch.arange(256, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()


def same_or_both_nan(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.all((a == b) | (np.isnan(a) & np.isnan(b)))


# ---------------------------------------------------------------- decode tables

def test_e4m3_table_matches_torch_float8_e4m3fn():
    t = oracle.decode_table("e4m3")
    assert same_or_both_nan(t, torch_decode(torch.float8_e4m3fn))


def test_e4m3_page_facts():
    t = oracle.decode_table("e4m3")
    # max 448 ("Why grind FP8 GEMM on CDNA4", section 3.3), at S.1111.110
    assert np.nanmax(t) == 448.0 and t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    finite_nonneg = t[:0x80][~np.isnan(t[:0x80])]
    assert finite_nonneg.size == 127            # codes 0x00..0x7E
    assert np.all(np.diff(finite_nonneg) > 0)   # increasing with the code
    assert t[1] == 2.0 ** -9                    # smallest subnormal
    assert t[8] == 2.0 ** -6                    # smallest normal
    assert not np.any(np.isinf(t))              # no infinity in E4M3 FN


def test_e5m2_table_matches_torch_float8_e5m2():
    t = oracle.decode_table("e5m2")
    assert same_or_both_nan(t, torch_decode(torch.float8_e5m2))
    assert t[0x7B] == 57344.0 and t[0x7C] == math.inf and t[0xFC] == -math.inf
    assert t[1] == 2.0 ** -16


def test_e2m1_table_is_the_pages_list():
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        vals = [float(v) for line in f if not line.startswith("#") for v in line.split()]
    t = oracle.decode_table("e2m1")
    assert list(t[:8]) == vals
    assert list(t[8:]) == [-v for v in vals]
    assert t[7] == 6.0


def test_e8m0_powers_of_two():
    t = oracle.decode_table("e8m0")
    for c in range(255):
        m, e = math.frexp(t[c])
        assert m == 0.5 and t[c] == 2.0 ** (c - 127)
    assert math.isnan(t[255])
    assert same_or_both_nan(t, torch_decode(torch.float8_e8m0fnu))


# ---------------------------------------------------------------- encode

def _fp8_probe_values(fmt):
    """Every finite code value, its FP32 neighbours, every midpoint between
    consecutive codes and its neighbours, both signs, plus random values."""
    t = oracle.decode_table(fmt)
    top = 0x7E if fmt == "e4m3" else 0x7B
    pos = t[: top + 1]
    vals = list(pos)
    mids = (pos[:-1] + pos[1:]) / 2
    vals += list(mids)
    base = np.array(vals, dtype=np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    rng = np.random.default_rng(7)
    rnd = (rng.standard_normal(20000) * np.exp2(rng.integers(-18, 10, 20000))).astype(np.float32)
    allv = np.concatenate([base, up, dn, -base, -up, -dn, rnd])
    return allv[np.abs(allv.astype(np.float64)) <= pos[-1]]


@pytest.mark.parametrize("fmt,dtype", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_encode_matches_torch_cast_in_range(fmt, dtype):
    v = _fp8_probe_values(fmt)
    ours = oracle.encode(fmt, v.astype(np.float64))
    ref = torch.from_numpy(v).to(dtype).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{fmt}: {v[bad[:5]]} -> {ours[bad[:5]]} vs {ref[bad[:5]]}"


def test_fp8_encode_saturates_and_keeps_sign_of_zero():
    assert oracle.encode("e4m3", [449.0, 463.9, 464.0, 480.0, 1e6, 1e30]).tolist() == [0x7E] * 6
    assert oracle.encode("e4m3", [-449.0, -1e6]).tolist() == [0xFE] * 2
    assert oracle.encode("e5m2", [57345.0, 61440.0, 1e9]).tolist() == [0x7B] * 3
    assert oracle.encode("e5m2", [-1e9]).tolist() == [0xFB]
    assert oracle.encode("e4m3", [0.0, -0.0]).tolist() == [0x00, 0x80]
    assert oracle.encode("e5m2", [0.0, -0.0]).tolist() == [0x00, 0x80]
    assert oracle.encode("e2m1", [0.0, -0.0]).tolist() == [0x0, 0x8]


def test_e2m1_encode_ties_to_even_by_hand():
    # midpoints between consecutive E2M1 magnitudes go to the code whose last bit is 0
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6]          # 0, 1, 1, 2, 2, 4, 4
    assert oracle.encode("e2m1", mids).tolist() == want
    assert oracle.encode("e2m1", [-m for m in mids]).tolist() == [w | 0x8 for w in want]
    assert oracle.encode("e2m1", [0.2499, 0.2501, 5.001, 6.0, 7.0, 100.0]).tolist() == \
        [0x0, 0x1, 0x7, 0x7, 0x7, 0x7]


def test_encode_is_nearest_exhaustively_on_a_dense_grid():
    """Brute force: on a dense grid the chosen code is a nearest representable
    value (saturating), for all three element formats."""
    for fmt, top in (("e4m3", 0x7E), ("e5m2", 0x7B), ("e2m1", 0x7)):
        t = oracle.decode_table(fmt)
        pos = t[: top + 1]
        grid = np.linspace(0, pos[-1] * 1.05, 40001)
        codes = oracle.encode(fmt, grid)
        got = t[codes]
        best = np.min(np.abs(pos[None, :] - np.minimum(grid, pos[-1])[:, None]), axis=1)
        assert np.all(np.abs(got - np.minimum(grid, pos[-1])) == best)


def test_mx_exponent_is_smallest_covering_power():
    rng = np.random.default_rng(3)
    for amax in list(np.exp2(rng.uniform(-120, 120, 2000))) + [6.0, 3.0, 12.0, 1.5, 6.0000001]:
        e = oracle.mx_exponent(float(amax))
        assert 6.0 * 2.0 ** e >= amax
        assert 6.0 * 2.0 ** (e - 1) < amax
    assert oracle.mx_exponent(1e-45) == -127        # clamped at the bottom of E8M0
    assert oracle.mx_exponent(3.4e38) == 126
