"""Pins of the oracle's quantisers: invariants the definition implies, worked
tiles, and properties checked by brute force.  CPU only."""
import numpy as np

import oracle
import workloads


def _ulp32(x):
    x = np.abs(np.float32(x))
    return float(np.nextafter(x, np.float32(np.inf)) - x)


def test_fp8_tile_worked_example():
    # one 128 x 32 tile whose maximum is 896: s = 896 / 448 = 2 exactly
    x = np.zeros((128, 32), dtype=np.float32)
    x[0, 0] = 896.0
    x[5, 7] = -3.0          # -3 / 2 = -1.5   -> E4M3 0xBC
    x[127, 31] = 0.3        # 0.15 -> nearest E4M3 0.15625 = 1.25 * 2^-3 (0x22)
    x[64, 16] = -0.0
    codes, scales = oracle.fp8_quantize(x, "e4m3")
    assert scales.shape == (1, 1) and scales[0, 0] == 2.0
    assert codes[0, 0] == 0x7E and codes[5, 7] == 0xBC and codes[127, 31] == 0x22
    assert codes[64, 16] == 0x80 and codes[1, 1] == 0x00


def test_fp8_all_zero_tile_has_unit_scale():
    x = np.zeros((130, 64), dtype=np.float32)
    x[129, 40] = 1.0                      # only the second K block of the last tile-row
    codes, scales = oracle.fp8_quantize(x, "e4m3")
    assert scales.shape == (2, 2)
    assert scales[0, 0] == 1.0 and scales[0, 1] == 1.0 and scales[1, 0] == 1.0
    assert scales[1, 1] == np.float32(1.0) / np.float32(448.0)
    assert codes[129, 40] == 0x7E


def _check_fp8_invariants(x, fmt, codes, scales, tile_rows=128):
    F = 448.0 if fmt == "e4m3" else 57344.0
    t = oracle.decode_table(fmt)
    rows, k = x.shape
    for ti in range(scales.shape[0]):
        for tj in range(scales.shape[1]):
            blk = x[ti * tile_rows:(ti + 1) * tile_rows, tj * 32:(tj + 1) * 32].astype(np.float64)
            cb = codes[ti * tile_rows:(ti + 1) * tile_rows, tj * 32:(tj + 1) * 32]
            s = float(scales[ti, tj])
            amax = np.max(np.abs(blk))
            if amax == 0:
                assert s == 1.0 and np.all(t[cb] == 0)
                continue
            # s is the FP32 value nearest to amax / F
            assert abs(s - amax / F) <= 0.5 * _ulp32(s)
            # the tile maximum lands on the format maximum
            i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert abs(t[cb[i]]) == F and np.sign(t[cb[i]]) == np.sign(blk[i])
            # every code is within half a code spacing of x / s (relative to the
            # local spacing of the format), and has the sign of x
            deq = t[cb]
            y = blk / s
            # neighbours of deq in the table bound the rounding error
            pos = np.unique(np.abs(t[np.isfinite(t)]))   # 0 counted once
            idx = np.searchsorted(pos, np.abs(deq))
            lo = pos[np.maximum(idx - 1, 0)]
            hi = pos[np.minimum(idx + 1, pos.size - 1)]
            err = np.abs(np.abs(y) - np.abs(deq))
            spacing = np.maximum(np.abs(deq) - lo, hi - np.abs(deq))
            assert np.all(err <= 0.5 * spacing + np.abs(y) * 2.0 ** -23)
            nz = deq != 0
            assert np.all(np.sign(deq[nz]) == np.sign(y[nz]))


def test_fp8_quantize_invariants_random_ragged():
    x = workloads.normal(11, 300, 96) * np.float32(3.0)
    x[:, 40:45] *= np.float32(1e-3)
    codes, scales = oracle.fp8_quantize(x, "e4m3")
    assert codes.shape == (300, 96) and scales.shape == (3, 3)
    _check_fp8_invariants(x, "e4m3", codes, scales)
    xl = workloads.laplace(12, 256, 64, 1e-3)
    codes, scales = oracle.fp8_quantize(xl, "e5m2")
    _check_fp8_invariants(xl, "e5m2", codes, scales)


def test_fp8_quantize_reconstruction_error_bound():
    """|deq - x| <= half an E4M3 spacing times s: relative 2^-4 for normals."""
    x = workloads.normal(13, 256, 256)
    codes, scales = oracle.fp8_quantize(x, "e4m3")
    deq = oracle.dequantize("e4m3", codes, scales)
    s_full = np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 32, 1)
    y = np.abs(x.astype(np.float64)) / s_full
    normal = y >= 2.0 ** -6
    rel = np.abs(deq - x)[normal] / np.abs(x.astype(np.float64))[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 2 ** -16)
    sub = ~normal
    assert np.all(np.abs(deq - x)[sub] <= 2.0 ** -10 * s_full[sub] * (1 + 2 ** -16))


def test_mxfp4_block_invariants():
    x = workloads.normal(21, 64, 256)
    x[3, :32] = 0.0                        # an all-zero block
    x[4, 32:64] *= np.float32(1e-30)       # a tiny block
    packed, scales = oracle.mxfp4_quantize(x)
    t4 = oracle.decode_table("e2m1")
    assert packed.shape == (64, 128) and scales.shape == (64, 8)
    lo = (packed & 0xF).astype(int)
    hi = (packed >> 4).astype(int)
    nib = np.empty((64, 256), dtype=int)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    for r in range(64):
        for b in range(8):
            blk = x[r, b * 32:(b + 1) * 32].astype(np.float64)
            e = int(scales[r, b]) - 127
            amax = np.max(np.abs(blk))
            if amax == 0:
                assert e == 0
                assert np.all(t4[nib[r, b * 32:(b + 1) * 32]] == 0)
                continue
            assert 6.0 * 2.0 ** e >= amax and (e == -127 or 6.0 * 2.0 ** (e - 1) < amax)
            if e > -127:
                assert 3.0 < amax * 2.0 ** -e <= 6.0
                i = np.argmax(np.abs(blk))
                assert abs(t4[nib[r, b * 32 + i]]) in (3.0, 4.0, 6.0)
            # each element is a nearest E2M1 value of x * 2^-e
            y = blk * 2.0 ** -e
            mags = t4[:8]
            got = np.abs(t4[nib[r, b * 32:(b + 1) * 32]])
            best = np.min(np.abs(mags[None, :] - np.abs(y)[:, None]), axis=1)
            assert np.all(np.abs(got - np.abs(y)) == best)


def test_mxfp4_packing_low_nibble_first():
    # a row whose elements are exactly E2M1 values with amax 6 -> e = 0
    vals = np.array([0.5, 6.0, -1.0, 3.0] + [0.0] * 28, dtype=np.float32)[None, :]
    packed, scales = oracle.mxfp4_quantize(vals)
    assert scales[0, 0] == 127
    assert packed[0, 0] == (0x1 | (0x7 << 4))       # 0.5 low, 6 high
    assert packed[0, 1] == (0xA | (0x5 << 4))       # -1 low, 3 high


# fl32(x / s) lands exactly on an E4M3 rounding midpoint, while x * fl32(1 / s)
# lands one FP32 step off it, towards the odd neighbour.  The quantiser divides
# (the pages divide each element by the scale), so the tie goes to the even
# code.  Bit patterns of the codes from the E4M3 definition (3 mantissa bits:
# 8 values per binade): 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A, 3.0 = 0x44,
# 3.25 = 0x45, 96 = 0x6C, 104 = 0x6D.
# (amax bits, x bits, midpoint, even code, odd code); cases found by a search
# over random tiles in numpy float32.
DIVISION_TIES = [
    (0x4178B033, 0x3D16FD44, 1.0625, 0x38, 0x39),
    (0x4BC1FA3E, 0x4783A0AA, 1.1875, 0x3A, 0x39),
    (0x3CED1854, 0x3BD3B127, 100.0, 0x6C, 0x6D),
    (0x3F4D4E11, 0x3BB74ED9, 3.125, 0x44, 0x45),
]


def test_fp8_quotient_is_a_division_not_a_reciprocal_product():
    for amax_bits, x_bits, mid, even, odd in DIVISION_TIES:
        amax = np.array([amax_bits], dtype=np.uint32).view(np.float32)[0]
        x = np.array([x_bits], dtype=np.uint32).view(np.float32)[0]
        s = np.float32(amax / np.float32(448.0))
        assert np.float32(x / s) == np.float32(mid)                       # an exact tie
        assert np.float32(x * np.float32(np.float32(1.0) / s)) != np.float32(mid)
        tile = np.zeros((128, 32), dtype=np.float32)
        tile[0, 0] = amax
        tile[1, 0] = x
        tile[2, 0] = -x
        codes, scales = oracle.fp8_quantize(tile, "e4m3")
        assert scales[0, 0] == s
        assert codes[1, 0] == even and codes[2, 0] == (even | 0x80), (hex(codes[1, 0]), hex(odd))
