"""Quantisation parity: the HIP kernels' codes and scales are byte-equal to the
oracle's, on edge values, ragged shapes, degenerate inputs and every workload
at full size.  Runs through the C ABI (the Python binding)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_common import from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def bsfp8():
    import block_scaled_precision_fp8_amd as b
    return b


def gpu_fp8(x, fmt, ld=None):
    import torch
    b = bsfp8()
    if ld is None:
        xd = to_dev(x)
    else:   # padded rows: leading dimension ld > k
        buf = np.zeros((x.shape[0], ld), dtype=np.float32)
        buf[:, : x.shape[1]] = x
        xd = to_dev(buf)[:, : x.shape[1]]
    codes, scales = b.fp8_quantize(xd, fmt)
    torch.cuda.synchronize()
    return from_dev(codes), from_dev(scales)


def gpu_fp8_t(xt, fmt, ld=None):
    """Transposing quantiser on xt (k x rows, as stored); returns codes and
    scales of xt^T."""
    import torch
    b = bsfp8()
    if ld is None:
        xd = to_dev(xt)
    else:
        buf = np.zeros((xt.shape[0], ld), dtype=np.float32)
        buf[:, : xt.shape[1]] = xt
        xd = to_dev(buf)[:, : xt.shape[1]]
    codes, scales = b.fp8_quantize_transposed(xd, fmt)
    torch.cuda.synchronize()
    return from_dev(codes), from_dev(scales)


def assert_fp8_t_equal(x, fmt, ld=None, label=""):
    """x is rows x k (the operand as the GEMM wants it); the GPU is given its
    transpose, stored k x rows, and must produce exactly the oracle's
    quantisation of x."""
    xt = np.ascontiguousarray(x.T)
    say(f"fp8_quantize_transposed {fmt} stored {xt.shape} ld={ld} {label}")
    c, s = gpu_fp8_t(xt, fmt, ld)
    rc, rs = oracle.fp8_quantize(x, fmt)
    assert s.view(np.uint32).tobytes() == rs.view(np.uint32).tobytes(), f"{label}: scales differ"
    bad = np.nonzero(c != rc)
    assert bad[0].size == 0, (f"{label}: {bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}:"
                              f" x={x[bad[0][0], bad[1][0]]!r} gpu={c[bad][0]:#x} oracle={rc[bad][0]:#x}")


def gpu_mx(x, ld=None):
    import torch
    b = bsfp8()
    if ld is None:
        xd = to_dev(x)
    else:
        buf = np.zeros((x.shape[0], ld), dtype=np.float32)
        buf[:, : x.shape[1]] = x
        xd = to_dev(buf)[:, : x.shape[1]]
    packed, scales = b.mxfp4_quantize(xd)
    torch.cuda.synchronize()
    return from_dev(packed), from_dev(scales)


def assert_fp8_equal(x, fmt, ld=None, label=""):
    say(f"fp8_quantize {fmt} {x.shape} ld={ld} {label}")
    c, s = gpu_fp8(x, fmt, ld)
    rc, rs = oracle.fp8_quantize(x, fmt)
    assert s.view(np.uint32).tobytes() == rs.view(np.uint32).tobytes(), f"{label}: scales differ"
    bad = np.nonzero(c != rc)
    assert bad[0].size == 0, (f"{label}: {bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}:"
                              f" x={x[bad[0][0], bad[1][0]]!r} gpu={c[bad][0]:#x} oracle={rc[bad][0]:#x}")


def assert_mx_equal(x, ld=None, label=""):
    say(f"mxfp4_quantize {x.shape} ld={ld} {label}")
    p, s = gpu_mx(x, ld)
    rp, rs = oracle.mxfp4_quantize(x)
    assert np.array_equal(s, rs), f"{label}: scales differ"
    bad = np.nonzero(p != rp)
    assert bad[0].size == 0, f"{label}: {bad[0].size} packed bytes differ"


def fp8_edge_tile(fmt):
    """A 128 x 128 block where each 128 x 32 tile has amax == F (scale 1), so the
    quantiser sees the probe values themselves: every code value, every midpoint,
    their FP32 neighbours, both signs, zeros."""
    t = oracle.decode_table(fmt)
    top = 0x7E if fmt == "e4m3" else 0x7B
    pos = t[: top + 1]
    F = pos[-1]
    vals = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2]).astype(np.float32)
    vals = np.concatenate([vals, np.nextafter(vals, np.float32(np.inf)),
                           np.nextafter(vals, np.float32(-np.inf))])
    vals = vals[np.abs(vals) <= F]
    vals = np.concatenate([vals, -vals, np.array([0.0, -0.0], dtype=np.float32)])
    n = 128 * 128
    reps = np.resize(vals, n).reshape(128, 128)
    reps[0, 0::32] = F          # each tile's maximum is exactly F -> scale 1
    return reps.astype(np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_edge_values(fmt):
    x = fp8_edge_tile(fmt)
    assert_fp8_equal(x, fmt, label="edge values, unit scale")
    # the same values under non-trivial scales (tile maxima 3x and 1e-3x F)
    y = x.copy()
    y[:, 0:32] *= np.float32(3.0)
    y[:, 32:64] *= np.float32(1e-3)
    y[:, 64:96] *= np.float32(1.0 / 3.0)
    assert_fp8_equal(y, fmt, label="edge values, scaled")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,k,ld", [(300, 96, None), (1, 32, None), (129, 160, 164),
                                       (127, 64, 68), (513, 256, None)])
def test_fp8_ragged(fmt, rows, k, ld):
    x = workloads.normal(100 + rows, rows, k) * np.float32(5.0)
    x[rows // 2, :] *= np.float32(1e4)
    assert_fp8_equal(x, fmt, ld, label="ragged")


def test_fp8_degenerate():
    assert_fp8_equal(np.zeros((130, 64), dtype=np.float32), "e4m3", label="all zero")
    z = np.full((128, 32), -0.0, dtype=np.float32)
    assert_fp8_equal(z, "e4m3", label="all negative zero")
    tiny = (workloads.normal(5, 128, 64) * np.float32(1e-38)).astype(np.float32)   # subnormal scale
    assert_fp8_equal(tiny, "e4m3", label="subnormal-scale tiles")
    big = (workloads.normal(6, 128, 64) * np.float32(1e37)).astype(np.float32)
    assert_fp8_equal(big, "e5m2", label="huge tiles")
    b = bsfp8()
    import torch
    e = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    c, s = b.fp8_quantize(e)
    assert c.shape == (0, 64) and s.shape == (0, 2)


def test_fp8_deterministic():
    x = workloads.normal(77, 512, 512)
    c1, s1 = gpu_fp8(x, "e4m3")
    c2, s2 = gpu_fp8(x, "e4m3")
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_transposed_edge_values(fmt):
    x = fp8_edge_tile(fmt)
    assert_fp8_t_equal(x, fmt, label="edge values, unit scale")
    y = x.copy()
    y[:, 0:32] *= np.float32(3.0)
    y[:, 32:64] *= np.float32(1e-3)
    y[:, 64:96] *= np.float32(1.0 / 3.0)
    assert_fp8_t_equal(y, fmt, label="edge values, scaled")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,k,ld", [(300, 96, None), (1, 32, 4), (129, 160, 132), (127, 64, 128),
                                       (513, 256, None), (130, 288, 132), (3, 64, 8)])
def test_fp8_transposed_ragged(fmt, rows, k, ld):
    """ld is the stored (k x rows) array's leading dimension."""
    x = workloads.normal(300 + rows, rows, k) * np.float32(5.0)
    x[rows // 2, :] *= np.float32(1e4)
    if ld is None and rows % 4:
        ld = rows + (-rows) % 4
    assert_fp8_t_equal(x, fmt, ld, label="ragged")


def test_fp8_transposed_degenerate():
    assert_fp8_t_equal(np.zeros((132, 64), dtype=np.float32), "e4m3", label="all zero")
    assert_fp8_t_equal(np.full((128, 32), -0.0, dtype=np.float32), "e4m3", label="negative zero")
    tiny = (workloads.normal(15, 128, 64) * np.float32(1e-38)).astype(np.float32)
    assert_fp8_t_equal(tiny, "e4m3", label="subnormal-scale tiles")
    big = (workloads.normal(16, 128, 64) * np.float32(1e37)).astype(np.float32)
    assert_fp8_t_equal(big, "e5m2", label="huge tiles")


def test_mxfp4_edge_values():
    # blocks whose maximum is 6 (e = 0) holding every E2M1 midpoint and neighbours
    mids = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6],
                    dtype=np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(10)), np.nextafter(mids, np.float32(-10))])
    vals = np.concatenate([vals, -vals])
    x = np.resize(vals, 64 * 256).reshape(64, 256).astype(np.float32)
    x[:, 0::32] = 6.0
    assert_mx_equal(x, label="E2M1 midpoints, e = 0")
    # exponent boundaries: block maxima at 6 * 2^e and just above / below
    rng = np.random.default_rng(1)
    y = np.empty((64, 256), dtype=np.float32)
    for r in range(64):
        for b in range(8):
            e = int(rng.integers(-125, 126))
            base = np.float32(6.0 * 2.0 ** e)
            m = [base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(0))][(r + b) % 3]
            blk = (rng.uniform(-0.9, 0.9, 32) * float(m)).astype(np.float32)
            blk[(r + 3 * b) % 32] = -m if b % 2 else m
            y[r, b * 32:(b + 1) * 32] = blk
    assert_mx_equal(y, label="exponent boundaries")


@pytest.mark.parametrize("rows,k,ld", [(300, 96, None), (1, 32, None), (129, 160, 164), (33, 64, 72)])
def test_mxfp4_ragged(rows, k, ld):
    x = workloads.normal(200 + rows, rows, k) * np.float32(7.0)
    assert_mx_equal(x, ld, label="ragged")


def test_mxfp4_degenerate():
    assert_mx_equal(np.zeros((40, 64), dtype=np.float32), label="all zero")
    assert_mx_equal((workloads.normal(8, 40, 64) * np.float32(1e-40)).astype(np.float32),
                    label="subnormal blocks")


@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_workload_operands_full_size(name):
    w = workloads.by_name(name)
    a, b = workloads.operands(w)
    if w.a_fmt == "mxfp4":
        assert_mx_equal(a, label=f"{name} A")
        assert_mx_equal(b, label=f"{name} B")
    else:
        assert_fp8_equal(a, w.a_fmt, label=f"{name} A")
        assert_fp8_equal(b, w.b_fmt, label=f"{name} B")


def test_workload_operands_transposed_full_size():
    """The weight-gradient workload with its operands stored token-major (G and
    X as K x M and K x N), quantised by the transposing kernel."""
    w = workloads.by_name("dw_e5m2xe4m3_4096x4096x16384")
    a, b = workloads.operands(w)
    assert_fp8_t_equal(a, w.a_fmt, label=f"{w.name} A from G")
    assert_fp8_t_equal(b, w.b_fmt, label=f"{w.name} B from X")


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("ra,rb,k,lda", [(300, 130, 288, 300), (0, 257, 160, None), (129, 0, 96, None),
                                         (1, 1, 32, None), (640, 1100, 1024, 1028)])
def test_fp8_quantize_pair(fa, fb, ra, rb, k, lda):
    """fp8_quantize_pair: A's and B's codes and scales byte-equal to the
    oracle's (and so to two fp8_quantize calls), ragged rows, a padded A, an
    empty side, mixed formats."""
    import torch
    b_ = bsfp8()
    rng = np.random.default_rng(ra * 7 + rb * 3 + k)
    x = (rng.standard_normal((ra, k)) * np.exp2(rng.integers(-20, 20, size=(ra, 1)))).astype(np.float32)
    y = rng.laplace(size=(rb, k)).astype(np.float32)
    if lda is None:
        xd = to_dev(x) if ra else torch.empty((0, k), dtype=torch.float32, device="cuda")
    else:
        buf = np.zeros((ra, lda), dtype=np.float32)
        buf[:, :k] = x
        xd = to_dev(buf)[:, :k]
    yd = to_dev(y) if rb else torch.empty((0, k), dtype=torch.float32, device="cuda")
    say(f"fp8_quantize_pair {fa} {fb} A {ra}x{k} ld={lda} B {rb}x{k}")
    qa, sa, qb, sb = b_.fp8_quantize_pair(xd, yd, fa, fb)
    torch.cuda.synchronize()
    for rows, xx, fmt, q, s in ((ra, x, fa, qa, sa), (rb, y, fb, qb, sb)):
        if rows == 0:
            continue
        rq, rs = oracle.fp8_quantize(xx, fmt)
        assert np.array_equal(from_dev(q), rq), f"{np.count_nonzero(from_dev(q) != rq)} codes differ"
        assert np.array_equal(from_dev(s), rs), "scales differ"


def test_fp8_quantize_pair_square_4096():
    """The two 4096 x 4096 operands of the square workload in one launch,
    byte-equal to the oracle."""
    import torch
    w = workloads.by_name("square_e4m3_4096")
    a, b = workloads.operands(w)
    say("fp8_quantize_pair square 4096")
    qa, sa, qb, sb = bsfp8().fp8_quantize_pair(to_dev(a), to_dev(b), w.a_fmt, w.b_fmt)
    torch.cuda.synchronize()
    for x, fmt, q, s in ((a, w.a_fmt, qa, sa), (b, w.b_fmt, qb, sb)):
        rq, rs = oracle.fp8_quantize(x, fmt)
        assert np.array_equal(from_dev(q), rq) and np.array_equal(from_dev(s), rs)


# ---------------------------------------------------------------- guard bands
@pytest.mark.parametrize("rows,k", [(200, 96), (1, 32), (129, 4128), (4100, 160)])
def test_quantiser_guard_bands(rows, k):
    """Codes and scales written into buffers with a canary tail of 256
    elements after them (the scale arrays of ragged shapes end mid-tile): every
    quantiser writes exactly its output and nothing past it, and the output is
    byte-equal to the oracle's."""
    import torch
    from gpu_common import guarded, untouched
    b = bsfp8()
    rng = np.random.default_rng(rows + k)
    x = (rng.standard_normal((rows, k)) * 3).astype(np.float32)
    xd = to_dev(x)
    T = 256
    ntile = (rows + 127) // 128

    say(f"guard bands fp8_quantize {rows}x{k}")
    cb, codes = guarded((rows, k), torch.uint8, tail=T)
    sbuf, scales = guarded((ntile * (k // 32),), torch.float32, tail=T)
    b.fp8_quantize(xd, "e4m3", codes=codes, scales=scales.view(ntile, k // 32))
    torch.cuda.synchronize()
    assert untouched(cb, (rows, k), tail=T) and untouched(sbuf, (ntile * (k // 32),), tail=T)
    rc, rs = oracle.fp8_quantize(x, "e4m3")
    assert np.array_equal(from_dev(codes), rc) and np.array_equal(from_dev(scales).reshape(rs.shape), rs)

    say(f"guard bands fp8_quantize_pair {rows}x{k} with {rows + 5}x{k}")
    x2 = (rng.standard_normal((rows + 5, k))).astype(np.float32)
    nt2 = (rows + 5 + 127) // 128
    cb1, c1 = guarded((rows, k), torch.uint8, tail=T)
    sb1, s1 = guarded((ntile * (k // 32),), torch.float32, tail=T)
    cb2, c2 = guarded((rows + 5, k), torch.uint8, tail=T)
    sb2, s2 = guarded((nt2 * (k // 32),), torch.float32, tail=T)
    b.fp8_quantize_pair(xd, to_dev(x2), "e4m3", "e5m2", c1, s1.view(ntile, k // 32), c2,
                        s2.view(nt2, k // 32))
    torch.cuda.synchronize()
    assert untouched(cb1, (rows, k), tail=T) and untouched(sb1, (ntile * (k // 32),), tail=T)
    assert untouched(cb2, (rows + 5, k), tail=T) and untouched(sb2, (nt2 * (k // 32),), tail=T)
    r2c, r2s = oracle.fp8_quantize(x2, "e5m2")
    assert np.array_equal(from_dev(c1), rc) and np.array_equal(from_dev(c2), r2c)
    assert np.array_equal(from_dev(s2).reshape(r2s.shape), r2s)

    say(f"guard bands fp8_quantize_transposed {rows}x{k}")
    cbt, ct = guarded((rows, k), torch.uint8, tail=T)
    sbt, st = guarded((ntile * (k // 32),), torch.float32, tail=T)
    ldt = (rows + 3) // 4 * 4      # x^T stored k x rows, rows padded to 16 bytes
    xt = np.zeros((k, ldt), dtype=np.float32)
    xt[:, :rows] = x.T
    b.fp8_quantize_transposed(to_dev(xt)[:, :rows], "e4m3", codes=ct,
                              scales=st.view(ntile, k // 32))
    torch.cuda.synchronize()
    assert untouched(cbt, (rows, k), tail=T) and untouched(sbt, (ntile * (k // 32),), tail=T)
    assert np.array_equal(from_dev(ct), rc)

    for gran, ns in (("row", rows), ("tensor", 1)):
        say(f"guard bands fp8_quantize_granular {gran} {rows}x{k}")
        cbg, cg = guarded((rows, k), torch.uint8, tail=T)
        sbg, sg = guarded((ns,), torch.float32, tail=T)
        b.fp8_quantize_granular(xd, "e4m3", gran, codes=cg, scales=sg)
        torch.cuda.synchronize()
        assert untouched(cbg, (rows, k), tail=T) and untouched(sbg, (ns,), tail=T)
        gc, gs = oracle.fp8_quantize_granular(x, "e4m3", gran)
        assert np.array_equal(from_dev(cg), gc) and np.array_equal(from_dev(sg).reshape(gs.shape), gs)

    say(f"guard bands mxfp4_quantize {rows}x{k}")
    pbm, pm = guarded((rows, k // 2), torch.uint8, tail=T)
    sbm, sm = guarded((rows * (k // 32),), torch.uint8, tail=T)
    b.mxfp4_quantize(xd, packed=pm, scales=sm.view(rows, k // 32))
    torch.cuda.synchronize()
    assert untouched(pbm, (rows, k // 2), tail=T) and untouched(sbm, (rows * (k // 32),), tail=T)
    mp, ms = oracle.mxfp4_quantize(x)
    assert np.array_equal(from_dev(pm), mp) and np.array_equal(from_dev(sm).reshape(ms.shape), ms)

    say(f"guard bands mx_quantize block 8 bf16 {rows}x{k}")
    pbx, px = guarded((rows, k // 2), torch.uint8, tail=T)
    sbx, sx = guarded((rows * (k // 8),), torch.int16, tail=T)
    b.mx_quantize(xd, 8, "bf16", packed=px, scales=sx.view(rows, k // 8))
    torch.cuda.synchronize()
    assert untouched(pbx, (rows, k // 2), tail=T) and untouched(sbx, (rows * (k // 8),), tail=T)
    xp, xs = oracle.mx_quantize(x, 8, "bf16")
    assert np.array_equal(from_dev(px), xp)
    assert np.array_equal(from_dev(sx).view(np.uint16).reshape(xs.shape), xs)
