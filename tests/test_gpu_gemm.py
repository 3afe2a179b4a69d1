"""GEMM parity: the HIP scaled_gemm against the oracle's fp64 product of the
dequantised operands, normalised by S = sum_k |a_k b_k|:
    max |D - D_ref| / S <= 2^-19 (FP32 output), <= 2^-7 (bf16 output).
Operand codes and scales come from the oracle's quantiser (so no oracle input
is produced by the HIP path); one end-to-end test per workload also runs the
HIP quantiser.  Runs through the C ABI (the Python binding)."""
import os

import numpy as np
import pytest

import oracle
import workloads
from gpu_common import check_gemm, check_gemm_ex, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bsfp8():
    import block_scaled_precision_fp8_amd as b
    return b


def oracle_quant(x, fmt):
    return oracle.mxfp4_quantize(x) if fmt == "mxfp4" else oracle.fp8_quantize(x, fmt)


def run_gpu_gemm(qa, sa, qb, sb, a_fmt, b_fmt, out, K):
    import torch
    d = bsfp8().scaled_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), a_fmt, b_fmt, out, K=K)
    torch.cuda.synchronize()
    return from_dev(d)


def full_check(M, N, K, a_fmt, b_fmt, out, seed, label):
    say(f"scaled_gemm {label} M={M} N={N} K={K} {a_fmt}x{b_fmt} -> {out}")
    a = workloads.normal(seed, M, K) * np.float32(2.0)
    b = workloads.normal(seed + 1, N, K)
    if a_fmt == "e5m2":
        a = workloads.laplace(seed, M, K, 1e-3)
    qa, sa = oracle_quant(a, a_fmt)
    qb, sb = oracle_quant(b, b_fmt)
    d = run_gpu_gemm(qa, sa, qb, sb, a_fmt, b_fmt, out, K)
    dr, sr = oracle.gemm_rows(a_fmt, qa, sa, b_fmt, qb, sb)
    return check_gemm(d, dr, sr, out, label)


def load_dot_examples():
    out = []
    with open(os.path.join(GOLDEN, "dot_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            a, b, exact, bits, h100 = [p.strip() for p in line.split("|")]
            out.append(([float(v) for v in a.split()], [float(v) for v in b.split()],
                        float(exact), int(bits, 16)))
    return out


def test_dot_examples_fp32_output_exact():
    """The pages' two dot examples through scaled_gemm with unit scales.  FP32
    output keeps 24 alignment bits, so both come out exact (not truncated)."""
    for a, b, exact, bits in load_dot_examples():
        qa = np.zeros((128, 32), dtype=np.uint8)
        qb = np.zeros((128, 32), dtype=np.uint8)
        qa[0, : len(a)] = oracle.encode("e4m3", a)
        qb[0, : len(b)] = oracle.encode("e4m3", b)
        one = np.ones((1, 1), dtype=np.float32)
        say(f"dot example {a} . {b}")
        d = run_gpu_gemm(qa, one, qb, one, "e4m3", "e4m3", "f32", 32)
        got = np.float32(d[0, 0]).view(np.uint32)
        say(f"  FP32 result {d[0, 0]!r} bits {got:#010x} (exact {bits:#010x})")
        assert got == bits
        assert np.all(d.reshape(-1)[1:] == 0)
        db = run_gpu_gemm(qa, one, qb, one, "e4m3", "e4m3", "bf16", 32)
        assert abs(db[0, 0] - exact) <= 2.0 ** -7 * sum(abs(x * y) for x, y in zip(a, b))


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmts", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("M,N,K", [(1, 257, 32), (33, 1000, 4128), (64, 4096, 8192), (17, 96, 96),
                                   (64, 130, 1024)])
def test_fp8_skinny(M, N, K, fmts, out):
    """Up to 64 rows: the skinny kernel (32 x 32 tiles; K split over four waves
    in chunks of 4 blocks, 128 bytes of a row, and summed in a fixed order).
    K = 32 leaves three waves without a block; K = 96 gives wave 0 one partial
    chunk; 129 blocks split 36 / 36 / 36 / 21, the last chunk holding one
    block; ragged N."""
    full_check(M, N, K, fmts[0], fmts[1], out, seed=M + N + K, label="skinny")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmts", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"),
                                  ("e5m2", "e5m2")])
@pytest.mark.parametrize("M,N,K", [(200, 328, 96), (1, 1, 32), (129, 255, 64),
                                   (256, 384, 544), (383, 130, 160)])
def test_fp8_small_ragged(M, N, K, fmts, out):
    full_check(M, N, K, fmts[0], fmts[1], out, seed=M * 7 + N * 3 + K, label="small")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [(200, 328, 96), (1, 1, 32), (129, 255, 64),
                                   (256, 256, 512), (130, 260, 288), (64, 64, 2080)])
def test_mxfp4_small_ragged(M, N, K, out):
    full_check(M, N, K, "mxfp4", "mxfp4", out, seed=M * 5 + N + K, label="small mxfp4")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [(1, 257, 32), (33, 1000, 4128), (64, 4096, 8192), (17, 96, 96),
                                   (48, 130, 2080)])
def test_mxfp4_skinny(M, N, K, out):
    """Up to 64 rows: the skinny MXFP4 kernel (32 x 32 tiles; K split over four
    waves in chunks of 8 blocks, 128 bytes of a row, and summed in a fixed
    order).  129 blocks split 40 / 40 / 40 / 9 and 65 blocks 24 / 24 / 17, each
    with a last chunk of one block; K = 32 leaves three waves without a block."""
    full_check(M, N, K, "mxfp4", "mxfp4", out, seed=M * 7 + N + K, label="skinny mxfp4")


def test_degenerate_shapes():
    import torch
    b = bsfp8()
    say("scaled_gemm degenerate shapes")
    # K = 0: D = 0
    a = torch.zeros((130, 0), dtype=torch.uint8, device="cuda")
    s = torch.zeros((2, 0), dtype=torch.float32, device="cuda")
    d = torch.full((130, 70), 7.0, dtype=torch.float32, device="cuda")
    b.scaled_gemm(a, s, a[:70], s[:1], "e4m3", "e4m3", "f32", d=d, K=0)
    torch.cuda.synchronize()
    assert torch.all(d == 0)
    # M = 0: nothing happens
    e = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    r = b.scaled_gemm(e, s, e, s, "e4m3", "e4m3", "bf16", K=64)
    assert r.shape == (0, 0)
    # all-zero codes: D = 0 exactly
    qa = np.zeros((256, 128), dtype=np.uint8)
    sa = np.ones((2, 4), dtype=np.float32)
    d = run_gpu_gemm(qa, sa, qa[:130], sa, "e4m3", "e4m3", "f32", 128)
    assert np.all(d == 0)


def _points(M, N, rng, n=3000):
    ii = np.concatenate([np.arange(min(128, M)), rng.integers(0, M, n), [M - 1] * 4])
    jj = np.concatenate([rng.integers(0, N, min(128, M)), rng.integers(0, N, n), [0, 1, N - 2, N - 1]])
    return ii.astype(np.int64), jj.astype(np.int64)


def _row_tiles(M, every):
    """Rows of every `every`-th 128-row tile of D, plus the last row."""
    rows = [np.arange(t, min(t + 128, M)) for t in range(0, M, 128 * every)]
    return np.unique(np.concatenate(rows + [np.array([M - 1])]))


@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_workload_full_size(name):
    """Every workload at its full size, in the launch configuration the benchmark
    times, compared with the oracle on whole rows of D: all of D for the small,
    decode-shaped and 4096-cube workloads, every 8th 128-row tile (all columns)
    plus the last row for the feed-forward, weight-gradient and MXFP4 ones."""
    w = workloads.by_name(name)
    a, b = workloads.operands(w)
    qa, sa = oracle_quant(a, w.a_fmt)
    qb, sb = oracle_quant(b, w.b_fmt)
    say(f"{name}: oracle codes ready; GPU scaled_gemm {w.M}x{w.N}x{w.K} -> {w.out}")
    d = run_gpu_gemm(qa, sa, qb, sb, w.a_fmt, w.b_fmt, w.out, w.K)
    every = 1 if w.M * w.N * w.K <= 4096 ** 3 else 8
    rows = _row_tiles(w.M, every)
    say(f"{name}: oracle on {rows.size} of {w.M} rows (every {every} row tiles)")
    if every == 1:
        dr, sr = oracle.gemm_rows(w.a_fmt, qa, sa, w.b_fmt, qb, sb)
    else:
        # the oracle on those rows: tile-aligned slices keep their tile's scales
        parts = []
        for t in range(0, w.M, 128 * every):
            r1 = min(t + 128, w.M)
            parts.append(oracle.gemm_rows(w.a_fmt, qa, sa, w.b_fmt, qb, sb, t, r1))
        if (w.M - 1) // 128 % every:
            parts.append(oracle.gemm_rows(w.a_fmt, qa, sa, w.b_fmt, qb, sb, w.M - 1, w.M))
        dr = np.concatenate([p[0] for p in parts])
        sr = np.concatenate([p[1] for p in parts])
    check_gemm(d[rows], dr, sr, w.out, name)


@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_workload_end_to_end(name):
    """HIP quantiser + HIP GEMM on the workload's FP32 operands against the
    oracle's quantiser + product (sampled outputs)."""
    import torch
    w = workloads.by_name(name)
    a, b = workloads.operands(w)
    bs = bsfp8()
    say(f"{name}: end to end on the GPU")
    ad, bd = to_dev(a), to_dev(b)
    if w.a_fmt == "mxfp4":
        ga, gsa = bs.mxfp4_quantize(ad)
        gb, gsb = bs.mxfp4_quantize(bd)
    else:
        ga, gsa = bs.fp8_quantize(ad, w.a_fmt)
        gb, gsb = bs.fp8_quantize(bd, w.b_fmt)
    d = bs.scaled_gemm(ga, gsa, gb, gsb, w.a_fmt, w.b_fmt, w.out, K=w.K)
    torch.cuda.synchronize()
    d = from_dev(d)
    del ad, bd, ga, gb
    qa, sa = oracle_quant(a, w.a_fmt)
    qb, sb = oracle_quant(b, w.b_fmt)
    rng = np.random.default_rng(100 + w.index)
    ii, jj = _points(w.M, w.N, rng, n=1000)
    dr, sr = oracle.gemm_points(w.a_fmt, qa, sa, w.b_fmt, qb, sb, ii, jj)
    check_gemm(d[ii, jj], dr, sr, w.out, name + " end-to-end")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmts,M,N,K", [
    (("mxfp4", "mxfp4"), 2088, 2072, 512),     # 256 x 256 MXFP4 kernel, ragged edges
    (("mxfp4", "mxfp4"), 2048, 2048, 768),     # scales: one partial 4-stage period, rows 8-byte aligned
    (("mxfp4", "mxfp4"), 2056, 2048, 1280),    # scales: a second period of one stage
    (("mxfp4", "mxfp4"), 2048, 2064, 2304),    # scales: two full periods and one stage
    (("mxfp4", "mxfp4"), 2088, 2072, 640),     # 256 x 256 ring kernel: K % 256 = 128
    (("mxfp4", "mxfp4"), 2056, 2048, 544),     # ring kernel: K / 32 = 17, scale rows unaligned
    (("mxfp4", "mxfp4"), 2048, 2304, 96),      # ring kernel: one partial 128-K buffer
    (("mxfp4", "mxfp4"), 2048, 2080, 1056),    # ring kernel: a partial last trip around the ring
    (("e4m3", "e4m3"), 2088, 2072, 512),       # large-tile FP8 path, ragged edges
    (("e5m2", "e4m3"), 2048, 2080, 384),
    (("e4m3", "e4m3"), 4100, 2049, 160),       # 4 rows in the last tile row, K % 128 = 32
    (("e5m2", "e4m3"), 4224, 2048, 384),
])
def test_medium_ragged_large_tile_kernels(fmts, M, N, K, out):
    """Shapes big enough for the large-tile kernels, with partial edge tiles,
    compared in full against the oracle."""
    full_check(M, N, K, fmts[0], fmts[1], out, seed=M + N + K, label="medium")


_TORCH_DT = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmts,M,N,K", [
    (("e4m3", "e4m3"), 200, 328, 160),
    (("e5m2", "e4m3"), 2088, 2072, 512),     # FP8 kernel, ragged edges
    (("mxfp4", "mxfp4"), 130, 260, 288),      # small MXFP4 kernel
    (("mxfp4", "mxfp4"), 2088, 2072, 512),    # 256 x 256 MXFP4 kernel
    (("e4m3", "e4m3"), 4100, 2049, 160),      # FP8 kernel, larger ragged shape
    (("e5m2", "e4m3"), 40, 300, 480),         # skinny FP8 kernel
    (("mxfp4", "mxfp4"), 40, 300, 480),       # skinny MXFP4 kernel
])
def test_alpha_beta_epilogue(fmts, M, N, K, out):
    """D = alpha A B + beta C through scaled_gemm_ex, C in the output type;
    then in place (C is D) with beta = 1; then beta = 0 (C not read)."""
    import torch
    a_fmt, b_fmt = fmts
    seed = M + 3 * N + K
    a = workloads.normal(seed, M, K) * np.float32(2.0)
    b = workloads.normal(seed + 1, N, K)
    qa, sa = oracle_quant(a, a_fmt)
    qb, sb = oracle_quant(b, b_fmt)
    dr, sr = oracle.gemm_rows(a_fmt, qa, sa, b_fmt, qb, sb)
    dt = getattr(torch, _TORCH_DT[out])
    c = (torch.from_numpy(workloads.normal(seed + 2, M, N) * np.float32(30.0))).to(dt).cuda()
    c_host = from_dev(c)
    bs = bsfp8()
    args = (to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), a_fmt, b_fmt, out)
    say(f"scaled_gemm_ex alpha/beta {M}x{N}x{K} {a_fmt}x{b_fmt} -> {out}")
    d = bs.scaled_gemm_ex(*args, alpha=-0.75, c=c, beta=1.5, K=K)
    torch.cuda.synchronize()
    check_gemm_ex(from_dev(d), dr, sr, -0.75, 1.5, c_host, out, "alpha/beta")
    # in place: D <- 0.5 A B + D
    d2 = c.clone()
    bs.scaled_gemm_ex(*args, alpha=0.5, c=d2, beta=1.0, d=d2, K=K)
    torch.cuda.synchronize()
    check_gemm_ex(from_dev(d2), dr, sr, 0.5, 1.0, c_host, out, "in place")
    # beta = 0: C is not read (NaN-filled C must not leak into D)
    junk = torch.full_like(c, float("nan"))
    d3 = bs.scaled_gemm_ex(*args, alpha=2.0, c=junk, beta=0.0, K=K)
    torch.cuda.synchronize()
    check_gemm_ex(from_dev(d3), dr, sr, 2.0, 0.0, None, out, "beta = 0")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_k_zero_writes_beta_c(out):
    import torch
    dt = getattr(torch, _TORCH_DT[out])
    c = torch.from_numpy(workloads.normal(9, 130, 70)).to(dt).cuda()
    e = torch.zeros((130, 0), dtype=torch.uint8, device="cuda")
    s = torch.zeros((2, 0), dtype=torch.float32, device="cuda")
    say(f"scaled_gemm_ex K = 0 -> {out}")
    d = bsfp8().scaled_gemm_ex(e, s, e[:70], s[:1], "e4m3", "e4m3", out, alpha=3.0, c=c,
                               beta=-2.0, K=0)
    torch.cuda.synchronize()
    expect = (-2.0 * c.float()).to(dt)   # one FP32 product, then the output rounding
    assert torch.equal(d, expect)


def test_fp8_operand_beyond_32bit_offsets():
    """An A operand larger than 2^32 bytes: 2^19 + 96 rows of 8192 E4M3 codes
    (4.3 GB), generated on the device.  Outputs in rows past the first 2^32
    bytes of A, and in the first and last rows, against the oracle on a
    sub-problem that holds just the sampled rows (each at the start of its own
    128-row tile, with that tile's scales)."""
    import torch
    M, N, K = (1 << 19) + 96, 256, 8192
    say(f"scaled_gemm with A of {M * K / 2**30:.2f} GiB ({M}x{N}x{K})")
    g = torch.Generator(device="cuda").manual_seed(7)
    # random codes with exponent bit 3 cleared: every value finite (no 0x7F / 0xFF)
    qa = torch.randint(0, 256, (M, K), dtype=torch.uint8, device="cuda", generator=g)
    qa &= 0xF7
    qb = torch.randint(0, 256, (N, K), dtype=torch.uint8, device="cuda", generator=g) & 0xF7
    sa = torch.rand(((M + 127) // 128, K // 32), device="cuda", generator=g) + 0.5
    sb = torch.rand(((N + 127) // 128, K // 32), device="cuda", generator=g) + 0.5
    d = bsfp8().scaled_gemm(qa, sa, qb, sb, "e4m3", "e4m3", "bf16")
    torch.cuda.synchronize()
    first_past = (1 << 32) // K                      # first row that starts past 2^32 bytes
    rng = np.random.default_rng(8)
    ii = np.unique(np.concatenate([[0, 1, first_past - 1, first_past, first_past + 1, M - 1, M - 2],
                                   rng.integers(first_past, M, 25)]))
    jj = rng.integers(0, N, ii.size)
    jj[-1] = N - 1
    rows = qa[torch.from_numpy(ii).cuda()].cpu().numpy()
    srows = sa[torch.from_numpy(ii // 128).cuda()].cpu().numpy()
    del qa
    sub = np.zeros((128 * ii.size, K), dtype=np.uint8)
    sub[0::128] = rows
    dr, sr = oracle.gemm_points("e4m3", sub, srows, "e4m3", from_dev(qb), from_dev(sb),
                                128 * np.arange(ii.size), jj)
    got = from_dev(d[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()])
    check_gemm(got, dr, sr, "bf16", "A beyond 2^32 bytes")


# ---------------------------------------------------------------- guard bands
_GUARD_CASES = [
    # (a_fmt, b_fmt, M, N, K, kernel exercised)
    ("e4m3", "e4m3", 1000, 4100, 288, "per-tile FP8, ragged edges and a partial K stage"),
    ("e5m2", "e4m3", 40, 300, 480, "skinny FP8"),
    ("mxfp4", "mxfp4", 2088, 2072, 512, "256 x 256 MXFP4"),
    ("mxfp4", "mxfp4", 2088, 2072, 544, "256 x 256 MXFP4 ring, ragged K"),
    ("mxfp4", "mxfp4", 130, 260, 288, "128 x 128 MXFP4"),
    ("mxfp4", "mxfp4", 40, 300, 480, "skinny MXFP4"),
]


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("a_fmt,b_fmt,M,N,K,what", _GUARD_CASES)
def test_strided_d_guard_band(a_fmt, b_fmt, M, N, K, what, out):
    """D written into rows of N + 64 elements (ldd > N), inside a buffer
    pre-filled with a canary: every output is checked against the oracle and
    the 64 columns past N of every row, and two rows past M, must still hold
    the canary (masked edge stores write nothing outside the M x N window)."""
    import torch
    from gpu_common import guarded, untouched
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out]
    say(f"guard band: {what} M={M} N={N} K={K} {a_fmt}x{b_fmt} -> {out}, ldd = N + 64")
    a = workloads.normal(M + K, M, K)
    b = workloads.normal(N + K, N, K)
    qa, sa = oracle_quant(a, a_fmt)
    qb, sb = oracle_quant(b, b_fmt)
    buf, d = guarded((M, N), dt, extra_cols=64, extra_rows=2, tail=64)
    assert d.stride(0) == N + 64
    bsfp8().scaled_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), a_fmt, b_fmt, out, d=d, K=K)
    torch.cuda.synchronize()
    assert untouched(buf, (M, N), extra_cols=64, extra_rows=2, tail=64), f"{what}: write outside D"
    dr, sr = oracle.gemm_rows(a_fmt, qa, sa, b_fmt, qb, sb)
    check_gemm(from_dev(d), dr, sr, out, f"guard band {what}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_strided_d_guard_band_alpha_beta(out):
    """The alpha / beta epilogue with ldd = ldc = N + 64 (C read from, and D
    written into, strided rows), both inside canary-filled buffers."""
    import torch
    from gpu_common import guarded, untouched
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[out]
    M, N, K = 1000, 4100, 160
    say(f"guard band alpha/beta M={M} N={N} K={K} -> {out}")
    a = workloads.normal(3, M, K)
    b = workloads.normal(4, N, K)
    c = workloads.normal(5, M, N)
    qa, sa = oracle.fp8_quantize(a, "e4m3")
    qb, sb = oracle.fp8_quantize(b, "e4m3")
    dbuf, d = guarded((M, N), dt, extra_cols=64, extra_rows=1)
    cbuf, cv = guarded((M, N), dt, extra_cols=64, extra_rows=1)
    cv.copy_(torch.from_numpy(c).to(dt).cuda())
    c_used = cv.float().cpu().numpy()
    bsfp8().scaled_gemm_ex(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), "e4m3", "e4m3", out,
                           alpha=0.5, c=cv, beta=-1.25, d=d, K=K)
    torch.cuda.synchronize()
    assert untouched(dbuf, (M, N), extra_cols=64, extra_rows=1), "write outside D"
    assert untouched(cbuf, (M, N), extra_cols=64, extra_rows=1), "write into C's guard band"
    dr, sr = oracle.gemm_rows("e4m3", qa, sa, "e4m3", qb, sb)
    check_gemm_ex(from_dev(d), dr, sr, 0.5, -1.25, c_used, out, "guard band alpha/beta")


@pytest.mark.parametrize("M,N,K", [(1000, 4100, 288), (1000, 4100, 4000), (640, 4608, 224),
                                   (4100, 2049, 96)])
def test_per_tile_ragged_k(M, N, K):
    """The per-tile FP8 kernel with K not a multiple of 128: the partial last
    stage (1 to 3 blocks) is loaded with range-checked offsets, so the chunks
    and scales past K read as zero; the whole product is compared."""
    for out in ("f32", "bf16"):
        full_check(M, N, K, "e4m3", "e4m3", out, seed=M + 3 * N + K, label=f"ragged K {K}")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmts,M,N,K", [
    (("e4m3", "e4m3"), 3000, 4200, 288),      # ragged M and N, a partial K stage of one block
    (("e5m2", "e4m3"), 4096, 3136, 224),      # a partial stage of three blocks only
    (("e4m3", "e5m2"), 3584, 3584, 640),      # five full stages (odd count)
])
def test_big_tile_kernel(fmts, M, N, K, out):
    """Shapes with at least 192 tiles of 256 x 256 run the large-tile per-tile
    kernel (8 waves of 64 x 128); whole D against the oracle."""
    full_check(M, N, K, fmts[0], fmts[1], out, seed=M + 5 * N + K, label="big tile")


def test_big_tile_kernel_long_ragged_k():
    full_check(3000, 4200, 4000, "e4m3", "e4m3", "bf16", seed=77, label="big tile K = 4000")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_big_tile_kernel_guard_band_alpha_beta(out):
    """The large-tile kernel's general epilogue (alpha, beta * C) with D and C
    in strided rows inside canary-filled buffers."""
    import torch
    from gpu_common import guarded, untouched
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[out]
    M, N, K = 3000, 4200, 160
    say(f"big tile guard band alpha/beta M={M} N={N} K={K} -> {out}")
    a = workloads.normal(13, M, K)
    b = workloads.normal(14, N, K)
    c = workloads.normal(15, M, N)
    qa, sa = oracle.fp8_quantize(a, "e4m3")
    qb, sb = oracle.fp8_quantize(b, "e4m3")
    dbuf, d = guarded((M, N), dt, extra_cols=64, extra_rows=1)
    cbuf, cv = guarded((M, N), dt, extra_cols=64, extra_rows=1)
    cv.copy_(torch.from_numpy(c).to(dt).cuda())
    c_used = cv.float().cpu().numpy()
    bsfp8().scaled_gemm_ex(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), "e4m3", "e4m3", out,
                           alpha=-1.5, c=cv, beta=0.75, d=d, K=K)
    torch.cuda.synchronize()
    assert untouched(dbuf, (M, N), extra_cols=64, extra_rows=1), "write outside D"
    assert untouched(cbuf, (M, N), extra_cols=64, extra_rows=1), "write into C's guard band"
    dr, sr = oracle.gemm_rows("e4m3", qa, sa, "e4m3", qb, sb)
    check_gemm_ex(from_dev(d), dr, sr, -1.5, 0.75, c_used, out, "big tile guard band alpha/beta")
