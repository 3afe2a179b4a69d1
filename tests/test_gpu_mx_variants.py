"""Parity of the MX variants ("Rubin FP4 GEMM deep dive": blocks of 16 or 8
elements, section 5.3; FP16 or BF16 block scales, section 3.2) on the GPU.

* mx_quantize: packed codes and scales byte-equal to the oracle's, for every
  block size and scale format, on ragged, padded and long rows, rows of every
  magnitude, and rows whose quotients and scales fall exactly on rounding
  midpoints.
* scaled_gemm_mx: D against the oracle's fp64 product of the dequantised
  operands, max |D - D_ref| / S within the output type's tolerance, for every
  block size and scale format, FP32 / bf16 / FP16 output, alpha / beta and
  ragged M, N, K, on the skinny kernel (up to 64 rows or few tiles), the
  128 x 128 kernel and both 256 x 256 kernels (E8M0; FP16 / BF16 scales),
  the large MXFP4 kernel's form for E8M0 blocks of 16 and 8 (two or four FP4
  instructions per 64 K, one per block of each lane's 32 values); and the
  8192^3 shape of the MXFP4 workload on sampled outputs.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_common import TOL, check_gemm, check_gemm_ex, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

SCALES = ["e8m0", "f16", "bf16"]


def bsfp8():
    import block_scaled_precision_fp8_amd as b
    return b


def inputs(seed, rows, k, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "laplace":
        return (rng.laplace(size=(rows, k)) * 1e-3).astype(np.float32)
    x = rng.standard_normal((rows, k))
    if kind == "rows":      # each row at its own magnitude, some all-zero rows
        x = x * np.exp2(rng.integers(-24, 24, size=(rows, 1)))
        x[rng.random(rows) < 0.1] = 0.0
    if kind.startswith("blocks"):  # "blocks<B>[_narrow]": each B-element block at its own magnitude
        bl = int(kind[6:].split("_")[0])
        nb = k // bl
        span = 8 if kind.endswith("_narrow") else 30   # narrow: products stay in FP16's range
        x = x * np.repeat(np.exp2(rng.integers(-span, span, size=(rows, nb))), bl, axis=1)
        x.reshape(rows, nb, bl)[rng.random((rows, nb)) < 0.05] = 0.0   # some all zero
    return x.astype(np.float32)


def midpoints(scale):
    """Blocks of 8: max 6 s for every s of one binade of the scale format, the
    rest s times the E2M1 midpoints; then amax / 6 halfway between two scale
    values (the oracle's own pins use the same construction)."""
    mant = {"f16": 10, "bf16": 7, "e8m0": 0}[scale]
    rows = []
    for j in range(2 ** mant):
        sv = 1.0 + j * 2.0 ** -mant
        rows.append([6 * sv] + [m * sv for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)])
    if mant:
        for j in (0, 1, 2, 3):
            half = 1.0 + (j + 0.5) * 2.0 ** -mant
            rows.append([6 * half, -half, 2 * half, 0.0, -3 * half, half / 4, 5 * half, -0.0])
    x = np.array(rows, dtype=np.float64)
    x = np.tile(x, (1, 4))                    # 32 columns
    return x.astype(np.float32)


def gpu_quant(x, block, scale, ld=None):
    import torch
    if ld is None:
        xd = to_dev(x)
    else:
        buf = np.zeros((x.shape[0], ld), dtype=np.float32)
        buf[:, : x.shape[1]] = x
        xd = to_dev(buf)[:, : x.shape[1]]
    p, s = bsfp8().mx_quantize(xd, block, scale)
    torch.cuda.synchronize()
    p, s = from_dev(p), from_dev(s)
    if scale != "e8m0":
        s = s.view(np.uint16)
    return p, s


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("block", [32, 16, 8])
@pytest.mark.parametrize("rows,k,ld,kind", [(1, 32, None, "normal"), (130, 288, 300, "rows"),
                                            (257, 4096, None, "laplace"), (7, 8192, None, "rows")])
def test_mx_quantize_matches_oracle(block, scale, rows, k, ld, kind):
    say(f"mx_quantize block={block} {scale} rows={rows} k={k} ld={ld} {kind}")
    x = inputs(rows + k + block, rows, k, kind)
    p, s = gpu_quant(x, block, scale, ld)
    rp, rs = oracle.mx_quantize(x, block, scale)
    assert np.array_equal(p, rp), f"{np.count_nonzero(p != rp)} code bytes differ"
    assert np.array_equal(s, rs), f"{np.count_nonzero(s != rs)} scales differ"


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("block", [32, 16, 8])
def test_mx_quantize_midpoints_and_edges(block, scale):
    x = midpoints(scale)
    x[0, 8:14] = [1e-42, -0.0, 3e38, -3e38, 1e-30, 0.0]      # subnormal, -0, near FLT_MAX
    say(f"mx_quantize midpoints block={block} {scale}")
    p, s = gpu_quant(x, block, scale)
    rp, rs = oracle.mx_quantize(x, block, scale)
    assert np.array_equal(p, rp), f"{np.count_nonzero(p != rp)} code bytes differ"
    assert np.array_equal(s, rs), f"{np.count_nonzero(s != rs)} scales differ"


def run_gemm(qa, sa, qb, sb, block, scale, out, K, alpha=1.0, c=None, beta=0.0):
    import torch
    conv = (lambda t: to_dev(t.view(np.int16))) if scale != "e8m0" else to_dev
    d = bsfp8().scaled_gemm_mx(to_dev(qa), conv(sa), to_dev(qb), conv(sb), block, scale, out,
                               alpha, c, beta, None, K)
    torch.cuda.synchronize()
    return from_dev(d)


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("block", [16, 8, 32])
@pytest.mark.parametrize("M,N,K", [(100, 72, 96), (256, 256, 128), (300, 260, 320), (1, 1, 32),
                                   (513, 200, 1056), (1000, 600, 96), (700, 1030, 320)])
def test_mx_gemm_parity(M, N, K, block, scale, out):
    """Shapes with fewer than 32 tiles of 128 x 128 take the skinny kernel, the
    last two (40 and 54 tiles, M > 64) the 128 x 128 kernel."""
    say(f"scaled_gemm_mx block={block} {scale} M={M} N={N} K={K} -> {out}")
    a = inputs(M + 3, M, K, "normal")
    b = inputs(N + 4, N, K, "laplace")
    qa, sa = oracle.mx_quantize(a, block, scale)
    qb, sb = oracle.mx_quantize(b, block, scale)
    d = run_gemm(qa, sa, qb, sb, block, scale, out, K)
    dr, sr = oracle.gemm_mx(qa, sa, qb, sb, block, scale)
    check_gemm(d, dr, sr, out, f"mx block={block} {scale} {M}x{N}x{K} {out}")


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("block", [16, 8])
def test_mx_gemm_alpha_beta(block, scale):
    import torch
    M, N, K = 270, 300, 192
    a = inputs(51, M, K)
    b = inputs(52, N, K)
    qa, sa = oracle.mx_quantize(a, block, scale)
    qb, sb = oracle.mx_quantize(b, block, scale)
    c32 = np.random.default_rng(53).standard_normal((M, N)).astype(np.float32) * 20
    say(f"scaled_gemm_mx alpha/beta block={block} {scale}")
    d = run_gemm(qa, sa, qb, sb, block, scale, "f32", K, -0.5, torch.from_numpy(c32).cuda(), 2.0)
    dr, sr = oracle.gemm_mx(qa, sa, qb, sb, block, scale)
    check_gemm_ex(d, dr, sr, -0.5, 2.0, c32.astype(np.float64), "f32", f"mx alpha/beta {block} {scale}")


@pytest.mark.parametrize("out", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("block,scale", [(16, "e8m0"), (8, "e8m0"), (32, "f16"), (16, "bf16"),
                                         (8, "f16"), (8, "bf16")])
@pytest.mark.parametrize("M,N,K", [(16, 1000, 4096), (1, 520, 416), (33, 300, 32), (64, 2100, 1568),
                                   (50, 64, 8192)])
def test_mx_gemm_skinny_parity(M, N, K, block, scale, out):
    """Up to 64 rows: the skinny kernel, whose four waves split K in chunks of
    8 blocks (K = 32: three waves idle; K = 416: 8 and 5 blocks on two waves;
    K = 1568: 16 / 16 / 16 / 1; long K: several rounds of its two-chunk
    prefetch), ragged M and N."""
    say(f"scaled_gemm_mx skinny block={block} {scale} M={M} N={N} K={K} -> {out}")
    a = inputs(M + K + 5, M, K, "normal")
    b = inputs(N + K + 6, N, K, "laplace")
    qa, sa = oracle.mx_quantize(a, block, scale)
    qb, sb = oracle.mx_quantize(b, block, scale)
    d = run_gemm(qa, sa, qb, sb, block, scale, out, K)
    dr, sr = oracle.gemm_mx(qa, sa, qb, sb, block, scale)
    check_gemm(d, dr, sr, out, f"mx skinny {block} {scale} {M}x{N}x{K} {out}")


@pytest.mark.parametrize("block,scale", [(16, "e8m0"), (8, "bf16")])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_mx_gemm_skinny_alpha_beta(block, scale, out):
    import torch
    M, N, K = 40, 700, 640
    a = inputs(91, M, K)
    b = inputs(92, N, K)
    qa, sa = oracle.mx_quantize(a, block, scale)
    qb, sb = oracle.mx_quantize(b, block, scale)
    c32 = np.random.default_rng(93).standard_normal((M, N)).astype(np.float32) * 20
    if out == "bf16":
        c = torch.from_numpy(c32).to(torch.bfloat16)
        cref = c.float().numpy().astype(np.float64)
    else:
        c = torch.from_numpy(c32)
        cref = c32.astype(np.float64)
    say(f"scaled_gemm_mx skinny alpha/beta block={block} {scale} -> {out}")
    d = run_gemm(qa, sa, qb, sb, block, scale, out, K, 1.25, c.cuda(), 0.5)
    dr, sr = oracle.gemm_mx(qa, sa, qb, sb, block, scale)
    check_gemm_ex(d, dr, sr, 1.25, 0.5, cref, out, f"mx skinny alpha/beta {block} {scale} {out}")


LARGE = [(16, "e8m0"), (8, "e8m0"), (32, "f16"), (16, "f16"), (8, "f16"),
         (32, "bf16"), (16, "bf16"), (8, "bf16")]


@pytest.mark.parametrize("out", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("block,scale", LARGE)
@pytest.mark.parametrize("M,N,K", [(4100, 2049, 160), (2304, 3840, 512), (2304, 3840, 32),
                                   (2304, 3840, 64)])
def test_mx_gemm_large_tile_parity(M, N, K, block, scale, out):
    """Shapes with at least 128 tiles of 256 x 256 take the large-tile kernels
    (E8M0 blocks of 16 or 8; FP16 / BF16 scales with any block): ragged M
    and N, K % 64 == 32, all outputs, and K of one or two 32-K blocks (the
    pipelines' shortest runs)."""
    say(f"scaled_gemm_mx large tile block={block} {scale} M={M} N={N} K={K} -> {out}")
    a = inputs(M + K, M, K, "normal")
    b = inputs(N + K, N, K, "laplace")
    qa, sa = oracle.mx_quantize(a, block, scale)
    qb, sb = oracle.mx_quantize(b, block, scale)
    d = run_gemm(qa, sa, qb, sb, block, scale, out, K)
    dr, sr = oracle.gemm_mx(qa, sa, qb, sb, block, scale)
    check_gemm(d, dr, sr, out, f"mx large tile {block} {scale} {M}x{N}x{K} {out}")


@pytest.mark.parametrize("out", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("M,N,K", [(2048, 2048, 256), (2056, 2048, 768), (2048, 2064, 1280),
                                   (2304, 3840, 512), (1000, 600, 96), (1536, 1032, 2080),
                                   (16, 1000, 4096), (64, 2100, 1568), (1, 520, 416)])
@pytest.mark.parametrize("block", [16, 8])
def test_mx_fp4_form_parity(block, M, N, K, out):
    """E8M0 blocks of 16 or 8 run on the block-scaled FP4 instruction, one per
    block of each lane's 32 K values (the others zero): on the large MXFP4
    kernel for K a multiple of 256 and at least 64 tiles of 256 x 256, on the
    128 x 128 one below 128 such tiles (1000 x 600 x 96 and 1536 x 1032 x 2080:
    K % 64 == 32 and a partial last stage), and on the skinny one for up to 64
    rows (the last three, K split over the waves with a ragged last chunk).  A's blocks each sit at their own
    power of two (some all zero; within 2^±8 for FP16 output, whose range the
    wider spread would overflow), so a block paired with a neighbour's scale
    fails; K = 256, 768 and 1280 give one stage, an odd number of stages and
    (blocks of 16) a partial last scale period; M and N are ragged."""
    say(f"scaled_gemm_mx blocks of {block} on the FP4 kernel M={M} N={N} K={K} -> {out}")
    kind = f"blocks{block}" + ("_narrow" if out == "f16" else "")
    a = inputs(M + 3 * K + block, M, K, kind)
    b = inputs(N + 5 * K, N, K, "laplace")
    qa, sa = oracle.mx_quantize(a, block, "e8m0")
    qb, sb = oracle.mx_quantize(b, block, "e8m0")
    d = run_gemm(qa, sa, qb, sb, block, "e8m0", out, K)
    dr, sr = oracle.gemm_mx(qa, sa, qb, sb, block, "e8m0")
    check_gemm(d, dr, sr, out, f"mx{block} fp4 kernel {M}x{N}x{K} {out}")


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("block", [16, 8])
@pytest.mark.parametrize("M,N,K", [(2304, 3840, 512), (1000, 600, 96), (40, 700, 640)])
def test_mx_fp4_form_alpha_beta(M, N, K, block, out):
    """alpha, beta * C on the large, 128 x 128 and skinny FP4 forms."""
    import torch
    a = inputs(91, M, K, f"blocks{block}")
    b = inputs(92, N, K, f"blocks{block}")
    qa, sa = oracle.mx_quantize(a, block, "e8m0")
    qb, sb = oracle.mx_quantize(b, block, "e8m0")
    c32 = np.random.default_rng(93).standard_normal((M, N)).astype(np.float32) * 20
    if out == "bf16":
        c = torch.from_numpy(c32).to(torch.bfloat16)
        cref = c.float().numpy().astype(np.float64)
    else:
        c = torch.from_numpy(c32)
        cref = c32.astype(np.float64)
    say(f"scaled_gemm_mx blocks of {block} on the FP4 kernel alpha/beta -> {out}")
    d = run_gemm(qa, sa, qb, sb, block, "e8m0", out, K, 0.75, c.cuda(), -1.5)
    dr, sr = oracle.gemm_mx(qa, sa, qb, sb, block, "e8m0")
    check_gemm_ex(d, dr, sr, 0.75, -1.5, cref, out, f"mx{block} fp4 kernel alpha/beta {out}")


@pytest.mark.parametrize("block,scale", [(16, "e8m0"), (8, "e8m0"), (16, "f16"), (8, "bf16")])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_mx_gemm_large_tile_alpha_beta(block, scale, out):
    import torch
    M, N, K = 2304, 3840, 224
    a = inputs(81, M, K)
    b = inputs(82, N, K)
    qa, sa = oracle.mx_quantize(a, block, scale)
    qb, sb = oracle.mx_quantize(b, block, scale)
    c32 = np.random.default_rng(83).standard_normal((M, N)).astype(np.float32) * 20
    if out == "bf16":
        c = torch.from_numpy(c32).to(torch.bfloat16)
        cref = c.float().numpy().astype(np.float64)
    else:
        c = torch.from_numpy(c32)
        cref = c32.astype(np.float64)
    say(f"scaled_gemm_mx large tile alpha/beta block={block} {scale} -> {out}")
    d = run_gemm(qa, sa, qb, sb, block, scale, out, K, 0.75, c.cuda(), -1.5)
    dr, sr = oracle.gemm_mx(qa, sa, qb, sb, block, scale)
    check_gemm_ex(d, dr, sr, 0.75, -1.5, cref, out, f"mx large tile alpha/beta {block} {scale} {out}")


@pytest.mark.parametrize("block,scale", [(16, "e8m0"), (8, "bf16")])
def test_mx_end_to_end(block, scale):
    """HIP quantiser then HIP GEMM against the oracle on the same FP32 inputs."""
    import torch
    M, N, K = 384, 256, 1024
    a = inputs(61, M, K)
    b = inputs(62, N, K, "laplace")
    b_ = bsfp8()
    say(f"mx end to end block={block} {scale}")
    qa, sa = b_.mx_quantize(to_dev(a), block, scale)
    qb, sb = b_.mx_quantize(to_dev(b), block, scale)
    d = b_.scaled_gemm_mx(qa, sa, qb, sb, block, scale, "bf16")
    torch.cuda.synchronize()
    rqa, rsa = oracle.mx_quantize(a, block, scale)
    rqb, rsb = oracle.mx_quantize(b, block, scale)
    assert np.array_equal(from_dev(qa), rqa) and np.array_equal(from_dev(qb), rqb)
    dr, sr = oracle.gemm_mx(rqa, rsa, rqb, rsb, block, scale)
    check_gemm(from_dev(d), dr, sr, "bf16", f"mx end to end {block} {scale}")


@pytest.mark.parametrize("block,scale", [(16, "e8m0"), (8, "e8m0"), (32, "bf16")])
def test_mx_gemm_8192_sampled(block, scale):
    """The 8192^3 shape of the MXFP4 workload, checked on sampled outputs."""
    w = workloads.by_name("mxfp4_8192")
    a, b = workloads.operands(w)
    qa, sa = oracle.mx_quantize(a, block, scale)
    qb, sb = oracle.mx_quantize(b, block, scale)
    say(f"scaled_gemm_mx 8192^3 block={block} {scale}")
    d = run_gemm(qa, sa, qb, sb, block, scale, "bf16", w.K)
    rng = np.random.default_rng(71)
    ii = np.concatenate([rng.integers(0, w.M, 150), [0, w.M - 1, 127, 128]])
    jj = np.concatenate([rng.integers(0, w.N, 150), [w.N - 1, 0, 128, 127]])
    ad = oracle.dequantize_mx(qa[ii], sa[ii], block, scale)
    bd = oracle.dequantize_mx(qb[jj], sb[jj], block, scale)
    dr = np.sum(ad * bd, axis=1)
    sr = np.sum(np.abs(ad * bd), axis=1)
    err = np.abs(d[ii, jj].astype(np.float64) - dr) / sr
    say(f"sampled max |D-Dref|/S = {err.max():.3e}")
    assert err.max() <= TOL["bf16"]
