"""Parity of the GEMM that quantises its FP32 A operand while loading it
(scaled_gemm_quantize_a; "Why grind FP8 GEMM on CDNA4", sections 3.3 and
4.2; "Rubin FP4 GEMM deep dive", section 4.2, step 4) on the GPU.

* The A codes and scales the kernel writes out are byte-equal to the
  oracle's per-tile quantisation of x, on ragged, padded and short inputs
  and on tiles of every magnitude (zero tiles, tiles far below and far above
  one, which take both quotient forms of the kernel).
* D against the oracle's fp64 product of the oracle's codes, within the
  output type's tolerance: ragged M, N, K (K % 128 in {0, 32, 64, 96}),
  FP32 / bf16 / FP16 output, alpha / beta, both A formats, per-tile and
  per-tensor B.
* The full 4096^3 launch of the square workload: every A code and scale, and
  sampled outputs.
With A's codes requested and more than three 128-wide column tiles of output
the call quantises A first and runs the per-tile GEMM; the single-launch
kernel runs otherwise, and the tests cover both (wide outputs without code
output included).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_common import TOL, check_gemm, check_gemm_ex, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def bsfp8():
    import block_scaled_precision_fp8_amd as b
    return b


def inputs(seed, rows, k, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "laplace":
        return (rng.laplace(size=(rows, k)) * 1e-3).astype(np.float32)
    x = rng.standard_normal((rows, k))
    if kind == "tiles":
        # every 128 x 32 tile at its own magnitude 2^u, u in [-90, 40]: tiles
        # whose scale is below 2^-82 (u below about -74) take the kernel's
        # general quotient form; a tenth of the tiles are all zero.  (Down to
        # 2^-90 the scale products and every partial sum stay normal FP32
        # numbers, so the tolerance relative to sum |a b| applies.)
        tr, tk = (rows + 127) // 128, k // 32
        u = rng.integers(-90, 41, size=(tr, tk)).astype(np.float64)
        f = np.exp2(u)
        f[rng.random((tr, tk)) < 0.1] = 0.0
        x = x * np.repeat(np.repeat(f, 128, axis=0)[:rows], 32, axis=1)
    return x.astype(np.float32)


def run(x, qb, sb, a_fmt, b_fmt, out, b_gran="tile", ldx=None, alpha=1.0, c=None, beta=0.0):
    import torch
    if ldx is None:
        xd = to_dev(x)
    else:
        buf = np.zeros((x.shape[0], ldx), dtype=np.float32)
        buf[:, : x.shape[1]] = x
        xd = to_dev(buf)[:, : x.shape[1]]
    d, qa, sa = bsfp8().scaled_gemm_quantize_a(xd, to_dev(qb), to_dev(sb), a_fmt, b_fmt, b_gran,
                                               out, alpha, c, beta, return_a=True)
    torch.cuda.synchronize()
    return from_dev(d), from_dev(qa), from_dev(sa)


def b_operand(seed, N, K, fmt, gran="tile", kind="laplace"):
    b = inputs(seed, N, K, kind)
    return oracle.fp8_quantize_granular(b, fmt, gran)


def check_codes(qa, sa, x, fmt, label):
    rq, rs = oracle.fp8_quantize(x, fmt)
    assert np.array_equal(qa, rq), f"{label}: {np.count_nonzero(qa != rq)} A codes differ"
    assert np.array_equal(sa.view(np.uint32), rs.view(np.uint32)), f"{label}: A scales differ"
    return rq, rs


SHAPES = [(100, 72, 96), (256, 256, 128), (300, 260, 320), (1, 1, 32), (513, 200, 1056),
          (129, 385, 224), (128, 128, 4096)]


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_online_a_parity(M, N, K, out):
    say(f"scaled_gemm_quantize_a e4m3 x e5m2 M={M} N={N} K={K} -> {out}")
    x = inputs(M * 3 + K, M, K, "normal" if out == "f16" else "tiles")
    qb, sb = b_operand(N + 5, N, K, "e5m2")
    d, qa, sa = run(x, qb, sb, "e4m3", "e5m2", out)
    rq, rs = check_codes(qa, sa, x, "e4m3", f"{M}x{N}x{K}")
    dr, sr = oracle.gemm_granular("e4m3", rq, rs, "tile", "e5m2", qb, sb, "tile")
    check_gemm(d, dr, sr, out, f"online A {M}x{N}x{K} {out}")


@pytest.mark.parametrize("fmts", [("e5m2", "e4m3"), ("e4m3", "e4m3"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("b_gran", ["tile", "tensor"])
def test_online_a_formats_and_b_granularity(fmts, b_gran):
    a_fmt, b_fmt = fmts
    M, N, K = 384, 320, 544
    say(f"scaled_gemm_quantize_a {a_fmt} x {b_fmt} B {b_gran}")
    x = inputs(71, M, K, "tiles")
    qb, sb = b_operand(72, N, K, b_fmt, b_gran, "normal")
    for out in ("f32", "bf16"):
        d, qa, sa = run(x, qb, sb, a_fmt, b_fmt, out, b_gran)
        rq, rs = check_codes(qa, sa, x, a_fmt, f"{a_fmt} {b_gran}")
        dr, sr = oracle.gemm_granular(a_fmt, rq, rs, "tile", b_fmt, qb, sb, b_gran)
        check_gemm(d, dr, sr, out, f"online A {a_fmt} x {b_fmt} B {b_gran} {out}")


def test_online_a_padded_rows_and_edge_values():
    """x with a leading dimension larger than K; saturation, ties, subnormal
    codes and negative zero inside one tile."""
    M, N, K = 130, 96, 160
    x = inputs(81, M, K)
    x[0, :6] = [448.0, -448.0, 1e-30, -0.0, 3.0, 1000.0]
    x[1, :4] = [1.0, 1.0625, 1.1875, -2.0 ** -9]
    x[129, 32:64] = 0.0
    x[129, 64] = -0.0
    qb, sb = b_operand(82, N, K, "e4m3", kind="normal")
    for a_fmt in ("e4m3", "e5m2"):
        say(f"scaled_gemm_quantize_a padded ldx {a_fmt}")
        d, qa, sa = run(x, qb, sb, a_fmt, "e4m3", "f32", ldx=K + 36)
        rq, rs = check_codes(qa, sa, x, a_fmt, f"padded {a_fmt}")
        dr, sr = oracle.gemm_granular(a_fmt, rq, rs, "tile", "e4m3", qb, sb, "tile")
        check_gemm(d, dr, sr, "f32", f"padded {a_fmt}")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_online_a_alpha_beta(out):
    import torch
    M, N, K = 270, 300, 192
    x = inputs(91, M, K)
    qb, sb = b_operand(92, N, K, "e4m3", kind="normal")
    c32 = np.random.default_rng(93).standard_normal((M, N)).astype(np.float32) * 50
    if out == "bf16":
        cdev = torch.from_numpy(c32).to(torch.bfloat16)
        c = cdev.float().numpy()
    else:
        dt = np.float32 if out == "f32" else np.float16
        cdev = torch.from_numpy(c32.astype(dt))
        c = c32.astype(dt).astype(np.float64)
    say(f"scaled_gemm_quantize_a alpha/beta {out}")
    d, qa, sa = run(x, qb, sb, "e4m3", "e4m3", out, alpha=-0.75, c=cdev.cuda(), beta=1.5)
    rq, rs = check_codes(qa, sa, x, "e4m3", "alpha/beta")
    dr, sr = oracle.gemm_granular("e4m3", rq, rs, "tile", "e4m3", qb, sb, "tile")
    check_gemm_ex(d, dr, sr, -0.75, 1.5, c, out, f"online A alpha/beta {out}")


def test_online_a_without_code_output_and_degenerate_sizes():
    """No A copies requested; K = 0 writes beta C; N = 0 still writes the codes."""
    import torch
    b_ = bsfp8()
    M, N, K = 200, 136, 256
    x = inputs(101, M, K)
    qb, sb = b_operand(102, N, K, "e4m3", kind="normal")
    say("scaled_gemm_quantize_a without code output")
    d = b_.scaled_gemm_quantize_a(to_dev(x), to_dev(qb), to_dev(sb), "e4m3", "e4m3", "tile", "bf16")
    torch.cuda.synchronize()
    rq, rs = oracle.fp8_quantize(x, "e4m3")
    dr, sr = oracle.gemm_granular("e4m3", rq, rs, "tile", "e4m3", qb, sb, "tile")
    check_gemm(from_dev(d), dr, sr, "bf16", "online A, no code output")

    say("scaled_gemm_quantize_a K = 0")
    c = torch.full((M, N), 2.0, dtype=torch.float32, device="cuda")
    d0 = b_.scaled_gemm_quantize_a(torch.empty((M, 0), device="cuda"), torch.empty((N, 0), dtype=torch.uint8, device="cuda"),
                                   torch.empty((2, 0), device="cuda"), out="f32", c=c, beta=0.5)
    torch.cuda.synchronize()
    assert np.all(from_dev(d0) == 1.0)

    say("scaled_gemm_quantize_a N = 0")
    _, qa, sa = b_.scaled_gemm_quantize_a(to_dev(x), torch.empty((0, K), dtype=torch.uint8, device="cuda"),
                                          torch.empty((0, K // 32), device="cuda"), return_a=True)
    torch.cuda.synchronize()
    check_codes(from_dev(qa), from_dev(sa), x, "e4m3", "N = 0")


def test_online_a_matches_quantise_then_gemm_bitwise():
    """Consistency of the two HIP paths (not a parity check; the oracle tests
    above are): the same codes go through the same accumulation, so D is the
    same bits as fp8_quantize followed by scaled_gemm.  The shape has 36 tiles
    of 128 x 128, so scaled_gemm takes the 128 x 128 kernel as well (below 32
    tiles it takes the skinny kernel, whose K split sums in another order)."""
    import torch
    b_ = bsfp8()
    M, N, K = 768, 768, 1184
    x = to_dev(inputs(111, M, K, "tiles"))
    qb, sb = b_operand(112, N, K, "e4m3", kind="normal")
    qbd, sbd = to_dev(qb), to_dev(sb)
    for out in ("f32", "bf16"):
        say(f"scaled_gemm_quantize_a vs quantise + scaled_gemm {out}")
        d1 = b_.scaled_gemm_quantize_a(x, qbd, sbd, "e4m3", "e4m3", "tile", out)
        qa, sa = b_.fp8_quantize(x, "e4m3")
        d2 = b_.scaled_gemm(qa, sa, qbd, sbd, "e4m3", "e4m3", out)
        torch.cuda.synchronize()
        assert torch.equal(d1.view(torch.int16 if out == "bf16" else torch.int32),
                           d2.view(torch.int16 if out == "bf16" else torch.int32))


def test_online_a_square_4096_full_codes_sampled_outputs():
    """The 4096^3 launch of the square workload: all 16.8M A codes and 4096
    scales byte-equal to the oracle's, and sampled outputs within tolerance."""
    w = workloads.by_name("square_e4m3_4096")
    a, b = workloads.operands(w)
    qb, sb = oracle.fp8_quantize(b, "e4m3")
    say("scaled_gemm_quantize_a square 4096^3 bf16")
    d, qa, sa = run(a, qb, sb, "e4m3", "e4m3", "bf16")
    rq, rs = check_codes(qa, sa, a, "e4m3", "square 4096")
    rng = np.random.default_rng(121)
    ii = np.concatenate([rng.integers(0, 4096, 300), [0, 4095, 127, 128]])
    jj = np.concatenate([rng.integers(0, 4096, 300), [4095, 0, 128, 127]])
    dr, sr = oracle.gemm_points("e4m3", rq, rs, "e4m3", qb, sb, ii, jj)
    err = np.abs(d[ii, jj].astype(np.float64) - dr) / sr
    say(f"sampled max |D-Dref|/S = {err.max():.3e}")
    assert err.max() <= TOL["bf16"]


@pytest.mark.parametrize("M,N,K,out", [(256, 1024, 512, "bf16"), (130, 700, 288, "f32"),
                                       (4096, 4096, 4096, "bf16")])
def test_online_a_wide_output_single_launch(M, N, K, out):
    """Without code output every shape runs the single-launch kernel; at
    4096^3 (the square workload's launch) outputs are sampled."""
    import torch
    say(f"scaled_gemm_quantize_a single launch M={M} N={N} K={K} -> {out}")
    if M == 4096:
        w = workloads.by_name("square_e4m3_4096")
        x, bh = workloads.operands(w)
        qb, sb = oracle.fp8_quantize(bh, "e4m3")
    else:
        x = inputs(M + N + K, M, K, "tiles")
        qb, sb = b_operand(N + 9, N, K, "e4m3", kind="normal")
    d = bsfp8().scaled_gemm_quantize_a(to_dev(x), to_dev(qb), to_dev(sb), "e4m3", "e4m3", "tile", out)
    torch.cuda.synchronize()
    d = from_dev(d)
    rq, rs = oracle.fp8_quantize(x, "e4m3")
    if M == 4096:
        rng = np.random.default_rng(131)
        ii = np.concatenate([rng.integers(0, M, 300), [0, M - 1, 127, 128]])
        jj = np.concatenate([rng.integers(0, N, 300), [N - 1, 0, 128, 127]])
        dr, sr = oracle.gemm_points("e4m3", rq, rs, "e4m3", qb, sb, ii, jj)
        err = np.abs(d[ii, jj].astype(np.float64) - dr) / sr
        say(f"sampled max |D-Dref|/S = {err.max():.3e}")
        assert err.max() <= TOL[out]
    else:
        dr, sr = oracle.gemm_granular("e4m3", rq, rs, "tile", "e4m3", qb, sb, "tile")
        check_gemm(d, dr, sr, out, f"single launch {M}x{N}x{K} {out}")
