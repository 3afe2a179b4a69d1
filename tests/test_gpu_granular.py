"""Parity of the FP8 scale granularities ("Why grind FP8 GEMM on CDNA4",
section 3.3: per row, per column, per tensor, per tile) on the GPU.

* fp8_quantize_granular: codes and scales byte-equal to the oracle's, per row
  and per tensor, on ragged, padded, short and long rows.
* scaled_gemm_granular: every supported combination against the oracle's
  fp64 product, max |D - D_ref| / S within the output type's tolerance:
  both scales constant along K (the K = 64 outer-scaled kernel), per-tile with
  per-tensor (the per-tile kernel), with alpha / beta and ragged M, N, K
  (including K % 64 == 32, which pads the last stage).  Operand codes and
  scales come from the oracle's quantiser; one end-to-end case per
  combination also runs the HIP quantiser.
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


def gpu_quant(x, fmt, gran, ld=None):
    import torch
    if ld is None:
        xd = to_dev(x)
    else:
        buf = np.zeros((x.shape[0], ld), dtype=np.float32)
        buf[:, : x.shape[1]] = x
        xd = to_dev(buf)[:, : x.shape[1]]
    q, s = bsfp8().fp8_quantize_granular(xd, fmt, gran)
    torch.cuda.synchronize()
    return from_dev(q), from_dev(s)


def inputs(seed, rows, k, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "laplace":
        return (rng.laplace(size=(rows, k)) * 1e-3).astype(np.float32)
    if kind == "wide":   # each row at its own magnitude, some all-zero rows
        x = rng.standard_normal((rows, k)) * np.exp2(rng.integers(-30, 30, size=(rows, 1)))
        x[rng.random(rows) < 0.1] = 0.0
        return x.astype(np.float32)
    return rng.standard_normal((rows, k)).astype(np.float32)


# ---------------------------------------------------------------- quantiser
@pytest.mark.parametrize("gran", ["row", "tensor"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,k,ld,kind", [
    (1, 32, None, "normal"), (3, 64, 96, "normal"), (130, 288, None, "wide"),
    (257, 4096, None, "laplace"), (5, 8192, None, "wide"), (64, 4128, None, "normal"),
    (9, 12320, 12352, "wide"), (6, 4064, 4100, "normal"),
])
def test_quantize_granular_matches_oracle(gran, fmt, rows, k, ld, kind):
    say(f"fp8_quantize_granular {gran} {fmt} rows={rows} k={k} ld={ld} {kind}")
    x = inputs(rows * 7 + k, rows, k, kind)
    q, s = gpu_quant(x, fmt, gran, ld)
    rq, rs = oracle.fp8_quantize_granular(x, fmt, gran)
    assert np.array_equal(q, rq), f"{np.count_nonzero(q != rq)} codes differ"
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("gran", ["row", "tensor"])
def test_quantize_granular_edge_values(gran):
    """Saturation, the E4M3 maximum, ties and subnormal codes, negative zero."""
    x = np.zeros((4, 64), dtype=np.float32)
    x[0, :6] = [448.0, -448.0, 1e-30, -0.0, 3.0, 1000.0]
    x[1, :4] = [1.0, 1.0625, 1.1875, -2.0 ** -9]
    x[2] = np.linspace(-1, 1, 64, dtype=np.float32)
    for fmt in ("e4m3", "e5m2"):
        q, s = gpu_quant(x, fmt, gran)
        rq, rs = oracle.fp8_quantize_granular(x, fmt, gran)
        assert np.array_equal(q, rq) and np.array_equal(s.view(np.uint32), rs.view(np.uint32))


# ---------------------------------------------------------------- GEMM
def run_gemm(qa, sa, ga, qb, sb, gb, a_fmt, b_fmt, out, K, alpha=1.0, c=None, beta=0.0):
    import torch
    cd = None if c is None else to_dev(c)
    d = bsfp8().scaled_gemm_granular(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), a_fmt, b_fmt,
                                     ga, gb, out, alpha, cd, beta, None, K)
    torch.cuda.synchronize()
    return from_dev(d)


COMBOS = [("row", "row"), ("row", "tensor"), ("tensor", "row"), ("tensor", "tensor"),
          ("tile", "tensor"), ("tensor", "tile"), ("tile", "row"), ("row", "tile")]


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("ga,gb", COMBOS)
@pytest.mark.parametrize("M,N,K", [(100, 72, 96), (256, 256, 64), (300, 260, 320), (1, 1, 32), (48, 300, 640),
                                   (16, 2050, 4128),
                                   (513, 200, 1056)])
def test_granular_gemm_parity(ga, gb, M, N, K, out):
    say(f"scaled_gemm_granular {ga}x{gb} M={M} N={N} K={K} -> {out}")
    # rows at their own magnitudes (up to 2^30) would overflow FP16 output
    a = inputs(M + 1, M, K, "wide" if ga == "row" and out != "f16" else "normal")
    b = inputs(N + 2, N, K, "laplace")
    qa, sa = oracle.fp8_quantize_granular(a, "e4m3", ga)
    qb, sb = oracle.fp8_quantize_granular(b, "e5m2", gb)
    d = run_gemm(qa, sa, ga, qb, sb, gb, "e4m3", "e5m2", out, K)
    dr, sr = oracle.gemm_granular("e4m3", qa, sa, ga, "e5m2", qb, sb, gb)
    check_gemm(d, dr, sr, out, f"{ga}x{gb} {M}x{N}x{K} {out}")


@pytest.mark.parametrize("fmts", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e5m2", "e4m3")])
def test_granular_gemm_formats(fmts):
    a_fmt, b_fmt = fmts
    M, N, K = 384, 320, 512
    a = inputs(11, M, K)
    b = inputs(12, N, K, "wide")
    qa, sa = oracle.fp8_quantize_granular(a, a_fmt, "row")
    qb, sb = oracle.fp8_quantize_granular(b, b_fmt, "row")
    for out in ("f32", "bf16"):
        d = run_gemm(qa, sa, "row", qb, sb, "row", a_fmt, b_fmt, out, K)
        dr, sr = oracle.gemm_granular(a_fmt, qa, sa, "row", b_fmt, qb, sb, "row")
        check_gemm(d, dr, sr, out, f"row x row {a_fmt}x{b_fmt} {out}")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("ga,gb", [("row", "row"), ("tile", "tensor"), ("tile", "row"), ("row", "tile")])
@pytest.mark.parametrize("M,N,K", [(270, 300, 192), (40, 300, 640)])   # the second: skinny kernel
def test_granular_alpha_beta(ga, gb, out, M, N, K):
    import torch
    a = inputs(21, M, K)
    b = inputs(22, N, K)
    qa, sa = oracle.fp8_quantize_granular(a, "e4m3", ga)
    qb, sb = oracle.fp8_quantize_granular(b, "e4m3", gb)
    dt = {"f32": np.float32, "bf16": None, "f16": np.float16}[out]
    c32 = np.random.default_rng(23).standard_normal((M, N)).astype(np.float32) * 50
    if out == "bf16":
        c = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()
        cdev = torch.from_numpy(c32).to(torch.bfloat16)
    else:
        c = c32.astype(dt).astype(np.float64)
        cdev = torch.from_numpy(c32.astype(dt))
    import block_scaled_precision_fp8_amd as bb
    d = bb.scaled_gemm_granular(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), "e4m3", "e4m3", ga, gb, out,
                                -0.75, cdev.cuda(), 1.5, None, K)
    torch.cuda.synchronize()
    dr, sr = oracle.gemm_granular("e4m3", qa, sa, ga, "e4m3", qb, sb, gb)
    check_gemm_ex(from_dev(d), dr, sr, -0.75, 1.5, c, out, f"alpha/beta {ga}x{gb} {out}")


@pytest.mark.parametrize("ga,gb", COMBOS)
def test_granular_end_to_end(ga, gb):
    """HIP quantiser then HIP GEMM, against the oracle on the same FP32 inputs."""
    M, N, K = 640, 512, 1024
    a = inputs(31, M, K)
    b = inputs(32, N, K, "laplace")
    import torch
    b_ = bsfp8()
    qa, sa = b_.fp8_quantize_granular(to_dev(a), "e4m3", ga)
    qb, sb = b_.fp8_quantize_granular(to_dev(b), "e4m3", gb)
    d = b_.scaled_gemm_granular(qa, sa, qb, sb, "e4m3", "e4m3", ga, gb, "bf16")
    torch.cuda.synchronize()
    rqa, rsa = oracle.fp8_quantize_granular(a, "e4m3", ga)
    rqb, rsb = oracle.fp8_quantize_granular(b, "e4m3", gb)
    assert np.array_equal(from_dev(qa), rqa) and np.array_equal(from_dev(qb), rqb)
    dr, sr = oracle.gemm_granular("e4m3", rqa, rsa, ga, "e4m3", rqb, rsb, gb)
    check_gemm(from_dev(d), dr, sr, "bf16", f"end to end {ga}x{gb}")


def test_square_4096_row_column_scales_sampled():
    """The 4096^3 shape of the square workload with per-row A and per-column B
    scales: the full launch the benchmark times, checked on sampled outputs."""
    import torch
    w = workloads.by_name("square_e4m3_4096")
    a, b = workloads.operands(w)
    qa, sa = oracle.fp8_quantize_granular(a, "e4m3", "row")
    qb, sb = oracle.fp8_quantize_granular(b, "e4m3", "row")
    say("scaled_gemm_granular row x row 4096^3 bf16")
    d = run_gemm(qa, sa, "row", qb, sb, "row", "e4m3", "e4m3", "bf16", 4096)
    rng = np.random.default_rng(41)
    ii = np.concatenate([rng.integers(0, 4096, 200), [0, 4095, 255, 256]])
    jj = np.concatenate([rng.integers(0, 4096, 200), [4095, 0, 256, 255]])
    ad = oracle.dequantize_granular("e4m3", qa[ii], sa[ii], "row")
    bd = oracle.dequantize_granular("e4m3", qb[jj], sb[jj], "row")
    dr = np.sum(ad * bd, axis=1)
    sr = np.sum(np.abs(ad * bd), axis=1)
    err = np.abs(d[ii, jj].astype(np.float64) - dr) / sr
    say(f"sampled max |D-Dref|/S = {err.max():.3e}")
    assert err.max() <= TOL["bf16"]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("ga,gb", [("tile", "tensor"), ("tensor", "tile"), ("tile", "row"), ("row", "tile")])
def test_granular_large_tile_kernel(ga, gb, out):
    """Per-tile with per-tensor or per-row scales on a shape with enough
    256 x 256 tiles for the large-tile per-tile kernel (ragged M and N, a
    partial K stage)."""
    M, N, K = 3000, 4200, 160
    say(f"scaled_gemm_granular {ga}x{gb} M={M} N={N} K={K} -> {out} (large-tile kernel)")
    a = inputs(31, M, K)
    b = inputs(32, N, K, "laplace")
    qa, sa = oracle.fp8_quantize_granular(a, "e4m3", ga)
    qb, sb = oracle.fp8_quantize_granular(b, "e5m2", gb)
    d = run_gemm(qa, sa, ga, qb, sb, gb, "e4m3", "e5m2", out, K)
    dr, sr = oracle.gemm_granular("e4m3", qa, sa, ga, "e5m2", qb, sb, gb)
    check_gemm(d, dr, sr, out, f"{ga}x{gb} {M}x{N}x{K} {out} large tile")
