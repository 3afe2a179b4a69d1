"""The Python binding's argument checks.

The C ABI takes plain pointers and sizes; the binding derives those sizes
from the tensors it is given.  A tensor that does not hold what the sizes say
(wrong dtype, wrong device, a column-sliced code matrix, an undersized scale
array, a D with too few rows) must raise ValueError before anything is
launched, never reach a kernel.  The CPU tests check the rejections that need
no device; the GPU tests check the rest and that the outputs they were given
are left untouched."""
import numpy as np
import pytest

import block_scaled_precision_fp8_amd as bs


# ------------------------------------------------------------------ CPU only
def test_cpu_tensors_are_rejected():
    import torch
    x = torch.zeros((128, 64), dtype=torch.float32)
    q = torch.zeros((128, 64), dtype=torch.uint8)
    s = torch.ones((1, 2), dtype=torch.float32)
    calls = [
        lambda: bs.fp8_quantize(x),
        lambda: bs.fp8_quantize_pair(x, x),
        lambda: bs.fp8_quantize_transposed(x),
        lambda: bs.fp8_quantize_granular(x, "e4m3", "row"),
        lambda: bs.mxfp4_quantize(x),
        lambda: bs.mx_quantize(x, 16, "bf16"),
        lambda: bs.scaled_gemm(q, s, q, s),
        lambda: bs.scaled_gemm_ex(q, s, q, s),
        lambda: bs.scaled_gemm_granular(q, s, q, s),
        lambda: bs.scaled_gemm_mx(q[:, :32], s, q[:, :32], s, 16, "e8m0"),
        lambda: bs.scaled_gemm_quantize_a(x, q, s),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError):
            call()


def test_unknown_names_are_rejected():
    import torch
    q = torch.zeros((4, 32), dtype=torch.uint8)
    s = torch.ones((1, 1), dtype=torch.float32)
    with pytest.raises(ValueError, match="format"):
        bs.scaled_gemm(q, s, q, s, "e3m4", "e4m3")
    with pytest.raises(ValueError, match="mixed"):
        bs.scaled_gemm(q, s, q, s, "mxfp4", "e4m3")
    with pytest.raises(ValueError, match="granularity"):
        bs.scaled_gemm_granular(q, s, q, s, a_gran="block")


# ------------------------------------------------------------------ GPU
@pytest.mark.gpu
def test_gemm_argument_checks_launch_nothing():
    import torch
    from gpu_common import say
    say("binding checks: scaled_gemm family")
    dev = torch.device("cuda")
    M, N, K = 256, 192, 128
    a = torch.randint(0, 0x7E, (M, K), dtype=torch.uint8, device=dev)
    b = torch.randint(0, 0x7E, (N, K), dtype=torch.uint8, device=dev)
    sa = torch.ones((2, K // 32), dtype=torch.float32, device=dev)
    sb = torch.ones((2, K // 32), dtype=torch.float32, device=dev)
    d = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=dev)
    bad = [
        ("codes as int8", lambda: bs.scaled_gemm(a.view(torch.int8), sa, b, sb, d=d)),
        ("column-sliced a", lambda: bs.scaled_gemm(torch.zeros((M, 2 * K), dtype=torch.uint8, device=dev)[:, :K],
                                                   sa, b, sb, d=d)),
        ("K larger than a's rows", lambda: bs.scaled_gemm(a, sa, b, sb, d=d, K=2 * K)),
        ("undersized a_scales", lambda: bs.scaled_gemm(a, sa[:1], b, sb, d=d)),
        ("float64 scales", lambda: bs.scaled_gemm(a, sa.double(), b, sb, d=d)),
        ("d with too few rows", lambda: bs.scaled_gemm(a, sa, b, sb, d=d[: M - 1])),
        ("float32 d for bf16 output", lambda: bs.scaled_gemm(a, sa, b, sb, "e4m3", "e4m3", "bf16",
                                                             d=torch.zeros((M, N), device=dev))),
        ("d with a column stride", lambda: bs.scaled_gemm(a, sa, b, sb, d=torch.zeros(
            (M, 2 * N), dtype=torch.bfloat16, device=dev)[:, ::2])),
        ("beta without c", lambda: bs.scaled_gemm_ex(a, sa, b, sb, beta=1.0, d=d)),
        ("c of the wrong dtype", lambda: bs.scaled_gemm_ex(a, sa, b, sb, beta=1.0, d=d,
                                                           c=torch.zeros((M, N), device=dev))),
        ("per-row scales too short", lambda: bs.scaled_gemm_granular(
            a, sa.reshape(-1)[: M - 1], b, sb, a_gran="row", b_gran="row", d=d)),
        ("MXFP4 scales too short", lambda: bs.scaled_gemm(
            a[:, : K // 2], torch.zeros(M * K // 32 - 1, dtype=torch.uint8, device=dev),
            b[:, : K // 2], torch.zeros(N * K // 32, dtype=torch.uint8, device=dev), "mxfp4", "mxfp4", d=d)),
    ]
    for what, call in bad:
        say(f"  expect ValueError: {what}")
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
    assert torch.all(d == 7.0), "a rejected call wrote its output"


@pytest.mark.gpu
def test_quantiser_argument_checks_launch_nothing():
    import torch
    from gpu_common import say
    say("binding checks: quantisers")
    dev = torch.device("cuda")
    rows, k = 200, 96
    x = torch.randn((rows, k), device=dev)
    codes = torch.full((rows, k), 0x55, dtype=torch.uint8, device=dev)
    scales = torch.full((2, k // 32), 3.0, device=dev)
    bad = [
        ("float16 x", lambda: bs.fp8_quantize(x.half(), codes=codes, scales=scales)),
        ("x with a column stride", lambda: bs.fp8_quantize(torch.randn((rows, 2 * k), device=dev)[:, ::2],
                                                          codes=codes, scales=scales)),
        ("codes too short", lambda: bs.fp8_quantize(x, codes=codes[: rows - 1], scales=scales)),
        ("codes column-sliced", lambda: bs.fp8_quantize(
            x, codes=torch.zeros((rows, 2 * k), dtype=torch.uint8, device=dev)[:, :k], scales=scales)),
        ("scales too short", lambda: bs.fp8_quantize(x, codes=codes, scales=scales[:1])),
        ("unknown format", lambda: bs.fp8_quantize(x, "e4m4", codes=codes, scales=scales)),
        ("pair with different K", lambda: bs.fp8_quantize_pair(x, x[:, :64], a_codes=codes, a_scales=scales)),
        ("per-row scales too short", lambda: bs.fp8_quantize_granular(
            x, "e4m3", "row", codes=codes, scales=torch.zeros(rows - 1, device=dev))),
        ("MXFP4 packed too narrow", lambda: bs.mxfp4_quantize(
            x, packed=torch.zeros((rows, k // 2 - 16), dtype=torch.uint8, device=dev))),
        ("MX scales of the wrong width", lambda: bs.mx_quantize(
            x, 16, "bf16", scales=torch.zeros((rows, k // 16), dtype=torch.float32, device=dev))),
        ("block of 4", lambda: bs.mx_quantize(x, 4)),
    ]
    for what, call in bad:
        say(f"  expect ValueError: {what}")
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
    assert torch.all(codes == 0x55) and torch.all(scales == 3.0), "a rejected call wrote its outputs"
