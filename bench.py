"""Benchmark of the block-scaled FP8 / MXFP4 hot path on one MI355X.

One step = one pass of the whole hot path over the workload's operands, which
are resident in HBM before the timed region starts:
    FP8 workloads:   fp8_quantize_pair(A, B) (both operands in one launch), scaled_gemm
    MXFP4 workload:  mxfp4_quantize(A), mxfp4_quantize(B), scaled_gemm
value = 2 M N K / (step time), in TFLOP/s, for the whole job.  The default
workload is the largest single-GPU one, the Transformer feed-forward shape
(M = 16384 tokens, N = 14336, K = 4096, E4M3, bf16 output).

Inputs are rotated: the step cycles through several independent sets of
operand, code, scale and output buffers, together larger than the 256 MB
last-level (MALL) cache, so that no step reads what an earlier step left in
that cache.

Also reported, on the same JSON line:
  roofline      the GEMM kernel: algorithmic FLOPs per launch / its average
                launch time (HIP events on the launch stream, over the timed
                steps), against the dense MFMA peak of the input type;
                traffic = HBM bytes per launch from the committed rocprofv3
                counter summary when it was taken on the current kernel source,
                else null;
  cpu_baseline  the CPU oracle (plain C, fp64) on a bounded sample of the same
                step, extrapolated to the whole job;
  kernels       per-kernel times (mean and median over the timed steps), GEMM
                TFLOP/s, quantiser GB/s against 8 TB/s;
  gpu           compute-unit count; the GEMM kernel's shader clock,
                matrix-core busy fraction and VALU instructions per MFMA from
                the committed rocprofv3 counter summary when it was taken on
                the current kernel source.

--mfma-rates prints instead the sustained rate and shader clock of the matrix
instructions the GEMMs use (the test instrument in tests/mfma_probe), one JSON
line per case.

FP8 workloads can also be run with scales constant along K
(--granularity row: per-row A and per-column B, or tensor: one scale per
operand); the step then uses fp8_quantize_granular and scaled_gemm_granular.
With --a-path online (per-tile scales) A is quantised inside the GEMM:
fp8_quantize(B), scaled_gemm_quantize_a(A) without code output.
The MXFP4 workload can also be run with blocks of 16 or 8 elements and with
FP16 / BF16 block scales (--mx-block, --mx-scale): mx_quantize(A),
mx_quantize(B), scaled_gemm_mx.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--granularity tile|row|tensor] [--a-path separate|online]
                       [--mx-block 32|16|8] [--mx-scale e8m0|f16|bf16] [--no-cpu-baseline]
                       [--copy-calibration] [--mfma-rates] [--rotate-mib MIB]
Only one GPU is supported; --gpus N with N > 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scaled-GEMM TFLOP/s and % of MI355X FP8/MXFP4 MFMA peak at 1 GPU"
PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0, "bf16": 2500.0}
HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "ffn_e4m3_16384x14336x4096"
ROTATE_MIB = 768         # rotated input sets span at least this much (MALL: 256 MB)
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(workload, source_file):
    """HBM bytes per GEMM launch from profiles/<kernel>_<workload>_traffic.txt,
    only if it was measured on the current kernel source (digest line)."""
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None, None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    digest = kernel_source_digest(source_file)
    if fields.get("kernel_source_sha256_16") != digest:
        return None, "stale (kernel changed since the counters were taken)"
    try:
        return float(fields["hbm_bytes_per_launch"]), path
    except (KeyError, ValueError):
        return None, None


def committed_counters(workload, source_file):
    """The GEMM kernel's shader clock, matrix-core busy fraction and VALU
    instructions per MFMA from profiles/counters_<workload>.txt (rocprofv3
    counters: GRBM_GUI_ACTIVE over the dispatch time, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_VALU / SQ_INSTS_MFMA), only if they were taken on the current
    kernel source.  Clock and power sensors read by rocm-smi or amdsmi do not
    follow a running kernel on this machine, so the counters stand in for them."""
    path = os.path.join(PROFILES, f"counters_{workload}.txt")
    if not os.path.exists(path):
        return {}
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_digest(source_file):
        return {"counters": "stale (kernel changed since the counters were taken)"}
    out = {"counters_source": os.path.relpath(path, ROOT)}
    for k in ("shader_clock_ghz", "mfma_busy_frac", "valu_per_mfma", "lds_bank_conflict_frac"):
        try:
            out[k] = float(fields[k])
        except (KeyError, ValueError):
            pass
    return out


def mx_fp4_kernel(w, block):
    """The MXFP4 kernel that E8M0 blocks of 16 or 8 run on (one FP4 MFMA per
    block), or None where they stay on a dequantising kernel (mirrors the
    library's dispatch)."""
    big_tiles = ((w.M + 255) // 256) * ((w.N + 255) // 256)
    if w.M <= 64 or ((w.M + 127) // 128) * ((w.N + 127) // 128) < 32:
        return "gemm_mxfp4_skinny_kernel"
    if (w.K % 256 == 0 and big_tiles >= 64 and
            w.M * (w.K // 2) < 2**31 and w.N * (w.K // 2) < 2**31):
        return "gemm_mxfp4_big_kernel"
    return "gemm_mxfp4_kernel" if big_tiles < 128 or block == 16 else None


def gemm_kernel_name(w, gran="tile", online=False, mx_variant=False, mx_block=32):
    """The kernel scaled_gemm dispatches for this workload (mirrors the
    launchers' selection)."""
    skinny = w.M <= 64 or ((w.M + 127) // 128) * ((w.N + 127) // 128) < 32
    if mx_variant:
        if mx_variant == "e8m0_fp4":
            return mx_fp4_kernel(w, mx_block)
        if skinny:
            return "gemm_mx_skinny_kernel"
        if ((w.M + 255) // 256) * ((w.N + 255) // 256) >= 128:
            return "gemm_mx_split_big_kernel" if mx_variant == "wide" else "gemm_mx_big_kernel"
        return "gemm_mx_kernel"
    if online:
        return "gemm_fp8_kernel (A quantised by quantiser waves)"
    if w.a_fmt != "mxfp4" and gran != "tile":
        return "gemm_fp8_outer_kernel"
    if skinny:
        return "gemm_mxfp4_skinny_kernel" if w.a_fmt == "mxfp4" else "gemm_fp8_skinny_kernel"
    if w.a_fmt == "mxfp4":
        big_tiles = ((w.M + 255) // 256) * ((w.N + 255) // 256)
        fits32 = w.M * (w.K // 2) < 2**31 and w.N * (w.K // 2) < 2**31
        if big_tiles >= 64 and fits32:
            return "gemm_mxfp4_big_kernel" if w.K % 256 == 0 else "gemm_mxfp4_ring_kernel"
        return "gemm_mxfp4_kernel"
    big_tiles = ((w.M + 255) // 256) * ((w.N + 255) // 256)
    if w.K < 2**23 and big_tiles >= 192:
        return "gemm_fp8_big_kernel"
    return "gemm_fp8_kernel"


def gemm_bytes(w, gran="tile", mx_block=32, mx_scale="e8m0", mx=False):
    """Algorithmic HBM bytes of one GEMM launch: the codes of A and B, their
    scales, and D (each read or written once)."""
    out_b = 4 if w.out == "f32" else 2
    if mx:
        sbytes = 1 if mx_scale == "e8m0" else 2
        return (w.M + w.N) * (w.K // 2 + (w.K // mx_block) * sbytes) + w.M * w.N * out_b
    nsc = {"tile": lambda r: ((r + 127) // 128) * (w.K // 32), "row": lambda r: r,
           "tensor": lambda r: 1}[gran]
    return (w.M + w.N) * w.K + (nsc(w.M) + nsc(w.N)) * 4 + w.M * w.N * out_b


def cpu_baseline(w, a, b, st, sample_rows, gran="tile", mx_block=32, mx_scale="e8m0",
                 token_major=False):
    """Time the oracle on a bounded sample: quantise all of B and `sample_rows`
    rows of A (whole 128-row tiles spread evenly over A), and compute the
    product rows of that sample; extrapolate the time to the whole step
    (quantising all of A, all M rows of D).  With per-row or per-tensor scales
    all of A is quantised (a per-tensor scale needs every row) and only the
    product is sampled.  The GPU's codes and D on the same rows (from `st`, the
    last step's buffers) are compared with the oracle's."""
    import numpy as np
    import oracle

    cores = oracle.threads()
    tiles = sample_tiles(w.M, sample_rows)
    idx = np.concatenate([np.arange(t, min(t + 128, w.M)) for t in tiles])
    rows = idx.size
    d_gpu = st["d"][idx.tolist()].float().cpu().numpy() if rows < w.M else st["d"].float().cpu().numpy()
    where = (f"A row tiles {tiles[0] // 128}, {tiles[1] // 128 if len(tiles) > 1 else ''}... "
             f"(every {max(1, (tiles[1] - tiles[0]) // 128) if len(tiles) > 1 else 1}th of "
             f"{(w.M + 127) // 128}, {len(tiles)} tiles, {rows} rows)")
    if gran != "tile" and w.a_fmt != "mxfp4":
        t0 = time.perf_counter()
        qb, sb = oracle.fp8_quantize_granular(b, w.b_fmt, gran)
        qa, sa = oracle.fp8_quantize_granular(a, w.a_fmt, gran)
        t1 = time.perf_counter()
        sa_rows = sa[idx] if gran == "row" else sa
        d_ref, s_ref = oracle.gemm_granular(w.a_fmt, qa[idx], sa_rows, gran, w.b_fmt, qb, sb, gran)
        t2 = time.perf_counter()
        scale = w.M / rows
        t_full = (t1 - t0) + (t2 - t1) * scale
        codes_equal = bool(np.array_equal(st["qa"].cpu().numpy(), qa) and
                           np.array_equal(st["qb"].cpu().numpy(), qb))
        err = np.abs(d_gpu.astype(np.float64) - d_ref)
        nz = s_ref > 0
        worst = float((err[nz] / s_ref[nz]).max()) if nz.any() else 0.0
        return {
            "value": w.flops / t_full / 1e12,
            "unit": "TFLOP/s",
            "cores": cores,
            "kind": "oracle",
            "sample": (f"oracle {gran} quantise of all of A and B, oracle fp64 product of {where} "
                       f"x {w.N} columns; measured {t2 - t0:.1f} s, extrapolated x{scale:g} on the "
                       f"product to the full {w.M}x{w.N}x{w.K} step"),
            "seconds_measured": round(t2 - t0, 3),
            "gpu_codes_bit_exact": codes_equal,
            "gpu_vs_oracle_max_err_over_S_on_sample": worst,
        }
    mxv = w.a_fmt == "mxfp4" and (mx_block != 32 or mx_scale != "e8m0")
    t0 = time.perf_counter()
    if mxv:
        qb, sb = oracle.mx_quantize(b, mx_block, mx_scale)
    elif w.a_fmt == "mxfp4":
        qb, sb = oracle.mxfp4_quantize(b)
    else:
        qb, sb = oracle.fp8_quantize(b, w.b_fmt)
    t1 = time.perf_counter()
    a_rows = np.ascontiguousarray(a[idx])
    if mxv:
        qa, sa = oracle.mx_quantize(a_rows, mx_block, mx_scale)
    elif w.a_fmt == "mxfp4":
        qa, sa = oracle.mxfp4_quantize(a_rows)
    else:
        qa, sa = oracle.fp8_quantize(a_rows, w.a_fmt)
    t2 = time.perf_counter()
    if mxv:
        d_ref, s_ref = oracle.gemm_mx(qa, sa, qb, sb, mx_block, mx_scale)
    else:
        d_ref, s_ref = oracle.gemm_rows(w.a_fmt, qa, sa, w.b_fmt, qb, sb)
    t3 = time.perf_counter()
    scale = w.M / rows
    t_full = (t1 - t0) + (t2 - t1) * scale + (t3 - t2) * scale
    value = w.flops / t_full / 1e12
    # the GPU's codes and scales of the same rows, and its D there
    qa_gpu = st["qa"][idx.tolist()].cpu().numpy()
    if w.a_fmt == "mxfp4" or gran != "tile":
        sa_gpu = st["sa"][idx.tolist()].cpu().numpy()
    else:
        sa_gpu = st["sa"][[t // 128 for t in tiles]].cpu().numpy()
    codes_equal = bool(np.array_equal(qa_gpu, qa) and np.array_equal(sa_gpu.view(sa.dtype), sa) and
                       np.array_equal(st["qb"].cpu().numpy(), qb) and
                       np.array_equal(st["sb"].cpu().numpy().view(sb.dtype), sb))
    err = np.abs(d_gpu.astype(np.float64) - d_ref)
    nz = s_ref > 0
    worst = float((err[nz] / s_ref[nz]).max()) if nz.any() else 0.0
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"oracle quantise of all of B ({w.N}x{w.K}) and of {where}, oracle fp64 product "
                   f"of those rows x {w.N} columns; measured {t3 - t0:.1f} s, extrapolated "
                   f"x{scale:g} on the A/product parts to the full {w.M}x{w.N}x{w.K} step"),
        "seconds_measured": round(t3 - t0, 3),
        "gpu_codes_bit_exact": codes_equal,
        "gpu_vs_oracle_max_err_over_S_on_sample": worst,
    }


def copy_calibration():
    """A plain device copy of known size, for scaling rocprofv3's HBM byte counters.
    The source is 1 GiB written before the copies start, so that the copies'
    reads come from HBM, not from the 256 MB last-level cache."""
    import torch
    n = 256 * 1024 * 1024          # 1 GiB of float32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 copies of {n * 4} bytes (read {n * 4}, write {n * 4} per copy)")


def mfma_rates():
    """Sustained issue rate and shader clock of the matrix instructions (the
    rate probe of tests/mfma_probe), one JSON line per case."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import mfma_probe as mp

    cases = [
        (mp.R_FP8_K16, mp.P_CHAINS, "random"), (mp.R_FP8_K16, mp.P_CHAINS, "zero"),
        (mp.R_SCALE_FP8_K64, mp.P_CHAINS, "random"), (mp.R_SCALE_FP8_K64, mp.P_CHAINS, "zero"),
        (mp.R_SCALE_FP4_K64, mp.P_CHAINS, "random"), (mp.R_SCALE_FP4_K64, mp.P_CHAINS, "zero"),
        (mp.R_BF16_K16, mp.P_CHAINS, "random"), (mp.R_FP8_16X16X32, mp.P_CHAINS, "random"),
        (mp.R_FP8_K16, mp.P_PROMOTE, "random"), (mp.R_FP8_K16, mp.P_PROMOTE, "zero"),
        (mp.R_FP8_16X16X32, mp.P_PROMOTE, "random"), (mp.R_BF16_K16, mp.P_PROMOTE, "random"),
        (mp.R_FP8_K16, mp.P_INTERLEAVE, "random"), (mp.R_FP8_K16, mp.P_INTERLEAVE, "zero"),
        (mp.R_FP8_16X16X32, mp.P_INTERLEAVE, "random"), (mp.R_BF16_K16, mp.P_INTERLEAVE, "random"),
        (mp.R_SCALE_FP8_K64, mp.P_INTERLEAVE, "random"),
    ]
    for instr, pattern, data in cases:
        for wps in ((1, 2) if pattern == mp.P_CHAINS else (1, 2, 3)):
            # about 50 ms per launch at 2.4 GHz: long enough for the clock to settle
            cyc = {mp.R_FP8_K16: 32, mp.R_SCALE_FP8_K64: 64, mp.R_SCALE_FP4_K64: 32,
                   mp.R_BF16_K16: 32, mp.R_FP8_16X16X32: 16}[instr]
            per_iter = cyc * (4 if pattern == mp.P_CHAINS else
                              {mp.R_FP8_K16: 8, mp.R_BF16_K16: 8, mp.R_FP8_16X16X32: 16}.get(instr, 4))
            iters = int(0.05 * 2.4e9 / (per_iter * wps))
            r = mp.rate(instr, pattern, data, waves_per_simd=wps, iters=iters)
            print(json.dumps(r), flush=True)


def sample_tiles(M, rows):
    """Row tiles of the CPU sample: `rows // 128` tiles spread evenly over the
    M / 128 row tiles of A (every s-th tile), as first-row indices."""
    tiles_m = (M + 127) // 128
    n = max(1, min(tiles_m, rows // 128))
    stride = max(1, tiles_m // n)
    return [t * 128 for t in range(0, tiles_m, stride)][:n]


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-gflop", type=float, default=650.0,
                   help="oracle product work to time (whole 128-row tiles spread over A)")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--mfma-rates", action="store_true",
                   help="print the matrix instructions' sustained rates and shader clock instead")
    p.add_argument("--rotate-mib", type=int, default=ROTATE_MIB,
                   help="rotate through input sets spanning at least this many MiB (at least 2 sets)")
    p.add_argument("--operand-layout", choices=["k-contiguous", "token-major"], default=None,
                   help="FP8 only: token-major stores A and B transposed (K x M, K x N, as the "
                        "gradient and activation of a weight-gradient product are) and quantises "
                        "them with fp8_quantize_transposed; default token-major for the dW "
                        "workload, k-contiguous otherwise")
    p.add_argument("--granularity", choices=["tile", "row", "tensor"], default="tile",
                   help="FP8 only: scale granularity of both operands (row = per-row A and "
                        "per-column B)")
    p.add_argument("--a-path", choices=["separate", "online"], default="separate",
                   help="FP8 per-tile only: online quantises A inside the GEMM "
                        "(scaled_gemm_quantize_a) instead of a separate fp8_quantize pass")
    p.add_argument("--mx-block", type=int, choices=[32, 16, 8], default=32,
                   help="MXFP4 only: elements per block scale")
    p.add_argument("--mx-scale", choices=["e8m0", "f16", "bf16"], default="e8m0",
                   help="MXFP4 only: block scale format")
    args = p.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on exactly one GPU; --gpus must be 1 "
              "(multi-GPU sharding is described in the design notes, not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_precision_fp8_amd as bs
    import workloads

    if args.copy_calibration:
        copy_calibration()
        return
    if args.mfma_rates:
        mfma_rates()
        return

    w = workloads.by_name(args.workload)
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: M={w.M} N={w.N} K={w.K} {w.a_fmt}x{w.b_fmt} -> {w.out}")
    a_host, b_host = workloads.operands(w)
    mx = w.a_fmt == "mxfp4"
    gran = "tile" if mx else args.granularity
    layout = args.operand_layout or ("token-major" if w.name.startswith("dw_") and gran == "tile"
                                     else "k-contiguous")
    token_major = layout == "token-major" and not mx
    if token_major and gran != "tile":
        print("bench.py: the token-major layout is quantised with per-tile scales only", file=sys.stderr)
        sys.exit(2)
    mxv = mx and (args.mx_block != 32 or args.mx_scale != "e8m0")
    mx_kind = ("wide" if args.mx_scale != "e8m0" else "e8m0") if mxv else False
    if mx_kind == "e8m0" and mx_fp4_kernel(w, args.mx_block):
        mx_kind = "e8m0_fp4"    # blocks of 16 or 8 on the large MXFP4 kernel (FP4 instruction)
    if not mx and (args.mx_block != 32 or args.mx_scale != "e8m0"):
        print("bench.py: --mx-block / --mx-scale apply to the MXFP4 workload", file=sys.stderr)
        sys.exit(2)
    online = args.a_path == "online"
    if online and (mx or gran != "tile" or token_major):
        print("bench.py: --a-path online needs FP8 per-tile scales and K-contiguous operands",
              file=sys.stderr)
        sys.exit(2)
    a_src = np.ascontiguousarray(a_host.T) if token_major else a_host
    b_src = np.ascontiguousarray(b_host.T) if token_major else b_host

    def scale_shape(rows):
        return {"tile": ((rows + 127) // 128, w.K // 32), "row": (rows,), "tensor": (1,)}[gran]

    def new_set(a_dev, b_dev):
        """One set of step buffers: FP32 inputs, codes, scales and D."""
        st = {"a": a_dev, "b": b_dev}
        if mx:
            st["qa"] = torch.empty((w.M, w.K // 2), dtype=torch.uint8, device=dev)
            st["qb"] = torch.empty((w.N, w.K // 2), dtype=torch.uint8, device=dev)
            sdt = torch.uint8 if args.mx_scale == "e8m0" else torch.int16
            st["sa"] = torch.empty((w.M, w.K // args.mx_block), dtype=sdt, device=dev)
            st["sb"] = torch.empty((w.N, w.K // args.mx_block), dtype=sdt, device=dev)
        else:
            st["qa"] = torch.empty((w.M, w.K), dtype=torch.uint8, device=dev)
            st["qb"] = torch.empty((w.N, w.K), dtype=torch.uint8, device=dev)
            st["sa"] = torch.empty(scale_shape(w.M), dtype=torch.float32, device=dev)
            st["sb"] = torch.empty(scale_shape(w.N), dtype=torch.float32, device=dev)
        st["d"] = torch.empty((w.M, w.N), dtype=torch.float32 if w.out == "f32" else torch.bfloat16,
                              device=dev)
        return st

    a0 = torch.from_numpy(a_src).to(dev)
    b0 = torch.from_numpy(b_src).to(dev)
    sets = [new_set(a0, b0)]
    set_bytes = sum(t.numel() * t.element_size() for t in sets[0].values())
    nsets = max(2, -(-args.rotate_mib * 2**20 // set_bytes))
    for _ in range(nsets - 1):
        sets.append(new_set(a0.clone(), b0.clone()))
    log(f"input rotation: {nsets} sets of {set_bytes / 2**20:.0f} MiB")

    stream = torch.cuda.current_stream(dev)   # the library launches on this stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def gemm(st):
        if mxv:
            bs.scaled_gemm_mx(st["qa"], st["sa"], st["qb"], st["sb"], args.mx_block, args.mx_scale,
                              w.out, d=st["d"], K=w.K)
        elif online:
            bs.scaled_gemm_quantize_a(st["a"], st["qb"], st["sb"], w.a_fmt, w.b_fmt, "tile", w.out,
                                      d=st["d"])
        elif gran != "tile":
            bs.scaled_gemm_granular(st["qa"], st["sa"], st["qb"], st["sb"], w.a_fmt, w.b_fmt, gran,
                                    gran, w.out, d=st["d"], K=w.K)
        else:
            bs.scaled_gemm(st["qa"], st["sa"], st["qb"], st["sb"], w.a_fmt, w.b_fmt, w.out,
                           d=st["d"], K=w.K)

    def step(st, marks=None):
        a, b, qa, sa, qb, sb = st["a"], st["b"], st["qa"], st["sa"], st["qb"], st["sb"]
        if marks:
            marks[0].record(stream)
        if mxv:
            bs.mx_quantize(a, args.mx_block, args.mx_scale, qa, sa)
            if marks:
                marks[1].record(stream)
            bs.mx_quantize(b, args.mx_block, args.mx_scale, qb, sb)
        elif mx:
            bs.mxfp4_quantize(a, qa, sa)
            if marks:
                marks[1].record(stream)
            bs.mxfp4_quantize(b, qb, sb)
        elif online:
            if marks:
                marks[1].record(stream)
            bs.fp8_quantize(b, w.b_fmt, codes=qb, scales=sb)
        elif gran != "tile":
            bs.fp8_quantize_granular(a, w.a_fmt, gran, codes=qa, scales=sa)
            if marks:
                marks[1].record(stream)
            bs.fp8_quantize_granular(b, w.b_fmt, gran, codes=qb, scales=sb)
        elif token_major:
            bs.fp8_quantize_transposed(a, w.a_fmt, codes=qa, scales=sa)
            if marks:
                marks[1].record(stream)
            bs.fp8_quantize_transposed(b, w.b_fmt, codes=qb, scales=sb)
        else:       # A and B in one launch
            bs.fp8_quantize_pair(a, b, w.a_fmt, w.b_fmt, qa, sa, qb, sb)
            if marks:
                marks[1].record(stream)
        if marks:
            marks[2].record(stream)
        gemm(st)
        if marks:
            marks[3].record(stream)

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize(dev)

    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[(args.warmup + i) % nsets], ev[i])
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    last = sets[(args.warmup + args.steps - 1) % nsets]

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gemm_t = np.array([e[2].elapsed_time(e[3]) for e in ev])
    quant_t = np.array([e[0].elapsed_time(e[2]) for e in ev])
    gemm_ms = float(gemm_t.mean())
    quant_ms = float(quant_t.mean())
    pair = not mx and not online and gran == "tile" and not token_major
    if not pair:
        qa_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
        qb_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12

    gpu_info = {"compute_units": torch.cuda.get_device_properties(dev).multi_processor_count}

    in_type = "bf16" if mxv and mx_kind != "e8m0_fp4" else ("fp4" if mx else "fp8")
    gemm_tflops = w.flops / (gemm_ms * 1e-3) / 1e12
    kname = gemm_kernel_name(w, gran, online, mx_kind, args.mx_block)
    src = os.path.join(ROOT, "block_scaled_precision_fp8_amd", "csrc",
                       "gemm_mx.hip" if mxv and mx_kind != "e8m0_fp4" else "gemm_mxfp4.hip" if mx else
                       "gemm_fp8_big.hip" if kname == "gemm_fp8_big_kernel" else
                       ("gemm_fp8.hip" if gran == "tile" else "gemm_fp8_outer.hip"))
    profile_tag = (f"{w.name}_b{args.mx_block}_{args.mx_scale}" if mxv else f"{w.name}_online" if online
                   else (w.name if gran == "tile" else f"{w.name}_{gran}"))
    traffic, traffic_src = committed_traffic(profile_tag, src)
    gpu_info.update(committed_counters(profile_tag, src))

    # quantiser bytes: read 4 B, write 1 B (FP8) or 0.5 B (MXFP4) per element, plus scales
    def qbytes(rows):
        if mx:
            sbytes = 1 if args.mx_scale == "e8m0" else 2
            return rows * w.K * 4 + rows * w.K // 2 + rows * (w.K // args.mx_block) * sbytes
        nscales = {"tile": ((rows + 127) // 128) * (w.K // 32), "row": rows, "tensor": 1}[gran]
        return rows * w.K * 4 + rows * w.K + nscales * 4

    # The GEMM's bound: HBM when its arithmetic intensity (FLOP per algorithmic
    # byte: codes of A and B, their scales, D) is below the ridge point
    # peak FLOP/s / peak bytes/s, the matrix cores otherwise.
    gbytes = gemm_bytes(w, gran, args.mx_block, args.mx_scale, mx)
    if w.flops / gbytes < PEAK_TFLOPS[in_type] * 1e12 / (HBM_GBPS * 1e9):
        gemm_gbps = gbytes / (gemm_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": gemm_kernel_name(w, gran, online, mx_kind, args.mx_block),
                    "achieved": round(gemm_gbps, 1), "peak": HBM_GBPS, "unit": "GB/s",
                    "frac": round(gemm_gbps / HBM_GBPS, 4), "algorithmic_bytes": gbytes}
    else:
        roofline = {"bound": "mfma", "kernel": gemm_kernel_name(w, gran, online, mx_kind, args.mx_block),
                    "achieved": round(gemm_tflops, 1), "peak": PEAK_TFLOPS[in_type], "unit": "TFLOP/s",
                    "frac": round(gemm_tflops / PEAK_TFLOPS[in_type], 4),
                    "algorithmic_flops": w.flops}
    roofline.update({"traffic": traffic, "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": gbytes,
                     "traffic_source": os.path.relpath(traffic_src, ROOT) if traffic else traffic_src})

    quant_bytes = (0 if online else qbytes(w.M)) + qbytes(w.N)
    kernels = {
        "scaled_gemm_ms": round(gemm_ms, 4),
        "scaled_gemm_ms_median": round(float(np.median(gemm_t)), 4),
        "scaled_gemm_tflops": round(gemm_tflops, 1),
        "scaled_gemm_frac_of_peak": round(gemm_tflops / PEAK_TFLOPS[in_type], 4),
        "quantize_AB_ms": round(quant_ms, 4),
        "quantize_AB_ms_median": round(float(np.median(quant_t)), 4),
        "quantize_AB_gbps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
    }
    if not pair:
        kernels["quantize_A_ms"] = round(qa_ms, 4)
        kernels["quantize_B_ms"] = round(qb_ms, 4)
    kernels["quantize_AB_frac_of_hbm"] = round(kernels["quantize_AB_gbps"] / HBM_GBPS, 4)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4e2m1 (dequantised to bf16)" if mxv and mx_kind != "e8m0_fp4" else "fp4e2m1" if mx else ("fp8e4m3" if w.a_fmt == w.b_fmt == "e4m3" else "fp8e5m2xe4m3"),
        "data": "synthetic (seeded numpy, distributions of the workload table)",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "a_fmt": w.a_fmt,
                   "b_fmt": w.b_fmt, "out": w.out,
                   "operand_layout": "k-contiguous" if not token_major else "token-major",
                   "scale_granularity": (f"{args.mx_scale.upper()} per {args.mx_block}-element K block" if mx else
                                         {"tile": "FP32 per 128x32 tile",
                                          "row": "FP32 per row of A and per column of B",
                                          "tensor": "FP32 per tensor"}[gran]),
                   "a_path": "quantised inside the GEMM" if online else "separate quantiser",
                   "input_sets": nsets, "input_set_mib": round(set_bytes / 2**20, 1),
                   "step": ("mx_quantize(A)+mx_quantize(B)+scaled_gemm_mx" if mxv else
                            "mxfp4_quantize(A)+mxfp4_quantize(B)+scaled_gemm" if mx else
                            "fp8_quantize(B)+scaled_gemm_quantize_a(A)" if online else
                            "fp8_quantize_granular(A)+fp8_quantize_granular(B)+scaled_gemm_granular"
                            if gran != "tile" else
                            "fp8_quantize_transposed(G)+fp8_quantize_transposed(X)+scaled_gemm"
                            if token_major else "fp8_quantize_pair(A, B)+scaled_gemm")},
        "roofline": roofline,
        "kernels": kernels,
        "gpu": gpu_info,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a bounded sample ...")
        rows = int(args.cpu_sample_gflop * 1e9 / (2.0 * w.N * w.K)) // 128 * 128
        rows = max(128, min(w.M, rows))
        result["cpu_baseline"] = cpu_baseline(w, a_host, b_host, last, rows, gran, args.mx_block,
                                              args.mx_scale, token_major)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
