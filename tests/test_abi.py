"""The C-ABI library loads, exports every function include/bsfp8.h declares,
and rejects invalid arguments on the host before launching anything.  No GPU
is needed: every call here returns from the host-side checks."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsfp8.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
E4M3, E5M2, MXFP4 = 0, 1, 2
F32, BF16, F16 = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:bsfp8_status|const char\s*\*|int)\s+(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    import block_scaled_precision_fp8_amd as b
    return b.lib()


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("fp8_quantize", "fp8_quantize_pair", "fp8_quantize_transposed", "fp8_quantize_granular",
              "mxfp4_quantize",
              "scaled_gemm", "scaled_gemm_ex", "scaled_gemm_granular", "scaled_gemm_quantize_a",
              "mx_quantize", "scaled_gemm_mx",
              "bsfp8_status_string",
              "bsfp8_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), f"missing export {n}"


def test_status_strings(L):
    assert L.bsfp8_status_string(0) == b"BSFP8_OK"
    assert L.bsfp8_status_string(1) == b"BSFP8_ERR_INVALID_ARG"
    assert L.bsfp8_status_string(2) == b"BSFP8_ERR_UNSUPPORTED"
    assert L.bsfp8_status_string(3) == b"BSFP8_ERR_HIP"
    assert L.bsfp8_status_string(99) == b"BSFP8_ERR_UNKNOWN"
    assert L.bsfp8_version() >= 1


P = 0x1000  # a fake, 4 KiB-aligned "device pointer": never dereferenced by these calls


def test_fp8_quantize_argument_checks(L):
    q = L.fp8_quantize
    assert q(P, 128, 48, 48, 128, E4M3, P, P, None) == INVALID      # k % 32
    assert q(P, -1, 64, 64, 128, E4M3, P, P, None) == INVALID       # negative rows
    assert q(P, 128, 64, 32, 128, E4M3, P, P, None) == INVALID      # ld < k
    assert q(P, 128, 64, 66, 128, E4M3, P, P, None) == INVALID      # ld % 4
    assert q(P + 4, 128, 64, 64, 128, E4M3, P, P, None) == INVALID  # x not 16-byte aligned
    assert q(0, 128, 64, 64, 128, E4M3, P, P, None) == INVALID      # null x
    assert q(P, 128, 64, 64, 64, E4M3, P, P, None) == UNSUPPORTED   # tile_rows
    assert q(P, 128, 64, 64, 128, MXFP4, P, P, None) == UNSUPPORTED
    assert q(P, 128, 64, 64, 128, 7, P, P, None) == UNSUPPORTED
    assert q(0, 0, 64, 64, 128, E4M3, 0, 0, None) == OK             # empty: nothing to do
    assert q(0, 128, 0, 0, 128, E4M3, 0, 0, None) == OK


def test_fp8_quantize_pair_argument_checks(L):
    # (a, a_rows, a_ld, a_fmt, a_codes, a_scales, b, b_rows, b_ld, b_fmt, b_codes, b_scales, k, stream)
    q = L.fp8_quantize_pair
    ok = (P, 128, 64, E4M3, P, P, P, 256, 64, E5M2, P, P, 64, None)

    def call(**kw):
        names = ["a", "a_rows", "a_ld", "a_fmt", "a_codes", "a_scales", "b", "b_rows", "b_ld",
                 "b_fmt", "b_codes", "b_scales", "k", "stream"]
        args = dict(zip(names, ok))
        args.update(kw)
        return q(*[args[n] for n in names])

    assert call(k=48, a_ld=48, b_ld=48) == INVALID            # k % 32
    assert call(a_ld=32) == INVALID                            # a_ld < k
    assert call(b_ld=32) == INVALID                            # b_ld < k
    assert call(a_ld=66) == INVALID                            # a_ld % 4
    assert call(a=0) == INVALID                                # null a, non-empty side
    assert call(b_codes=0) == INVALID                          # null codes, non-empty side
    assert call(b_scales=0) == INVALID                         # null scales, non-empty side
    assert call(a=P + 4) == INVALID                            # a not 16-byte aligned
    assert call(a_codes=P + 2) == INVALID                      # codes not 4-byte aligned
    assert call(b_scales=P + 2) == INVALID                     # scales not 4-byte aligned
    assert call(a_rows=-1) == INVALID
    assert call(a_fmt=MXFP4) == UNSUPPORTED
    assert call(b_fmt=9) == UNSUPPORTED
    # a side with no rows ignores its pointers: nothing is launched for it, and
    # with both sides empty (or k = 0) nothing at all
    assert call(a_rows=0, b_rows=0, a=0, a_codes=0, a_scales=0, b=0, b_codes=0, b_scales=0) == OK
    assert call(k=0, a=0, b=0, a_codes=0, b_codes=0, a_scales=0, b_scales=0) == OK


def test_fp8_quantize_transposed_argument_checks(L):
    q = L.fp8_quantize_transposed     # (x, k, rows, ld, tile_rows, fmt, codes, scales, stream)
    assert q(P, 48, 128, 128, 128, E4M3, P, P, None) == INVALID     # k % 32
    assert q(P, 64, -1, 64, 128, E4M3, P, P, None) == INVALID       # negative rows
    assert q(P, 64, 128, 64, 128, E4M3, P, P, None) == INVALID      # ld < rows
    assert q(P, 64, 128, 130, 128, E4M3, P, P, None) == INVALID     # ld % 4
    assert q(P + 4, 64, 128, 128, 128, E4M3, P, P, None) == INVALID  # x alignment
    assert q(P, 64, 128, 128, 128, E4M3, P + 4, P, None) == INVALID  # codes alignment
    assert q(0, 64, 128, 128, 128, E4M3, P, P, None) == INVALID     # null x
    assert q(P, 64, 128, 128, 64, E4M3, P, P, None) == UNSUPPORTED  # tile_rows
    assert q(P, 64, 128, 128, 128, MXFP4, P, P, None) == UNSUPPORTED
    assert q(0, 64, 0, 0, 128, E4M3, 0, 0, None) == OK              # empty
    assert q(0, 0, 128, 128, 128, E4M3, 0, 0, None) == OK


def test_mxfp4_quantize_argument_checks(L):
    q = L.mxfp4_quantize
    assert q(P, 16, 48, 48, P, P, None) == INVALID
    assert q(P, 16, 64, 60, P, P, None) == INVALID
    assert q(P, -3, 64, 64, P, P, None) == INVALID
    assert q(P, 16, 64, 64, 0, P, None) == INVALID
    assert q(P + 8, 16, 64, 64, P, P, None) == INVALID
    assert q(0, 0, 64, 64, 0, 0, None) == OK


def test_scaled_gemm_argument_checks(L):
    g = L.scaled_gemm
    assert g(128, 128, 48, E4M3, P, P, E4M3, P, P, BF16, P, 128, None) == INVALID   # K % 32
    assert g(-1, 128, 64, E4M3, P, P, E4M3, P, P, BF16, P, 128, None) == INVALID
    assert g(128, 128, 64, E4M3, P, P, E4M3, P, P, BF16, P, 100, None) == INVALID  # ldd < N
    assert g(128, 128, 64, E4M3, 0, P, E4M3, P, P, BF16, P, 128, None) == INVALID  # null a
    assert g(128, 128, 64, E4M3, P, P, E4M3, P, 0, BF16, P, 128, None) == INVALID  # null scales
    assert g(128, 128, 64, E4M3, P + 8, P, E4M3, P, P, BF16, P, 128, None) == INVALID
    assert g(128, 128, 64, E4M3, P, P, E4M3, P, P, F32, P + 2, 128, None) == INVALID
    assert g(128, 128, 64, E4M3, P, P, MXFP4, P, P, BF16, P, 128, None) == UNSUPPORTED
    assert g(128, 128, 64, MXFP4, P, P, E5M2, P, P, BF16, P, 128, None) == UNSUPPORTED
    assert g(128, 128, 64, E4M3, P, P, E4M3, P, P, 5, P, 128, None) == UNSUPPORTED
    assert g(0, 128, 64, E4M3, 0, 0, E4M3, 0, 0, BF16, 0, 128, None) == OK      # empty
    assert g(128, 0, 64, E4M3, 0, 0, E4M3, 0, 0, F32, 0, 0, None) == OK
    # FP8: a 128-row band of an operand must fit 32-bit offsets (K < 2^24)
    assert g(128, 128, 1 << 24, E4M3, P, P, E4M3, P, P, BF16, P, 128, None) == UNSUPPORTED
    # MXFP4: a 32-row band must fit 32-bit byte offsets (K < 2^26)
    assert g(64, 128, 1 << 26, MXFP4, P, P, MXFP4, P, P, BF16, P, 128, None) == UNSUPPORTED
    assert g(64, 128, (1 << 26) + 32, MXFP4, P, P, MXFP4, P, P, BF16, P, 128, None) == UNSUPPORTED



def test_scaled_gemm_ex_argument_checks(L):
    g = L.scaled_gemm_ex   # (M, N, K, af, a, sa, bf, b, sb, alpha, c, ldc, beta, out, d, ldd, stream)
    ok = (128, 128, 64, E4M3, P, P, E4M3, P, P)
    assert g(*ok, 1.0, 0, 0, 1.0, BF16, P, 128, None) == INVALID          # beta != 0, null C
    assert g(*ok, 1.0, P, 100, 1.0, BF16, P, 128, None) == INVALID        # ldc < N
    assert g(*ok, 1.0, P + 1, 128, 1.0, F16, P, 128, None) == INVALID     # C alignment
    assert g(*ok, 1.0, P, 128, 0.5, 3, P, 128, None) == UNSUPPORTED       # bad output type
    assert g(128, 128, 48, E4M3, P, P, E4M3, P, P, 1.0, 0, 0, 0.0, F32, P, 128, None) == INVALID
    assert g(0, 128, 64, E4M3, 0, 0, E4M3, 0, 0, 1.0, 0, 0, 1.0, F16, 0, 128, None) == OK  # empty


def test_mfma_probe_loads_and_rejects_bad_arguments():
    """The matrix-core test probe (a test instrument) loads without a GPU and
    rejects bad arguments before any launch."""
    import mfma_probe
    P = mfma_probe.lib()
    assert [P.mfma_probe_k(i) for i in range(10)] == [16, 16, 16, 16, 16, 64, 64, 64, 64, 64]
    assert P.mfma_probe_k(10) == 0 and P.mfma_probe_k(-1) == 0
    buf = ctypes.create_string_buffer(256)
    p = ctypes.addressof(buf)
    assert P.mfma_probe_dot(10, 1, p, p, None, None, p, p, None) == 1     # unknown instruction
    assert P.mfma_probe_dot(0, -1, p, p, None, None, p, p, None) == 1     # negative count
    assert P.mfma_probe_dot(0, 1, None, p, None, None, p, p, None) == 1   # null operand
    assert P.mfma_probe_dot(5, 1, p, p, None, p, p, p, None) == 1         # scaled without scales
    assert P.mfma_probe_dot(0, 0, None, None, None, None, None, None, None) == 0   # nothing to do


TILE, ROW, TENSOR, MX32 = 0, 1, 2, 3


def test_fp8_quantize_granular_argument_checks(L):
    q = L.fp8_quantize_granular   # (x, rows, k, ld, granularity, fmt, codes, scales, stream)
    assert q(P, 4, 64, 64, 4, E4M3, P, P, None) == UNSUPPORTED         # unknown granularity
    assert q(P, 4, 64, 64, MX32, E4M3, P, P, None) == UNSUPPORTED      # MX blocks are MXFP4 only
    assert q(P, 4, 64, 64, ROW, MXFP4, P, P, None) == UNSUPPORTED      # not an FP8 format
    assert q(P, 4, 48, 64, ROW, E4M3, P, P, None) == INVALID           # k % 32
    assert q(P, 4, 64, 32, TENSOR, E4M3, P, P, None) == INVALID        # ld < k
    assert q(0, 4, 64, 64, ROW, E4M3, P, P, None) == INVALID           # null x
    assert q(P + 4, 4, 64, 64, TENSOR, E5M2, P, P, None) == INVALID    # x alignment
    assert q(P, 4, 64, 64, TENSOR, E5M2, P, P + 2, None) == INVALID    # scales alignment
    assert q(0, 0, 64, 64, ROW, E4M3, 0, 0, None) == OK                # empty
    assert q(0, 4, 0, 0, TENSOR, E4M3, 0, 0, None) == OK


def test_scaled_gemm_granular_argument_checks(L):
    g = L.scaled_gemm_granular
    # (M, N, K, af, a, sa, ag, bf, b, sb, bg, alpha, c, ldc, beta, out, d, ldd, stream)
    def call(ag, bg, af=E4M3, bf=E4M3, K=64, out=BF16):
        return g(128, 128, K, af, P, P, ag, bf, P, P, bg, 1.0, 0, 0, 0.0, out, P, 128, None)
    # per-row with per-tile scales is accepted: a bad K is what it rejects
    assert call(TILE, ROW, K=48) == INVALID
    assert call(ROW, TILE, K=48) == INVALID
    assert call(TILE, MX32) == UNSUPPORTED         # E8M0 blocks with FP8 operands
    assert call(MX32, MX32, af=MXFP4, bf=E4M3) == UNSUPPORTED
    assert call(TILE, TILE, af=MXFP4, bf=MXFP4) == UNSUPPORTED
    assert call(ROW, 7) == UNSUPPORTED
    assert call(ROW, ROW, K=1 << 23) == UNSUPPORTED   # K beyond the K-constant kernel's range
    assert call(ROW, TENSOR, K=48) == INVALID
    assert g(128, 128, 64, E4M3, P, 0, ROW, E4M3, P, P, ROW, 1.0, 0, 0, 0.0, BF16, P, 128, None) == INVALID
    assert g(128, 128, 64, E4M3, P, P + 2, ROW, E4M3, P, P, TENSOR, 1.0, 0, 0, 0.0, BF16, P, 128, None) == INVALID
    assert g(0, 128, 64, E4M3, 0, 0, ROW, E4M3, 0, 0, TENSOR, 1.0, 0, 0, 0.0, F32, 0, 128, None) == OK


def test_scaled_gemm_quantize_a_argument_checks(L):
    g = L.scaled_gemm_quantize_a
    # (M, N, K, x, ldx, af, bf, b, sb, bg, alpha, c, ldc, beta, out, d, ldd, a_codes, a_scales, stream)
    def call(M=128, N=128, K=64, x=P, ldx=64, af=E4M3, bf=E4M3, b=P, sb=P, bg=TILE, c=0, ldc=0,
             beta=0.0, out=BF16, d=P, ldd=128, ac=0, asc=0):
        return g(M, N, K, x, ldx, af, bf, b, sb, bg, 1.0, c, ldc, beta, out, d, ldd, ac, asc, None)
    assert call(af=MXFP4) == UNSUPPORTED
    assert call(bf=MXFP4) == UNSUPPORTED
    assert call(bg=ROW) == UNSUPPORTED               # per-row B: not built with online A
    assert call(bg=MX32) == UNSUPPORTED
    assert call(out=7) == UNSUPPORTED
    assert call(K=48, ldx=48) == INVALID              # K not a multiple of 32
    assert call(ldx=32) == INVALID                    # ldx < K
    assert call(ldx=66) == INVALID                    # ldx not a multiple of 4
    assert call(x=P + 4) == INVALID                   # x not 16-byte aligned
    assert call(x=0) == INVALID
    assert call(ldx=1 << 22, K=64) == UNSUPPORTED     # beyond the kernel's 32-bit band offsets
    assert call(ac=P) == INVALID                      # codes without scales
    assert call(asc=P) == INVALID
    assert call(ac=P + 2, asc=P) == INVALID
    assert call(b=0) == INVALID
    assert call(sb=P + 2) == INVALID
    assert call(d=0) == INVALID
    assert call(ldd=100) == INVALID
    assert call(beta=1.0) == INVALID                  # beta != 0 needs C
    assert call(M=-1) == INVALID
    assert call(M=0, x=0, d=0) == OK                  # nothing to do
    assert call(N=0, d=0) == OK                       # no output and no codes requested


def test_mx_quantize_argument_checks(L):
    q = L.mx_quantize
    # (x, rows, k, ld, block, sfmt, packed, scales, stream)
    assert q(P, 4, 64, 64, 4, 0, P, P, None) == UNSUPPORTED        # block size
    assert q(P, 4, 64, 64, 16, 3, P, P, None) == UNSUPPORTED       # scale format
    assert q(P, 4, 48, 48, 16, 0, P, P, None) == INVALID           # k % 32
    assert q(P, 4, 64, 32, 8, 1, P, P, None) == INVALID            # ld < k
    assert q(P + 4, 4, 64, 64, 8, 1, P, P, None) == INVALID        # x alignment
    assert q(P, 4, 64, 64, 8, 1, P, P + 1, None) == INVALID        # 16-bit scales alignment
    assert q(0, 4, 64, 64, 8, 2, P, P, None) == INVALID
    assert q(0, 0, 64, 64, 8, 2, 0, 0, None) == OK                 # nothing to do


def test_scaled_gemm_mx_argument_checks(L):
    g = L.scaled_gemm_mx
    # (M, N, K, block, sfmt, a, sa, b, sb, alpha, c, ldc, beta, out, d, ldd, stream)
    def call(block=16, sfmt=0, K=64, a=P, sa=P, b=P, sb=P, out=BF16, d=P, ldd=128, beta=0.0, c=0):
        return g(128, 128, K, block, sfmt, a, sa, b, sb, 1.0, c, 0, beta, out, d, ldd, None)
    assert call(block=64) == UNSUPPORTED
    assert call(sfmt=5) == UNSUPPORTED
    assert call(out=9) == UNSUPPORTED
    assert call(K=48) == INVALID
    assert call(a=P + 8) == INVALID
    assert call(sfmt=1, sa=P + 1) == INVALID
    assert call(sfmt=0, sb=P + 4) == INVALID              # scales read 8 bytes at a time
    assert call(d=0) == INVALID
    assert call(beta=1.0) == INVALID
    assert call(block=32, sfmt=0, K=48) == INVALID        # the MXFP4 path checks too
