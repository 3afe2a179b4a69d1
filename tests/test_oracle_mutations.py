"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c (a wrong constant,
index, sign, rounding rule or operand), builds it, and runs the oracle pin
tests against that build in a subprocess: at least one pin must fail.  A
control case checks that an unmodified copy passes.  CPU only; nothing here
touches the HIP library."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_formats.py", "tests/test_oracle_quantize.py", "tests/test_oracle_gemm.py",
        "tests/test_oracle_granular.py", "tests/test_oracle_mx_variants.py"]

# (name, text in oracle.c, replacement): each a mistake someone could make.
# Left out as equivalent (no result can differ): reading both GEMM operands'
# nibbles in swapped order (the same K pairs swap in A and B, so every product
# and every sum is unchanged; the packing itself is pinned on the quantiser),
# and a mistake in either one of the two searching loops of the MX exponent
# (each loop alone finds the smallest covering power from its side).
MUTATIONS = [
    ("e4m3-bias", "decode_fields(c, 4, 3, 7)", "decode_fields(c, 4, 3, 8)"),
    ("e5m2-bias", "decode_fields(c, 5, 2, 15)", "decode_fields(c, 5, 2, 14)"),
    ("e2m1-bias", "decode_fields(c, 2, 1, 1)", "decode_fields(c, 2, 1, 2)"),
    ("subnormal-exponent", "v = ldexp(frac, 1 - bias);", "v = ldexp(frac, -bias);"),
    ("tie-rounds-up", "else                   code = (lo % 2 == 0) ? lo : hi;",
     "else                   code = hi;"),
    ("truncating-encode", "if (a < midpoint)      code = lo;", "if (a < t[hi])         code = lo;"),
    ("saturate-one-below", "code = top;                          /* saturate */",
     "code = top - 1;                      /* saturate */"),
    ("negative-zero-sign", "unsigned sign = signbit(v) ? sign_bit(fmt) : 0u;",
     "unsigned sign = (v < 0) ? sign_bit(fmt) : 0u;"),
    ("fnuz-e4m3-max", "return fmt == ORC_E4M3 ? 448.0f : 57344.0f;",
     "return fmt == ORC_E4M3 ? 240.0f : 57344.0f;"),
    ("zero-tile-scale", "            if (s == 0.0f) s = 1.0f;\n            scales[ti * tk + tj] = s;",
     "            scales[ti * tk + tj] = s;"),
    ("reciprocal-multiply", "float q = x[r * ld + c] / s;  /* IEEE binary32 division */",
     "float q = x[r * ld + c] * (1.0f / s);"),
    ("tile-columns-64", "oracle_fp8_quantize_groups(x, rows, k, ld, tile_rows, 32, fmt, codes, scales)",
     "oracle_fp8_quantize_groups(x, rows, k, ld, tile_rows, 64, fmt, codes, scales)"),
    ("group-column-end", "int64_t c0 = tj * group_k, c1 = c0 + group_k < k ? c0 + group_k : k;",
     "int64_t c0 = tj * group_k, c1 = c0 + group_k < k ? c0 + group_k : k - 1;"),
    ("group-row-start", "int64_t r0 = ti * group_rows, r1", "int64_t r0 = ti * group_rows + (ti > 0), r1"),
    ("mx-exponent-clamp", "if (e < -127) e = -127;", "if (e < -126) e = -126;"),
    ("mx-exponent-off-by-one", "    if (e > 127) e = 127;\n    return e;",
     "    if (e > 127) e = 127;\n    return e + 1;"),
    ("mx-scale-bias", "scales[r * nb + b] = (uint8_t)(e + 127);", "scales[r * nb + b] = (uint8_t)(e + 128);"),
    ("nibble-order", "if ((c % 2) == 0) *byte = (uint8_t)((*byte & 0xF0u) | q);\n                else              *byte = (uint8_t)((*byte & 0x0Fu) | (q << 4));",
     "if ((c % 2) == 1) *byte = (uint8_t)((*byte & 0xF0u) | q);\n                else              *byte = (uint8_t)((*byte & 0x0Fu) | (q << 4));"),
    ("dequant-drops-scale", "out[c] = t[q[row * k + c]] * (double)s[c / 32];", "out[c] = t[q[row * k + c]];"),
    ("scale-block-index", "out[c] = t[q[row * k + c]] * (double)s[c / 32];",
     "out[c] = t[q[row * k + c]] * (double)s[c / 64];"),
    ("per-row-scales", "const float* s = (const float*)scales + (row / tile_rows) * nb;",
     "const float* s = (const float*)scales + (row % tile_rows) * nb;"),
    ("mx-scale-ignored", "out[c] = tab_e2m1[nib] * tab_e8m0[s[c / 32]];", "out[c] = tab_e2m1[nib];"),
    ("b-decoded-as-a", "for (int64_t j = 0; j < N; ++j) dequant_row(b_fmt, b, b_scales, tile_rows, K, j, bd + j * K);",
     "for (int64_t j = 0; j < N; ++j) dequant_row(a_fmt, b, b_scales, tile_rows, K, j, bd + j * K);"),
    ("product-sign", "                        double p = ar[c] * bj[c];\n                        acc += p;",
     "                        double p = ar[c] * bj[c];\n                        acc += (c % 2) ? -p : p;"),
    ("magnitude-signed", "                        mag += fabs(p);", "                        mag += p;"),
    ("mx-variant-half-block", "int64_t c0 = b * block, c1 = c0 + block;",
     "int64_t c0 = b * block, c1 = c0 + block / 2;"),
    ("f16-scale-precision", "*p = 11; *emin = -14; *bias = 15; *vmax = 65504.0;",
     "*p = 10; *emin = -14; *bias = 15; *vmax = 65504.0;"),
    ("bf16-scale-precision", "*p = 8; *emin = -126; *bias = 127;", "*p = 9; *emin = -126; *bias = 127;"),
    ("scale-ties-up", "(2.0 * rem == ulp && fmod(n, 2.0) != 0.0)", "(2.0 * rem == ulp)"),
    ("scale-truncated", "if (2.0 * rem > ulp || (2.0 * rem == ulp", "if (2.0 * rem > 2.0 * ulp || (2.0 * rem == ulp"),
    ("scale-unsaturated", "return r > vmax ? vmax : r;", "return r;"),
    ("scale-zero-kept", "if (sd == 0.0) sd = 1.0;", "if (sd == 0.0) sd = 0.5;"),
    ("subnormal-scale-bits", "return (unsigned)ldexp(v, p - 1 - emin);", "return (unsigned)ldexp(v, p - emin);"),
    ("scale-denominator", "round_to_format(amax / 6.0, p, emin, vmax)", "round_to_format(amax / 4.0, p, emin, vmax)"),
    ("wide-scale-reciprocal", "float y = x[r * ld + c] / sf;  /* IEEE binary32 division */",
     "float y = x[r * ld + c] * (1.0f / sf);"),
    ("dropped-last-term", "                    for (int64_t c = 0; c < K; ++c) {\n                        double p = ar[c] * bj[c];",
     "                    for (int64_t c = 0; c + 1 < K; ++c) {\n                        double p = ar[c] * bj[c];"),
]


def build(src_text, out_dir):
    src = os.path.join(out_dir, "oracle_mut.c")
    lib = os.path.join(out_dir, "liboracle_mut.so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-I", os.path.dirname(ORACLE_C), "-o", lib, src, "-lm"],
                   check=True, capture_output=True)
    return lib


def run_pins(lib):
    env = dict(os.environ, ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes_the_pins(tmp_path):
    r = run_pins(build(open(ORACLE_C).read(), str(tmp_path)))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(ORACLE_C).read()
    assert text.count(old) == 1, f"{name}: the patched text must occur exactly once"
    r = run_pins(build(text.replace(old, new), str(tmp_path)))
    assert r.returncode != 0, f"planted mistake '{name}' survived every pin"
