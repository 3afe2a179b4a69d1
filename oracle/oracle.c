/*
 * oracle.c -- CPU oracle for block-scaled FP8 / MXFP4 quantisation and GEMM.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load this library.
 * It shares no code, table or constant generator with the HIP kernels.
 *
 * Plain and slow on purpose: every number format is an explicit decode table
 * built from its bit fields, every encode is a search in that table with an
 * exact midpoint comparison, and the GEMM is an fp64 dot product of the
 * dequantised operands.  Pages cited (by title and section):
 *   [CDNA4-FP8]  "Why grind FP8 GEMM on CDNA4" article (dpshk.com)
 *   [RUBIN-FP4]  "Rubin FP4 GEMM deep dive: from Blackwell to the next GPU"
 *   [HOPPER-MMA] "FP8 MMA internals on Hopper" (Simon Veitner)
 *   [AMD-MFMA]   "Exact models of AMD matrix cores" (Khattak, Mikaitis, Graziani)
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes of the repository):
 *   - E4M3 is the OCP "FN" variant: max 448, no infinity, S.1111.111 is NaN.
 *     E5M2 is the OCP variant: max 57344, exponent 31 is inf/NaN.
 *   - Scale denominator F is the element format's maximum: 448 (E4M3, stated
 *     in [CDNA4-FP8] section 3.3) and 57344 (E5M2, by analogy).
 *   - An all-zero FP8 tile takes scale 1.0; an all-zero MX block takes E8M0
 *     code 127 (scale 1.0).
 *   - Rounding is to nearest, ties to the code with an even last bit; finite
 *     values beyond the format maximum saturate to +-max; the sign of zero is
 *     kept.  Inputs must be finite.
 *   - The MX block exponent is the smallest integer e with 6 * 2^e >= amax
 *     ("nearest power of two" in [RUBIN-FP4] section 4.2 read so that the
 *     block maximum never saturates), clamped to the E8M0 range [-127, 127].
 *   - Scale products are applied per 32-wide K block (the K blocking of
 *     [RUBIN-FP4] section 2.2 and the per-tile scales of [CDNA4-FP8] section
 *     3.3), so D is the plain product of the dequantised operands.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Decode tables (format definitions)                                        */
/* ------------------------------------------------------------------------ */

/* Generic "sign | exponent | mantissa" decode with IEEE-style subnormals:
 *   e == 0 : (m / 2^mbits) * 2^(1 - bias)
 *   e >  0 : (1 + m / 2^mbits) * 2^(e - bias)
 * Special encodings (NaN / inf) are patched in by the callers. */
static double decode_fields(unsigned code, int ebits, int mbits, int bias) {
    unsigned m = code & ((1u << mbits) - 1u);
    unsigned e = (code >> mbits) & ((1u << ebits) - 1u);
    unsigned s = (code >> (mbits + ebits)) & 1u;
    double frac = (double)m / (double)(1u << mbits);
    double v;
    if (e == 0)
        v = ldexp(frac, 1 - bias);
    else
        v = ldexp(1.0 + frac, (int)e - bias);
    return s ? -v : v;
}

static double tab_e4m3[256], tab_e5m2[256], tab_e2m1[16], tab_e8m0[256];
static int tables_ready = 0;

static void build_tables(void) {
    if (tables_ready) return;
    for (unsigned c = 0; c < 256; ++c) {
        /* E4M3 (OCP FN): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
         * exponent 15 with mantissa 7 is NaN, everything else is finite. */
        tab_e4m3[c] = decode_fields(c, 4, 3, 7);
        if ((c & 0x7Fu) == 0x7Fu) tab_e4m3[c] = NAN;
        /* E5M2 (OCP): 1 sign, 5 exponent (bias 15), 2 mantissa bits;
         * exponent 31 is infinity (mantissa 0) or NaN. */
        tab_e5m2[c] = decode_fields(c, 5, 2, 15);
        if (((c >> 2) & 31u) == 31u)
            tab_e5m2[c] = (c & 3u) ? NAN : ((c & 0x80u) ? -INFINITY : INFINITY);
        /* E8M0: 8 exponent bits, no sign, no mantissa: 2^(c - 127); 255 is NaN. */
        tab_e8m0[c] = (c == 255u) ? NAN : ldexp(1.0, (int)c - 127);
    }
    /* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; all 16 codes finite. */
    for (unsigned c = 0; c < 16; ++c) tab_e2m1[c] = decode_fields(c, 2, 1, 1);
    tables_ready = 1;
}

/* Largest finite non-negative code of each element format; the finite
 * non-negative values are exactly codes 0..maxcode, in increasing order. */
static int max_code(int fmt) {
    switch (fmt) {
    case ORC_E4M3: return 0x7E;  /* 448   */
    case ORC_E5M2: return 0x7B;  /* 57344 */
    case ORC_E2M1: return 0x7;   /* 6     */
    default: return -1;
    }
}

static const double* table_of(int fmt) {
    build_tables();
    switch (fmt) {
    case ORC_E4M3: return tab_e4m3;
    case ORC_E5M2: return tab_e5m2;
    case ORC_E2M1: return tab_e2m1;
    case ORC_E8M0: return tab_e8m0;
    default: return NULL;
    }
}

static unsigned sign_bit(int fmt) { return fmt == ORC_E2M1 ? 0x8u : 0x80u; }

int oracle_decode_table(int fmt, double* out) {
    const double* t = table_of(fmt);
    if (!t || !out) return -1;
    int n = (fmt == ORC_E2M1) ? 16 : 256;
    memcpy(out, t, sizeof(double) * (size_t)n);
    return n;
}

double oracle_decode(int fmt, unsigned code) {
    const double* t = table_of(fmt);
    return t[code & ((fmt == ORC_E2M1) ? 0xFu : 0xFFu)];
}

/* ------------------------------------------------------------------------ */
/* Encode: saturating round-to-nearest-even by table search                 */
/* ------------------------------------------------------------------------ */

unsigned oracle_encode(int fmt, double v) {
    const double* t = table_of(fmt);
    int top = max_code(fmt);
    double a = fabs(v);
    unsigned sign = signbit(v) ? sign_bit(fmt) : 0u;
    int code;
    if (a >= t[top]) {
        code = top;                          /* saturate */
    } else {
        /* find lo with t[lo] <= a < t[lo + 1] */
        int lo = 0, hi = top;                /* invariant: t[lo] <= a < t[hi] */
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (t[mid] <= a) lo = mid; else hi = mid;
        }
        double midpoint = 0.5 * (t[lo] + t[hi]);   /* exact in fp64 */
        if (a < midpoint)      code = lo;
        else if (a > midpoint) code = hi;
        else                   code = (lo % 2 == 0) ? lo : hi;  /* tie: even code */
    }
    return (unsigned)code | sign;
}

void oracle_encode_array(int fmt, const double* v, int64_t n, uint8_t* codes) {
    for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)oracle_encode(fmt, v[i]);
}

/* ------------------------------------------------------------------------ */
/* FP8 quantisation with per-tile, per-row or per-tensor scales             */
/* ([CDNA4-FP8] sections 3.3 and 4.2; the granularities of section 3.3)     */
/* ------------------------------------------------------------------------ */

static float fp8_denominator(int fmt) { return fmt == ORC_E4M3 ? 448.0f : 57344.0f; }

/* x: rows x k FP32, row stride ld.  One scale per group of group_rows x
 * group_k elements along (row, k); edge groups may be partial.  codes: rows x
 * k (stride k).  scales: FP32 [ceil(rows / group_rows)][ceil(k / group_k)],
 * K-group index fastest.
 * Per group: amax = max |x|; s = fl32(amax / F) (1.0 if that is zero);
 * code = encode(fl32(x / s)).
 * Per tile: group 128 x 32.  Per row: 1 x k.  Per tensor: rows x k. */
int oracle_fp8_quantize_groups(const float* x, int64_t rows, int64_t k, int64_t ld,
                               int64_t group_rows, int64_t group_k, int fmt, uint8_t* codes,
                               float* scales) {
    if (fmt != ORC_E4M3 && fmt != ORC_E5M2) return -1;
    if (rows < 0 || k < 0 || ld < k || group_rows < 1 || group_k < 1) return -1;
    build_tables();
    const float F = fp8_denominator(fmt);
    int64_t tr = (rows + group_rows - 1) / group_rows;
    int64_t tk = (k + group_k - 1) / group_k;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t ti = 0; ti < tr; ++ti) {
        for (int64_t tj = 0; tj < tk; ++tj) {
            int64_t r0 = ti * group_rows, r1 = r0 + group_rows < rows ? r0 + group_rows : rows;
            int64_t c0 = tj * group_k, c1 = c0 + group_k < k ? c0 + group_k : k;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float a = fabsf(x[r * ld + c]);
                    if (a > amax) amax = a;
                }
            float s = amax / F;                 /* IEEE binary32 division */
            if (s == 0.0f) s = 1.0f;
            scales[ti * tk + tj] = s;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float q = x[r * ld + c] / s;  /* IEEE binary32 division */
                    codes[r * k + c] = (uint8_t)oracle_encode(fmt, (double)q);
                }
        }
    }
    return 0;
}

/* Per-tile scales: tiles of tile_rows x 32. */
int oracle_fp8_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                        int64_t tile_rows, int fmt, uint8_t* codes, float* scales) {
    return oracle_fp8_quantize_groups(x, rows, k, ld, tile_rows, 32, fmt, codes, scales);
}

/* ------------------------------------------------------------------------ */
/* MXFP4 block quantisation  ([RUBIN-FP4] sections 2.1, 2.2, 3.1, 4.2)      */
/* ------------------------------------------------------------------------ */

/* Smallest integer e with 6 * 2^e >= amax (amax > 0), clamped to [-127, 127]. */
int oracle_mx_exponent(double amax) {
    if (!(amax > 0.0)) return 0;
    int e = ilogb(amax) - 3;                 /* start below the answer */
    while (6.0 * ldexp(1.0, e) < amax) ++e;  /* exact comparisons in fp64 */
    while (6.0 * ldexp(1.0, e - 1) >= amax) --e;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* x: rows x k FP32 (stride ld), k even.  Blocks are 32 consecutive K elements
 * of one row (the last block of a row may be partial).  packed: rows x (k/2)
 * bytes, element k in the low nibble of byte k/2 when k is even, in the high
 * nibble when k is odd.  scales: E8M0 bytes [rows][ceil(k / 32)]. */
int oracle_mxfp4_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                          uint8_t* packed, uint8_t* scales) {
    if (rows < 0 || k < 0 || ld < k || (k % 2) != 0) return -1;
    build_tables();
    int64_t nb = (k + 31) / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            int64_t c0 = b * 32, c1 = c0 + 32 < k ? c0 + 32 : k;
            double amax = 0.0;
            for (int64_t c = c0; c < c1; ++c) {
                double a = fabs((double)x[r * ld + c]);
                if (a > amax) amax = a;
            }
            int e = (amax == 0.0) ? 0 : oracle_mx_exponent(amax);
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (int64_t c = c0; c < c1; ++c) {
                double y = ldexp((double)x[r * ld + c], -e);   /* exact */
                unsigned q = oracle_encode(ORC_E2M1, y);
                uint8_t* byte = &packed[r * (k / 2) + c / 2];
                if ((c % 2) == 0) *byte = (uint8_t)((*byte & 0xF0u) | q);
                else              *byte = (uint8_t)((*byte & 0x0Fu) | (q << 4));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* MX variants: blocks of 32, 16 or 8 elements and FP16 / BF16 block scales */
/* ([RUBIN-FP4] section 5.3 offers blocks of 16 and 8 where 32 is too       */
/* coarse; section 3.2 offers FP16 or BF16 scales where a power of two is)  */
/* ------------------------------------------------------------------------ */

/* Nearest value to v >= 0 of a binary format with p significand bits (the
 * hidden one included) whose smallest normal value is 2^emin, with
 * subnormals below it; ties go to the even last significand bit; results
 * beyond vmax become vmax (the scale saturates like the elements do). */
static double round_to_format(double v, int p, int emin, double vmax) {
    if (v == 0.0) return 0.0;
    int e;
    (void)frexp(v, &e);                            /* v in [2^(e-1), 2^e) */
    int lsb_exp = (e - 1 > emin ? e - 1 : emin) - (p - 1);
    double ulp = ldexp(1.0, lsb_exp);
    double n = floor(v / ulp);                     /* exact: scaling by a power of two */
    double rem = v - n * ulp;                      /* exact */
    if (2.0 * rem > ulp || (2.0 * rem == ulp && fmod(n, 2.0) != 0.0)) n += 1.0;
    double r = n * ulp;
    return r > vmax ? vmax : r;
}

/* Bits of a value produced by round_to_format (exactly representable). */
static unsigned format_bits(double v, int p, int emin, int bias) {
    if (v == 0.0) return 0u;
    int e;
    double f = frexp(v, &e);                       /* v = f 2^e, f in [1/2, 1) */
    if (e - 1 < emin)                              /* subnormal: v = m 2^(emin - p + 1) */
        return (unsigned)ldexp(v, p - 1 - emin);
    unsigned field = (unsigned)(e - 1 + bias);
    unsigned mant = (unsigned)ldexp(2.0 * f - 1.0, p - 1);
    return (field << (p - 1)) | mant;
}

/* Scale formats: p, emin, bias, largest finite value. */
static void scale_format(int sfmt, int* p, int* emin, int* bias, double* vmax) {
    if (sfmt == ORC_SCALE_F16) {                   /* IEEE binary16 */
        *p = 11; *emin = -14; *bias = 15; *vmax = 65504.0;
    } else {                                       /* bfloat16: binary32 range, 8-bit significand */
        *p = 8; *emin = -126; *bias = 127; *vmax = ldexp(255.0, 120);
    }
}

/* x: rows x k FP32 (stride ld), k a multiple of `block` (32, 16 or 8).
 * packed: rows x k/2 bytes, low nibble first.
 * scales: [rows][k / block]; E8M0 bytes (sfmt ORC_SCALE_E8M0) or the 16-bit
 * patterns of FP16 / BF16 values (ORC_SCALE_F16, ORC_SCALE_BF16).
 * Per block: amax = max |x|;
 *   E8M0: e = smallest integer with 6 2^e >= amax (0 when amax is 0),
 *         clamped to [-127, 127]; code = encode_E2M1(x 2^-e) (exact scaling);
 *   FP16 / BF16: s = the scale-format value nearest to amax / 6 (saturating;
 *         s = 1 when that is zero); code = encode_E2M1(fl32(x / s)), the
 *         FP8 rule of [CDNA4-FP8] section 3.3 with F = 6. */
int oracle_mx_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int64_t block,
                       int sfmt, uint8_t* packed, void* scales) {
    if (rows < 0 || k < 0 || ld < k) return -1;
    if (block != 32 && block != 16 && block != 8) return -1;
    if ((k % block) != 0) return -1;
    if (sfmt != ORC_SCALE_E8M0 && sfmt != ORC_SCALE_F16 && sfmt != ORC_SCALE_BF16) return -1;
    build_tables();
    int64_t nb = k / block;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            int64_t c0 = b * block, c1 = c0 + block;
            double amax = 0.0;
            for (int64_t c = c0; c < c1; ++c) {
                double a = fabs((double)x[r * ld + c]);
                if (a > amax) amax = a;
            }
            unsigned q[32];
            if (sfmt == ORC_SCALE_E8M0) {
                int e = (amax == 0.0) ? 0 : oracle_mx_exponent(amax);
                ((uint8_t*)scales)[r * nb + b] = (uint8_t)(e + 127);
                for (int64_t c = c0; c < c1; ++c)
                    q[c - c0] = oracle_encode(ORC_E2M1, ldexp((double)x[r * ld + c], -e));
            } else {
                int p, emin, bias;
                double vmax;
                scale_format(sfmt, &p, &emin, &bias, &vmax);
                double sd = round_to_format(amax / 6.0, p, emin, vmax);
                if (sd == 0.0) sd = 1.0;
                ((uint16_t*)scales)[r * nb + b] = (uint16_t)format_bits(sd, p, emin, bias);
                const float sf = (float)sd;        /* exact: every FP16 / BF16 value is an FP32 value */
                for (int64_t c = c0; c < c1; ++c) {
                    float y = x[r * ld + c] / sf;  /* IEEE binary32 division */
                    q[c - c0] = oracle_encode(ORC_E2M1, (double)y);
                }
            }
            for (int64_t c = c0; c < c1; ++c) {
                uint8_t* byte = &packed[r * (k / 2) + c / 2];
                unsigned code = q[c - c0];
                if ((c % 2) == 0) *byte = (uint8_t)((*byte & 0xF0u) | code);
                else              *byte = (uint8_t)((*byte & 0x0Fu) | (code << 4));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantisation and GEMM  ([AMD-MFMA] section 2, eq. (1) with c = 0)      */
/* ------------------------------------------------------------------------ */

/* One row of an operand, dequantised to fp64: out[c] = decode(code) * scale.
 * FP8 operands: codes rows x k, FP32 scales [ceil(rows/tile_rows)][ceil(k/32)].
 * MXFP4 operands: packed rows x k/2, E8M0 scales [rows][ceil(k/32)]. */
static void dequant_row(int fmt, const uint8_t* q, const void* scales, int64_t tile_rows,
                        int64_t k, int64_t row, double* out) {
    int64_t nb = (k + 31) / 32;
    if (fmt == ORC_E4M3 || fmt == ORC_E5M2) {
        const double* t = table_of(fmt);
        const float* s = (const float*)scales + (row / tile_rows) * nb;
        for (int64_t c = 0; c < k; ++c)
            out[c] = t[q[row * k + c]] * (double)s[c / 32];
    } else {
        const uint8_t* s = (const uint8_t*)scales + row * nb;
        for (int64_t c = 0; c < k; ++c) {
            uint8_t byte = q[row * (k / 2) + c / 2];
            unsigned nib = (c % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
            out[c] = tab_e2m1[nib] * tab_e8m0[s[c / 32]];
        }
    }
}

static int fmt_ok(int fa, int fb) {
    int a8 = (fa == ORC_E4M3 || fa == ORC_E5M2), b8 = (fb == ORC_E4M3 || fb == ORC_E5M2);
    return (a8 && b8) || (fa == ORC_MXFP4 && fb == ORC_MXFP4);
}

/* Rows [row0, row1) of D = deq(A) * deq(B)^T where B is stored N x K (a
 * K x N column-major matrix); FP8 scale tiles are tile_rows x 32 for both.
 * d, s: (row1-row0) x N, row-major;
 * d = sum_k a*b, s = sum_k |a*b|, both in fp64. */
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K, int64_t tile_rows,
                     int a_fmt, const uint8_t* a, const void* a_scales,
                     int b_fmt, const uint8_t* b, const void* b_scales,
                     int64_t row0, int64_t row1, double* d, double* s) {
    if (!fmt_ok(a_fmt, b_fmt) || row0 < 0 || row1 > M || row0 > row1 || N < 0 || K < 0 ||
        tile_rows < 1) return -1;
    build_tables();
    double* bd = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!bd) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j) dequant_row(b_fmt, b, b_scales, tile_rows, K, j, bd + j * K);
    int err = 0;
#pragma omp parallel
    {
        double* ar = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!ar) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = row0; i < row1; ++i) {
                dequant_row(a_fmt, a, a_scales, tile_rows, K, i, ar);
                for (int64_t j = 0; j < N; ++j) {
                    const double* bj = bd + j * K;
                    double acc = 0.0, mag = 0.0;
                    for (int64_t c = 0; c < K; ++c) {
                        double p = ar[c] * bj[c];
                        acc += p;
                        mag += fabs(p);
                    }
                    d[(i - row0) * N + j] = acc;
                    s[(i - row0) * N + j] = mag;
                }
            }
            free(ar);
        }
    }
    free(bd);
    return err;
}

/* The same sums at npts chosen output positions (ii[p], jj[p]). */
int oracle_gemm_points(int64_t M, int64_t N, int64_t K, int64_t tile_rows,
                       int a_fmt, const uint8_t* a, const void* a_scales,
                       int b_fmt, const uint8_t* b, const void* b_scales,
                       int64_t npts, const int64_t* ii, const int64_t* jj,
                       double* d, double* s) {
    if (!fmt_ok(a_fmt, b_fmt) || N < 0 || K < 0 || tile_rows < 1) return -1;
    for (int64_t p = 0; p < npts; ++p)
        if (ii[p] < 0 || ii[p] >= M || jj[p] < 0 || jj[p] >= N) return -1;
    build_tables();
    int err = 0;
#pragma omp parallel
    {
        double* ar = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* br = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!ar || !br) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t p = 0; p < npts; ++p) {
                dequant_row(a_fmt, a, a_scales, tile_rows, K, ii[p], ar);
                dequant_row(b_fmt, b, b_scales, tile_rows, K, jj[p], br);
                double acc = 0.0, mag = 0.0;
                for (int64_t c = 0; c < K; ++c) {
                    double q = ar[c] * br[c];
                    acc += q;
                    mag += fabs(q);
                }
                d[p] = acc;
                s[p] = mag;
            }
        }
        free(ar);
        free(br);
    }
    return err;
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
