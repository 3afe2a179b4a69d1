/*
 * bsfp8.h -- block-scaled FP8 / MXFP4 quantisation and GEMM on AMD MI355X (gfx950).
 *
 * A small C ABI over hand-written HIP kernels.  Every pointer argument is a
 * DEVICE pointer owned by the caller; the library never allocates, frees or
 * synchronises.  Every call is asynchronous on `stream` (0 = the null stream).
 * All argument checks run on the host before anything is launched: a call
 * that returns a status other than BSFP8_OK has launched nothing.  After a
 * launch the HIP launch error, if any, is returned as BSFP8_ERR_HIP.  No
 * global state: calls are thread-safe; calls that write the same output
 * buffer concurrently race.
 *
 * Pages cited (by title and section):
 *   [CDNA4-FP8] "Why grind FP8 GEMM on CDNA4" (dpshk.com article)
 *   [RUBIN-FP4] "Rubin FP4 GEMM deep dive: from Blackwell to the next GPU"
 *   [HOPPER-MMA] "FP8 MMA internals on Hopper"
 *
 * Layout conventions ([CDNA4-FP8] section 3.1, [RUBIN-FP4] section 3.1):
 * A is M x K row-major (K contiguous); B is K x N column-major, i.e. stored as
 * N rows of K contiguous elements; D is M x N row-major with leading
 * dimension ldd (elements).  A "K block" is 32 consecutive K indices.
 */
#ifndef BSFP8_H
#define BSFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same typedef as the HIP runtime's; repeating it is harmless. */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    BSFP8_OK = 0,
    BSFP8_ERR_INVALID_ARG = 1,  /* null pointer, negative size, K not a multiple of 32, ld < k, ... */
    BSFP8_ERR_UNSUPPORTED = 2,  /* undefined enum value or format mix, tile_rows != 128 */
    BSFP8_ERR_HIP = 3           /* the HIP runtime reported a launch error */
} bsfp8_status;

typedef enum {
    BSFP8_E4M3 = 0,   /* OCP E4M3 ("FN"): max 448, no infinity */
    BSFP8_E5M2 = 1,   /* OCP E5M2: max 57344 */
    BSFP8_MXFP4 = 2   /* E2M1 elements, two per byte, E8M0 scale per 32-element K block */
} bsfp8_format;

typedef enum {
    BSFP8_OUT_F32 = 0,
    BSFP8_OUT_BF16 = 1,
    BSFP8_OUT_F16 = 2   /* IEEE binary16, round to nearest even, overflow to +-inf */
} bsfp8_out;

/*
 * fp8_quantize -- per-tile FP8 quantisation ([CDNA4-FP8] sections 3.3 and 4.2).
 *
 * x:      rows x k FP32, row-major, leading dimension ld (elements).
 *         16-byte aligned, ld a multiple of 4, ld >= k.
 * rows:   >= 0, any value; the last tile may have fewer than tile_rows rows.
 * k:      >= 0, a multiple of 32.
 * tile_rows: rows per scale tile; must be 128 (tiles are 128 x 32).
 * fmt:    BSFP8_E4M3 (F = 448) or BSFP8_E5M2 (F = 57344).
 * codes:  out, rows x k bytes, row stride k, 16-byte aligned.
 * scales: out, FP32 [ceil(rows / 128)][k / 32], K-block index fastest.
 *
 * Per tile: amax = max |x|, s = amax / F rounded to FP32 (s = 1 when that is
 * zero), code = saturating round-to-nearest-even of (x / s rounded to FP32).
 * Output is bit-exact: the same bytes on every call and every launch shape.
 * Finite inputs only.  A B operand (K x N column-major) is quantised by
 * passing its N x K storage: rows = N, k = K, giving the 32 x 128 (K x N)
 * tiles of the pages.
 */
bsfp8_status fp8_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int tile_rows,
                          bsfp8_format fmt, uint8_t* codes, float* scales, hipStream_t stream);

/*
 * fp8_quantize_pair -- fp8_quantize of the two operands of one GEMM, A
 * (a_rows x k) and B (b_rows x k, N x K storage), in a single launch
 * ([CDNA4-FP8] sections 3.3 and 4.2; 128 x 32 tiles as fp8_quantize).
 *
 * Each operand takes the arguments, layout, alignment and ownership rules of
 * fp8_quantize for its side (x, ld, fmt, codes, scales), with one shared k.
 * The outputs are byte-for-byte those of two fp8_quantize calls.  Either side
 * may have 0 rows (its pointers are then ignored).  Errors as fp8_quantize;
 * nothing is launched unless both sides pass the checks.  The two sides'
 * buffers must not overlap.
 */
bsfp8_status fp8_quantize_pair(const float* a, int64_t a_rows, int64_t a_ld, bsfp8_format a_fmt,
                               uint8_t* a_codes, float* a_scales, const float* b, int64_t b_rows,
                               int64_t b_ld, bsfp8_format b_fmt, uint8_t* b_codes, float* b_scales,
                               int64_t k, hipStream_t stream);

/*
 * fp8_quantize_transposed -- per-tile FP8 quantisation of x^T, for operands
 * stored the other way round, such as the gradient G and activation X of a
 * weight-gradient product dW = G^T X ([CDNA4-FP8] section 3.3's per-tile
 * scales; section 2.2 of the same page puts gradients in E5M2).
 *
 * x:      k x rows FP32, row-major, leading dimension ld (elements):
 *         16-byte aligned, ld a multiple of 4, ld >= rows.
 * k:      >= 0, a multiple of 32 (the K dimension of the GEMM operand).
 * rows:   >= 0, any value (M for an A operand, N for a B operand).
 * tile_rows, fmt: as for fp8_quantize.
 * codes:  out, rows x k bytes, row stride k, 16-byte aligned.
 * scales: out, FP32 [ceil(rows / 128)][k / 32].
 *
 * The result is byte-for-byte that of fp8_quantize applied to an explicitly
 * transposed copy of x (rows x k, row-major); no transposed copy is made.
 */
bsfp8_status fp8_quantize_transposed(const float* x, int64_t k, int64_t rows, int64_t ld,
                                     int tile_rows, bsfp8_format fmt, uint8_t* codes,
                                     float* scales, hipStream_t stream);

/*
 * mxfp4_quantize -- MXFP4 block quantisation ([RUBIN-FP4] sections 2.1, 2.2, 3.1, 4.2).
 *
 * x:      rows x k FP32, row-major, leading dimension ld; 16-byte aligned,
 *         ld a multiple of 4, ld >= k.  rows >= 0; k >= 0, a multiple of 32.
 * packed: out, rows x (k / 2) bytes, row stride k / 2.  Element 2i sits in the
 *         low nibble of byte i, element 2i+1 in the high nibble.
 * scales: out, E8M0 bytes [rows][k / 32].
 *
 * Per 32-element block of a row: e = the smallest integer with 6 * 2^e >= amax
 * (e = 0 when amax is 0), clamped to [-127, 127]; scale byte = e + 127;
 * element code = round-to-nearest-even E2M1 of x * 2^-e (exact scaling).
 * Bit-exact.  Finite inputs only.
 */
bsfp8_status mxfp4_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                            uint8_t* packed, uint8_t* scales, hipStream_t stream);

/*
 * scaled_gemm -- D = deq(A) * deq(B) with FP32 accumulation
 * ([CDNA4-FP8] sections 2.3, 3.2-3.4, 4.3, 4.4; [RUBIN-FP4] sections 2.2, 3.1-3.3).
 *
 * M, N >= 0 (any value; edge tiles are masked), K >= 0 a multiple of 32.
 * FP8 operands (a_fmt, b_fmt each BSFP8_E4M3 or BSFP8_E5M2, any mix):
 *   a: M x K codes (row stride K); a_scales: FP32 [ceil(M/128)][K/32]
 *   b: N x K codes (row stride K); b_scales: FP32 [ceil(N/128)][K/32]
 *   exactly the outputs of fp8_quantize with tile_rows = 128.
 *   Each 32-wide K block's partial product is scaled by
 *   a_scale(tile, block) * b_scale(tile, block) before it is accumulated.
 * MXFP4 operands (a_fmt = b_fmt = BSFP8_MXFP4):
 *   a: M x K/2 packed bytes; a_scales: E8M0 [M][K/32]
 *   b: N x K/2 packed bytes; b_scales: E8M0 [N][K/32]
 *   (the outputs of mxfp4_quantize).
 * out:  BSFP8_OUT_F32, BSFP8_OUT_BF16 or BSFP8_OUT_F16 (the last two round
 *       to nearest even; [CDNA4-FP8] section 4.4 writes 16-bit results to halve
 *       the output traffic).
 * d:    M x N row-major, leading dimension ldd >= N (elements), aligned to
 *       its element size.
 * a, b must be 16-byte aligned.  K = 0 writes zeros.  FP8 operands need
 * K < 2^24 (the kernel addresses a 128-row band of an operand with 32-bit
 * offsets) and MXFP4 operands K < 2^26 (a 32-row band); larger K returns
 * BSFP8_ERR_UNSUPPORTED.  M and N are limited only
 * by the 2^31 - 1 bound on each dimension and on the number of 128 x 128 tiles.
 *
 * Accuracy: with S = sum_k |a_k b_k| (dequantised operands), every output
 * satisfies |D - exact| <= 2^-19 S for FP32 output and <= 2^-7 S for bf16 and
 * FP16 output on the synthetic workloads the library is tested on.  The FP8
 * matrix instructions used for 16-bit outputs align each group of 8 products
 * to 13 fraction bits below the group's largest exponent and cut the rest
 * (the truncation studied for Hopper in [HOPPER-MMA] is present on gfx950
 * too): at most 7 * 2^-13 S per 32-element block.  FP32 output widens the
 * codes to bf16 and uses instructions that keep 24 fraction bits: about
 * 2^-20.4 S per block, plus one FP32 rounding per block of the accumulation.
 */
bsfp8_status scaled_gemm(int64_t M, int64_t N, int64_t K,
                         bsfp8_format a_fmt, const void* a, const void* a_scales,
                         bsfp8_format b_fmt, const void* b, const void* b_scales,
                         bsfp8_out out, void* d, int64_t ldd, hipStream_t stream);

/*
 * scaled_gemm_ex -- D = alpha * deq(A) deq(B) + beta * C (the alpha/beta
 * epilogue of the CUTLASS argument list in [RUBIN-FP4] section 3.4).
 *
 * All arguments as for scaled_gemm, plus:
 * alpha: scales the FP32 accumulator (alpha * acc is rounded to FP32).
 * c:     M x N row-major, the same element type as d, leading dimension
 *        ldc >= N, aligned to its element size.  Read only when beta != 0
 *        (then it must not be null); it may be d itself (with ldc == ldd) to
 *        accumulate in place.  Any other overlap of c and d is undefined.
 * beta:  beta * C is added to alpha * acc with one FP32 fused multiply-add,
 *        then the sum is converted to the output type.
 * K = 0 writes beta * C (zeros when beta == 0).
 * scaled_gemm(...) is scaled_gemm_ex(..., 1.0f, NULL, 0, 0.0f, ...).
 *
 * Accuracy: |D - (alpha exact + beta C)| <= tau (|alpha| S + |beta C|), with
 * tau as for scaled_gemm (plus one FP32 rounding for FP32 output).
 */
bsfp8_status scaled_gemm_ex(int64_t M, int64_t N, int64_t K,
                            bsfp8_format a_fmt, const void* a, const void* a_scales,
                            bsfp8_format b_fmt, const void* b, const void* b_scales,
                            float alpha, const void* c, int64_t ldc, float beta,
                            bsfp8_out out, void* d, int64_t ldd, hipStream_t stream);

/*
 * Scale granularity of an operand ([CDNA4-FP8] section 3.3 weighs per-row,
 * per-column and per-tensor scales against per-tile ones and keeps per tile;
 * its closing section keeps a per-matrix scale for evenly distributed data).
 * The rows are those of the operand's rows x K storage: per-row scales of A
 * are per output row, per-row scales of B (stored N x K) are per output column.
 */
typedef enum {
    BSFP8_GRAN_TILE = 0,    /* FP8: FP32 [ceil(rows / 128)][K / 32], one per 128 x 32 tile */
    BSFP8_GRAN_ROW = 1,     /* FP8: FP32 [rows], one per row, constant along K */
    BSFP8_GRAN_TENSOR = 2,  /* FP8: FP32 [1], one for the whole operand */
    BSFP8_GRAN_MX32 = 3     /* MXFP4: E8M0 [rows][K / 32], one per 32-element K block */
} bsfp8_granularity;

/*
 * fp8_quantize_granular -- FP8 quantisation with the scale granularity g.
 *
 * x, rows, k, ld, fmt, codes: as for fp8_quantize.
 * g: BSFP8_GRAN_TILE (exactly fp8_quantize with tile_rows = 128),
 *    BSFP8_GRAN_ROW or BSFP8_GRAN_TENSOR; BSFP8_GRAN_MX32 is UNSUPPORTED.
 * scales: out, FP32, the shape g names (4-byte aligned).
 *
 * Per scale group (tile, row or whole operand): amax = max |x|, s = amax / F
 * rounded to FP32 (s = 1 when that is zero), code = saturating round-to-
 * nearest-even of (x / s rounded to FP32).  Bit-exact.  rows == 0 or k == 0
 * writes nothing.  BSFP8_GRAN_TENSOR runs three launches and keeps partial
 * maxima in the codes buffer between them, so reads of codes or scales[0]
 * that overlap the call race with it.
 */
bsfp8_status fp8_quantize_granular(const float* x, int64_t rows, int64_t k, int64_t ld,
                                   bsfp8_granularity g, bsfp8_format fmt, uint8_t* codes,
                                   float* scales, hipStream_t stream);

/*
 * scaled_gemm_granular -- scaled_gemm_ex with a scale granularity per operand:
 * D = alpha * deq(A) deq(B) + beta * C, deq(X)[r][k] = code * scale(r, k).
 *
 * All arguments as for scaled_gemm_ex, plus a_g and b_g, the granularities of
 * a_scales and b_scales.  Supported combinations:
 *   FP8, both scales constant along K (ROW or TENSOR on each side): the scale
 *     product multiplies the FP32 sum over all of K once, at write-back.
 *   FP8, TILE with TILE or TENSOR: the product of the two K block scales
 *     multiplies each 32-wide K block's partial sum, as in scaled_gemm.
 *   FP8, TILE with ROW (either side): the TILE side's K block scale
 *     multiplies each K block's partial sum, and the ROW side's scale (of the
 *     output row for A, of the output column for B) multiplies the FP32 sum
 *     over K at write-back.
 *   MXFP4: MX32 on both sides (as scaled_gemm).
 * Other combinations return BSFP8_ERR_UNSUPPORTED, and so does K >= 2^23
 * with both FP8 scales constant along K.
 * Accuracy as for scaled_gemm_ex.
 */
bsfp8_status scaled_gemm_granular(int64_t M, int64_t N, int64_t K,
                                  bsfp8_format a_fmt, const void* a, const void* a_scales,
                                  bsfp8_granularity a_g,
                                  bsfp8_format b_fmt, const void* b, const void* b_scales,
                                  bsfp8_granularity b_g,
                                  float alpha, const void* c, int64_t ldc, float beta,
                                  bsfp8_out out, void* d, int64_t ldd, hipStream_t stream);

/*
 * MX variants ([RUBIN-FP4] section 5.3 offers blocks of 16 or 8 elements where
 * 32 is too coarse; section 3.2 offers FP16 or BF16 block scales where a power
 * of two is too coarse, at twice the scale storage).
 */
typedef enum {
    BSFP8_MX_E8M0 = 0,  /* one byte, 2^(code - 127) */
    BSFP8_MX_F16 = 1,   /* IEEE binary16 bit pattern */
    BSFP8_MX_BF16 = 2   /* bfloat16 bit pattern (upper half of a binary32) */
} bsfp8_mx_scale;
/*
 * mx_quantize -- E2M1 quantisation with blocks of `block` consecutive K
 * elements (32, 16 or 8) and block scales of format sfmt.
 *
 * x:      rows x k FP32, row-major, leading dimension ld; 16-byte aligned,
 *         ld a multiple of 4, ld >= k.  rows >= 0; k >= 0, a multiple of 32.
 * packed: out, rows x (k / 2) bytes, row stride k / 2, low nibble first.
 * scales: out, [rows][k / block]: bytes (E8M0) or 16-bit patterns (FP16,
 *         BF16, 2-byte aligned).
 *
 * Per block, amax = max |x|:
 *   E8M0: as mxfp4_quantize (block = 32 with E8M0 is exactly mxfp4_quantize);
 *   FP16 / BF16: s = the format's value nearest to amax / 6 (ties to even),
 *         the largest finite value when beyond it, 1 when it is zero (or
 *         amax is 0); code = saturating round-to-nearest-even E2M1 of
 *         (x / s rounded to FP32).
 * Bit-exact.  Finite inputs only.
 */
bsfp8_status mx_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int block,
                         bsfp8_mx_scale sfmt, uint8_t* packed, void* scales, hipStream_t stream);

/*
 * scaled_gemm_mx -- D = alpha * deq(A) deq(B) + beta * C for E2M1 operands
 * with blocks of `block` (32, 16, 8) K values and sfmt block scales, as
 * mx_quantize writes them.
 *
 * a: M x K/2 packed bytes, a_scales [M][K/block]; b: N x K/2 packed bytes
 * (the K x N column-major operand), b_scales [N][K/block]; a and b 16-byte
 * aligned, the scale arrays 8-byte aligned.  M, N >= 0; K >= 0 a multiple of
 * 32, below 2^23 unless block == 32 with E8M0 scales (BSFP8_ERR_UNSUPPORTED).
 * alpha, c, ldc, beta, out, d, ldd: as for scaled_gemm_ex.
 * block = 32 with E8M0 scales runs the block-scaled MXFP4 GEMM of
 * scaled_gemm.  block = 16 or 8 with E8M0 scales runs on the same
 * block-scaled instruction (block = 8 except on shapes with at least 128
 * tiles of 256 x 256 that the large MXFP4 tiling does not take):
 * each 32-value K block of an operand lane is multiplied in 32 / block
 * passes, one per block with the other values zeroed, each under its own
 * block's scale, so every block keeps its exact scale.  Every other combination is beyond
 * the matrix instructions' block scaling (one E8M0 scale per 32 K values): its
 * operands are dequantised exactly to bf16 (a wide scale as an exact bf16
 * pair hi + lo) and multiplied with FP32 accumulation; 16-bit outputs leave
 * out the lo * lo products (below 2^-16 of hi * hi).  Accuracy as for
 * scaled_gemm_ex.
 */
bsfp8_status scaled_gemm_mx(int64_t M, int64_t N, int64_t K, int block, bsfp8_mx_scale sfmt,
                            const void* a, const void* a_scales, const void* b,
                            const void* b_scales, float alpha, const void* c, int64_t ldc,
                            float beta, bsfp8_out out, void* d, int64_t ldd, hipStream_t stream);

/*
 * scaled_gemm_quantize_a -- D = alpha * deq(Q(x)) deq(B) + beta * C, where
 * Q(x) is the per-tile FP8 quantisation of the FP32 matrix x, carried out
 * inside the GEMM while x is loaded (activations quantised online:
 * [CDNA4-FP8] section 4.2 converts and scales on load, section 3.3 computes
 * each tile's scale from its maximum; [RUBIN-FP4] section 4.2, step 4).
 *
 * x:       M x K FP32, row-major, leading dimension ldx (elements): 16-byte
 *          aligned, ldx a multiple of 4, K <= ldx < 2^22.
 * a_fmt:   the FP8 format of A's codes (E4M3 or E5M2).
 * b_fmt, b, b_scales: as for scaled_gemm; b_g is BSFP8_GRAN_TILE (b_scales
 *          FP32 [ceil(N/128)][K/32]) or BSFP8_GRAN_TENSOR (b_scales FP32 [1]).
 * alpha, c, ldc, beta, out, d, ldd: as for scaled_gemm_ex.
 * a_codes, a_scales: both NULL, or both non-NULL and 4-byte aligned: then
 *          they receive A's codes (M x K bytes, row stride K) and scales
 *          (FP32 [ceil(M/128)][K/32]), byte-for-byte what fp8_quantize with
 *          tile_rows = 128 writes for x (for instance to keep the quantised
 *          activations for a backward pass).  With them and N > 384 the call
 *          runs fp8_quantize into them and then the GEMM (two launches, the
 *          same result): quantising every A tile once beats re-quantising it
 *          for every column of output tiles.
 *
 * The codes the GEMM multiplies are exactly those of fp8_quantize, so D is
 * that of fp8_quantize followed by scaled_gemm_ex, with the same accuracy.
 * M, N >= 0 (any value), K >= 0 a multiple of 32.  K = 0 writes beta * C.
 * N = 0 writes only a_codes / a_scales (when given).  x must not overlap d,
 * a_codes or a_scales.  Every output tile that reads the same rows of x
 * quantises them again, so the single-launch form pays off on narrow outputs
 * (a few hundred columns) and small, launch-bound products.
 */
bsfp8_status scaled_gemm_quantize_a(int64_t M, int64_t N, int64_t K, const float* x, int64_t ldx,
                                    bsfp8_format a_fmt, bsfp8_format b_fmt, const void* b,
                                    const void* b_scales, bsfp8_granularity b_g, float alpha,
                                    const void* c, int64_t ldc, float beta, bsfp8_out out,
                                    void* d, int64_t ldd, uint8_t* a_codes, float* a_scales,
                                    hipStream_t stream);

/*
 * bsfp8_status_string -- the name of a status code ("BSFP8_OK", ...;
 * "BSFP8_ERR_UNKNOWN" for a value that is not a bsfp8_status), in static
 * storage owned by the library; never NULL.  The status values follow the
 * check-then-run flow of the CUTLASS GEMM interface in [RUBIN-FP4] section
 * 3.4 (can_implement, then initialize and run): every argument check happens
 * before anything runs, and a rejected call reports why instead of running.
 */
const char* bsfp8_status_string(bsfp8_status s);

/* Library version, (major << 16) | minor. */
int bsfp8_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BSFP8_H */
