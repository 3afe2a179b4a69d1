/*
 * oracle.h -- CPU oracle for block-scaled FP8 / MXFP4 quantisation and GEMM.
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.
 */
#ifndef BSFP8_ORACLE_H
#define BSFP8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_E4M3 = 0, ORC_E5M2 = 1, ORC_E2M1 = 2, ORC_E8M0 = 3, ORC_MXFP4 = 2 };
/* block scale formats of oracle_mx_quantize */
enum { ORC_SCALE_E8M0 = 0, ORC_SCALE_F16 = 1, ORC_SCALE_BF16 = 2 };

int oracle_decode_table(int fmt, double* out);          /* returns entry count */
double oracle_decode(int fmt, unsigned code);
unsigned oracle_encode(int fmt, double v);               /* saturating RNE */
void oracle_encode_array(int fmt, const double* v, int64_t n, uint8_t* codes);
int oracle_mx_exponent(double amax);

int oracle_fp8_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                        int64_t tile_rows, int fmt, uint8_t* codes, float* scales);
int oracle_fp8_quantize_groups(const float* x, int64_t rows, int64_t k, int64_t ld,
                               int64_t group_rows, int64_t group_k, int fmt, uint8_t* codes,
                               float* scales);
int oracle_mxfp4_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                          uint8_t* packed, uint8_t* scales);
int oracle_mx_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int64_t block,
                       int sfmt, uint8_t* packed, void* scales);

int oracle_gemm_rows(int64_t M, int64_t N, int64_t K, int64_t tile_rows,
                     int a_fmt, const uint8_t* a, const void* a_scales,
                     int b_fmt, const uint8_t* b, const void* b_scales,
                     int64_t row0, int64_t row1, double* d, double* s);
int oracle_gemm_points(int64_t M, int64_t N, int64_t K, int64_t tile_rows,
                       int a_fmt, const uint8_t* a, const void* a_scales,
                       int b_fmt, const uint8_t* b, const void* b_scales,
                       int64_t npts, const int64_t* ii, const int64_t* jj,
                       double* d, double* s);

int oracle_threads(void);
void oracle_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
