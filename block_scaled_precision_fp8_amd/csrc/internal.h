// internal.h -- private declarations shared by the HIP sources of libbsfp8.
// Not installed; the public interface is include/bsfp8.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsfp8.h"

namespace bsfp8 {

// Host-side launchers; each assumes its arguments were validated by the API
// layer and returns the launch status.
hipError_t launch_fp8_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int fmt,
                               uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_fp8_quantize_pair(const float* a, int64_t rows_a, int64_t lda, int fmt_a,
                                    uint8_t* codes_a, float* scales_a, const float* b, int64_t rows_b,
                                    int64_t ldb, int fmt_b, uint8_t* codes_b, float* scales_b, int64_t k,
                                    hipStream_t stream);
hipError_t launch_fp8_quantize_t(const float* x, int64_t k, int64_t rows, int64_t ld, int fmt,
                                 uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_fp8_quantize_rows(const float* x, int64_t rows, int64_t k, int64_t ld, int fmt,
                                    uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_fp8_quantize_tensor(const float* x, int64_t rows, int64_t k, int64_t ld, int fmt,
                                      uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_mxfp4_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                                 uint8_t* packed, uint8_t* scales, hipStream_t stream);
// E2M1 with blocks of `block` (32, 16, 8) K elements and sfmt block scales
hipError_t launch_mx_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int block,
                              int sfmt, uint8_t* packed, void* scales, hipStream_t stream);
// The GEMM epilogue: D = alpha * (A B) + beta * C, C of D's element type.
// beta == 0 means C is not read (c may be null).  row_scale (col_scale), when
// set, multiplies output row m (column n) by row_scale[m] (col_scale[n]): the
// per-row scales of an operand whose other side has per-tile scales, applied
// to the FP32 sum at write-back (only finish_row_chunk applies them).
struct Epilogue {
    float alpha;
    float beta;
    const void* c;
    int64_t ldc;
    const float* row_scale = nullptr;
    const float* col_scale = nullptr;
};

// Per-tile FP8 scales; bit 0 (bit 1) of tensor_mask marks a_scales (b_scales)
// as one scale for the whole operand instead, and bit 2 (bit 3) with it makes
// that scale 1 (the operand's per-row scales ride in the epilogue).
hipError_t launch_gemm_fp8(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                           const float* a_scales, int b_fmt, const uint8_t* b,
                           const float* b_scales, int out, void* d, int64_t ldd,
                           const Epilogue& ep, hipStream_t stream, int tensor_mask = 0);
// The 256 x 256-tile form of the per-tile FP8 GEMM (same arithmetic, no
// online A); fits when the problem has enough 256 x 256 tiles to fill the chip.
bool gemm_fp8_big_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_fp8_big(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                               const float* a_scales, int b_fmt, const uint8_t* b,
                               const float* b_scales, int out, void* d, int64_t ldd,
                               const Epilogue& ep, int tensor_mask, hipStream_t stream);
// FP8 operands whose scales are constant along K: a_scales[m * a_step] and
// b_scales[n * b_step] (step 1 for per-row scales, 0 for one per tensor).
// The skinny per-tile GEMM in its K-constant-scales form (up to 64 rows).
bool skinny_outer_fits(int64_t M);
hipError_t launch_gemm_fp8_skinny_outer(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                                        const float* a_scales, int a_step, int b_fmt, const uint8_t* b,
                                        const float* b_scales, int b_step, int out, void* d, int64_t ldd,
                                        const Epilogue& ep, hipStream_t stream);
hipError_t launch_gemm_fp8_outer(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                                 const float* a_scales, int a_step, int b_fmt, const uint8_t* b,
                                 const float* b_scales, int b_step, int out, void* d, int64_t ldd,
                                 const Epilogue& ep, hipStream_t stream);
// The A operand given in FP32 (x, M x K, leading dimension ldx elements) and
// quantised per 128 x 32 tile inside the per-tile FP8 GEMM, exactly as
// launch_fp8_quantize would; codes / scales, when not null, receive copies of
// A's codes (M x K, row stride K) and scales ([ceil(M / 128)][K / 32]).
struct OnlineA {
    const float* x;
    int64_t ldx;
    uint8_t* codes;
    float* scales;
};
// b_tensor: b_scales is one scale for the whole of B.
hipError_t launch_gemm_fp8_online_a(int64_t M, int64_t N, int64_t K, int a_fmt, const OnlineA& qa,
                                    int b_fmt, const uint8_t* b, const float* b_scales,
                                    int b_tensor, int out, void* d, int64_t ldd,
                                    const Epilogue& ep, hipStream_t stream);
hipError_t launch_gemm_mxfp4(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                             const uint8_t* a_scales, const uint8_t* b, const uint8_t* b_scales,
                             int out, void* d, int64_t ldd, const Epilogue& ep,
                             hipStream_t stream);
// E2M1 operands with blocks of 16 or 8 K values and E8M0 scales on the
// block-scaled FP4 instruction (two or four MFMAs per 64 K, each on one block
// of every lane's 32 values, the others zero): the skinny MXFP4 kernel for
// up to 64 rows or few tiles, the large-tile one where mx_fp4_big_applies (K
// a multiple of 256, enough 256 x 256 tiles), else the 128 x 128 one.
bool mx_fp4_big_applies(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_mx_fp4(int64_t M, int64_t N, int64_t K, int block, const uint8_t* a,
                              const uint8_t* a_scales, const uint8_t* b, const uint8_t* b_scales,
                              int out, void* d, int64_t ldd, const Epilogue& ep, hipStream_t stream);
// E2M1 operands with blocks of `block` K values and sfmt block scales
// (not the hardware-scaled block = 32 / E8M0 case), dequantised to bf16;
// E8M0 blocks of 16 and 8 go to launch_gemm_mx_fp4 wherever one of its
// forms applies.
hipError_t launch_gemm_mx(int64_t M, int64_t N, int64_t K, int block, int sfmt, const uint8_t* a,
                          const void* a_scales, const uint8_t* b, const void* b_scales, int out,
                          void* d, int64_t ldd, const Epilogue& ep, hipStream_t stream);
// K = 0: D = beta * C (zeros when beta == 0).
hipError_t launch_fill(int64_t M, int64_t N, int out, void* d, int64_t ldd, const Epilogue& ep,
                       hipStream_t stream);
// 16-byte row stores of D (and loads of C) are allowed: row strides and base
// pointers all 16-byte aligned.
inline int vec16_ok(int out, const void* d, int64_t ldd, const Epilogue& ep) {
    const int64_t es = out == BSFP8_OUT_F32 ? 4 : 2;
    const bool dok = (ldd * es) % 16 == 0 && reinterpret_cast<uintptr_t>(d) % 16 == 0;
    const bool cok = ep.beta == 0.0f ||
                     ((ep.ldc * es) % 16 == 0 && reinterpret_cast<uintptr_t>(ep.c) % 16 == 0);
    return dok && cok ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Output element conversions, round to nearest even (FP16 overflows to +-inf).
template <int OUT>
__device__ __forceinline__ uint16_t to_half_bits(float v) {
    if constexpr (OUT == BSFP8_OUT_BF16) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}
template <int OUT>
__device__ __forceinline__ float from_half_bits(uint16_t h) {
    if constexpr (OUT == BSFP8_OUT_BF16) return __uint_as_float(static_cast<uint32_t>(h) << 16);
    else return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Finish NV (4 or 8) consecutive outputs D[m][n .. n+NV-1]: v = alpha * acc
// (times the row and column scales when set) (+ beta * C), converted to the output type; masked at the edges, one
// 16-byte store when vec allows (NV = 4 for FP32, 8 for 16-bit outputs).
template <int OUT, int NV>
__device__ __forceinline__ void finish_row_chunk(void* D, int64_t ldd, const Epilogue& ep, int m,
                                                 int n, int M, int N, int vec, const float* acc) {
    if (m >= M) return;
    float v[NV];
    if (ep.row_scale || ep.col_scale) {
        const float rs = ep.row_scale ? ep.row_scale[m] : 1.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const float cs = ep.col_scale && n + j < N ? ep.col_scale[n + j] : 1.0f;
            v[j] = ep.alpha * ((rs * cs) * acc[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = ep.alpha * acc[j];
    }
    const bool full = vec && n + NV <= N;
    if (ep.beta != 0.0f) {
        if constexpr (OUT == BSFP8_OUT_F32) {
            const float* cp = static_cast<const float*>(ep.c) + static_cast<int64_t>(m) * ep.ldc + n;
            if (full) {
                const float4 c4 = *reinterpret_cast<const float4*>(cp);
                v[0] = fmaf(ep.beta, c4.x, v[0]); v[1] = fmaf(ep.beta, c4.y, v[1]);
                v[2] = fmaf(ep.beta, c4.z, v[2]); v[3] = fmaf(ep.beta, c4.w, v[3]);
            } else {
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    if (n + j < N) v[j] = fmaf(ep.beta, cp[j], v[j]);
            }
        } else {
            const uint16_t* cp = static_cast<const uint16_t*>(ep.c) + static_cast<int64_t>(m) * ep.ldc + n;
            if (full) {
                uint32_t w[4];
                if constexpr (NV == 8) {
                    const uint4 c4 = *reinterpret_cast<const uint4*>(cp);
                    w[0] = c4.x; w[1] = c4.y; w[2] = c4.z; w[3] = c4.w;
                } else {
                    const uint2 c2 = *reinterpret_cast<const uint2*>(cp);
                    w[0] = c2.x; w[1] = c2.y; w[2] = 0u; w[3] = 0u;
                }
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    v[j] = fmaf(ep.beta, from_half_bits<OUT>(static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)))), v[j]);
            } else {
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    if (n + j < N) v[j] = fmaf(ep.beta, from_half_bits<OUT>(cp[j]), v[j]);
            }
        }
    }
    if constexpr (OUT == BSFP8_OUT_F32) {
        float* dp = static_cast<float*>(D) + static_cast<int64_t>(m) * ldd + n;
        if (full) {
            *reinterpret_cast<float4*>(dp) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int j = 0; j < NV; ++j)
                if (n + j < N) dp[j] = v[j];
        }
    } else {
        uint16_t* dp = static_cast<uint16_t*>(D) + static_cast<int64_t>(m) * ldd + n;
        uint16_t h[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) h[j] = to_half_bits<OUT>(v[j]);
        if (full) {
            if constexpr (NV == 8)
                *reinterpret_cast<uint4*>(dp) =
                    make_uint4(h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16),
                               h[4] | (static_cast<uint32_t>(h[5]) << 16), h[6] | (static_cast<uint32_t>(h[7]) << 16));
            else
                *reinterpret_cast<uint2*>(dp) =
                    make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16));
        } else {
#pragma unroll
            for (int j = 0; j < NV; ++j)
                if (n + j < N) dp[j] = h[j];
        }
    }
}

// Store 8 already converted 16-bit outputs D[m][n .. n+7] (masked at the edges).
__device__ __forceinline__ void store_half8(void* D, int64_t ldd, int m, int n, int M, int N,
                                            int vec, uint4 w) {
    if (m >= M) return;
    uint16_t* dp = static_cast<uint16_t*>(D) + static_cast<int64_t>(m) * ldd + n;
    if (vec && n + 8 <= N) {
        *reinterpret_cast<uint4*>(dp) = w;
        return;
    }
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (n + j < N) dp[j] = static_cast<uint16_t>(ww[j >> 1] >> (16 * (j & 1)));
}

// Map a linear workgroup id to an output tile (tm, tn).
// Workgroups are handed to the 8 XCDs round-robin; when the tile count allows
// it, consecutive logical tiles are gathered onto one XCD so that they share
// that XCD's L2.  Within that order, tiles are walked in groups of `group`
// tile-rows so that a group's A rows and B columns stay cache-resident.
__device__ __forceinline__ void map_tile(int pid, int tiles_m, int tiles_n, int group,
                                         int* tm, int* tn) {
    const int total = tiles_m * tiles_n;
    if ((total & 7) == 0) {
        const int per = total >> 3;
        pid = (pid & 7) * per + (pid >> 3);
    }
    const int span = group * tiles_n;
    const int g = pid / span;
    const int first = g * group;
    int gm = tiles_m - first;
    if (gm > group) gm = group;
    const int r = pid - g * span;
    *tm = first + r % gm;
    *tn = r / gm;
}

}  // namespace bsfp8
