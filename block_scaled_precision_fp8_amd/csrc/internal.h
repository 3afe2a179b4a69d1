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
hipError_t launch_fp8_quantize_t(const float* x, int64_t k, int64_t rows, int64_t ld, int fmt,
                                 uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_mxfp4_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                                 uint8_t* packed, uint8_t* scales, hipStream_t stream);
hipError_t launch_gemm_fp8(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                           const float* a_scales, int b_fmt, const uint8_t* b,
                           const float* b_scales, int out, void* d, int64_t ldd,
                           hipStream_t stream);
hipError_t launch_gemm_mxfp4(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                             const uint8_t* a_scales, const uint8_t* b, const uint8_t* b_scales,
                             int out, void* d, int64_t ldd, hipStream_t stream);
hipError_t launch_fill_zero(int64_t M, int64_t N, int out, void* d, int64_t ldd,
                            hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// FP32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
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
