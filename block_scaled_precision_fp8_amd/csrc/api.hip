// api.hip -- the C ABI of libbsfp8 (declared in include/bsfp8.h).
// Validates every argument on the host, then launches; a non-OK status means
// nothing was launched.  No allocation, no synchronisation, no global state.
#include "internal.h"

#include <limits>

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline bool is_fp8(int f) { return f == BSFP8_E4M3 || f == BSFP8_E5M2; }
constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();
// scaled_gemm_quantize_a: from this many 128-wide output column tiles on, a
// call that also asks for A's codes quantises A once and runs the per-tile
// GEMM (measured on MI355X: the in-kernel quantisation costs about one GEMM's
// time again, the separate pass about M K 5 bytes at 5.5 TB/s, which it
// undercuts below about 450 output columns)
constexpr int64_t kOnlineMaxColumnTiles = 4;

inline bsfp8_status from_hip(hipError_t e) { return e == hipSuccess ? BSFP8_OK : BSFP8_ERR_HIP; }

}  // namespace

extern "C" {

bsfp8_status fp8_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int tile_rows,
                          bsfp8_format fmt, uint8_t* codes, float* scales, hipStream_t stream) {
    if (!is_fp8(fmt)) return BSFP8_ERR_UNSUPPORTED;
    if (tile_rows != 128) return BSFP8_ERR_UNSUPPORTED;
    if (rows < 0 || k < 0 || ld < k || (k % 32) != 0) return BSFP8_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return BSFP8_OK;
    if (!x || !codes || !scales) return BSFP8_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld % 4) != 0 || !aligned(codes, 4) || !aligned(scales, 4))
        return BSFP8_ERR_INVALID_ARG;
    const int64_t blocks = ((rows + 127) / 128) * ((k + 127) / 128);
    if (blocks > kI32Max) return BSFP8_ERR_INVALID_ARG;
    return from_hip(bsfp8::launch_fp8_quantize(x, rows, k, ld, fmt, codes, scales, stream));
}

bsfp8_status fp8_quantize_pair(const float* a, int64_t a_rows, int64_t a_ld, bsfp8_format a_fmt,
                               uint8_t* a_codes, float* a_scales, const float* b, int64_t b_rows,
                               int64_t b_ld, bsfp8_format b_fmt, uint8_t* b_codes, float* b_scales,
                               int64_t k, hipStream_t stream) {
    if (!is_fp8(a_fmt) || !is_fp8(b_fmt)) return BSFP8_ERR_UNSUPPORTED;
    if (a_rows < 0 || b_rows < 0 || k < 0 || a_ld < k || b_ld < k || (k % 32) != 0)
        return BSFP8_ERR_INVALID_ARG;
    if (k == 0) return BSFP8_OK;
    if (a_rows == 0) a = nullptr;
    if (b_rows == 0) b = nullptr;
    if (a_rows > 0 && (!a || !a_codes || !a_scales || !aligned(a, 16) || (a_ld % 4) != 0 ||
                       !aligned(a_codes, 4) || !aligned(a_scales, 4)))
        return BSFP8_ERR_INVALID_ARG;
    if (b_rows > 0 && (!b || !b_codes || !b_scales || !aligned(b, 16) || (b_ld % 4) != 0 ||
                       !aligned(b_codes, 4) || !aligned(b_scales, 4)))
        return BSFP8_ERR_INVALID_ARG;
    const int64_t ncb = (k + 127) / 128;
    if (((a_rows + 127) / 128 + (b_rows + 127) / 128) * ncb > kI32Max) return BSFP8_ERR_INVALID_ARG;
    return from_hip(bsfp8::launch_fp8_quantize_pair(a, a_rows, a_ld, a_fmt, a_codes, a_scales, b, b_rows,
                                                    b_ld, b_fmt, b_codes, b_scales, k, stream));
}

bsfp8_status fp8_quantize_transposed(const float* x, int64_t k, int64_t rows, int64_t ld,
                                     int tile_rows, bsfp8_format fmt, uint8_t* codes,
                                     float* scales, hipStream_t stream) {
    if (!is_fp8(fmt)) return BSFP8_ERR_UNSUPPORTED;
    if (tile_rows != 128) return BSFP8_ERR_UNSUPPORTED;
    if (rows < 0 || k < 0 || ld < rows || (k % 32) != 0) return BSFP8_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return BSFP8_OK;
    if (!x || !codes || !scales) return BSFP8_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld % 4) != 0 || !aligned(codes, 16) || !aligned(scales, 4))
        return BSFP8_ERR_INVALID_ARG;
    const int64_t blocks = ((rows + 127) / 128) * ((k + 127) / 128);
    if (blocks > kI32Max) return BSFP8_ERR_INVALID_ARG;
    return from_hip(bsfp8::launch_fp8_quantize_t(x, k, rows, ld, fmt, codes, scales, stream));
}

bsfp8_status fp8_quantize_granular(const float* x, int64_t rows, int64_t k, int64_t ld,
                                   bsfp8_granularity g, bsfp8_format fmt, uint8_t* codes,
                                   float* scales, hipStream_t stream) {
    if (g == BSFP8_GRAN_TILE) return fp8_quantize(x, rows, k, ld, 128, fmt, codes, scales, stream);
    if (g != BSFP8_GRAN_ROW && g != BSFP8_GRAN_TENSOR) return BSFP8_ERR_UNSUPPORTED;
    if (!is_fp8(fmt)) return BSFP8_ERR_UNSUPPORTED;
    if (rows < 0 || k < 0 || ld < k || (k % 32) != 0) return BSFP8_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return BSFP8_OK;
    if (!x || !codes || !scales) return BSFP8_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld % 4) != 0 || !aligned(codes, 4) || !aligned(scales, 4))
        return BSFP8_ERR_INVALID_ARG;
    if ((rows + 3) / 4 > kI32Max) return BSFP8_ERR_INVALID_ARG;
    if (g == BSFP8_GRAN_ROW)
        return from_hip(bsfp8::launch_fp8_quantize_rows(x, rows, k, ld, fmt, codes, scales, stream));
    return from_hip(bsfp8::launch_fp8_quantize_tensor(x, rows, k, ld, fmt, codes, scales, stream));
}

bsfp8_status mxfp4_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                            uint8_t* packed, uint8_t* scales, hipStream_t stream) {
    if (rows < 0 || k < 0 || ld < k || (k % 32) != 0) return BSFP8_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return BSFP8_OK;
    if (!x || !packed || !scales) return BSFP8_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld % 4) != 0 || !aligned(packed, 2)) return BSFP8_ERR_INVALID_ARG;
    const int64_t blocks = (rows * (k / 4) + 255) / 256;
    if (rows > kI32Max * 256 || blocks > kI32Max) return BSFP8_ERR_INVALID_ARG;
    return from_hip(bsfp8::launch_mxfp4_quantize(x, rows, k, ld, packed, scales, stream));
}

bsfp8_status mx_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int block,
                         bsfp8_mx_scale sfmt, uint8_t* packed, void* scales, hipStream_t stream) {
    if (block != 32 && block != 16 && block != 8) return BSFP8_ERR_UNSUPPORTED;
    if (sfmt != BSFP8_MX_E8M0 && sfmt != BSFP8_MX_F16 && sfmt != BSFP8_MX_BF16)
        return BSFP8_ERR_UNSUPPORTED;
    if (rows < 0 || k < 0 || ld < k || (k % 32) != 0) return BSFP8_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return BSFP8_OK;
    if (!x || !packed || !scales) return BSFP8_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (ld % 4) != 0 || !aligned(packed, 2)) return BSFP8_ERR_INVALID_ARG;
    if (sfmt != BSFP8_MX_E8M0 && !aligned(scales, 2)) return BSFP8_ERR_INVALID_ARG;
    const int64_t blocks = (rows * (k / 4) + 255) / 256;
    if (rows > kI32Max * 256 || blocks > kI32Max) return BSFP8_ERR_INVALID_ARG;
    return from_hip(bsfp8::launch_mx_quantize(x, rows, k, ld, block, sfmt, packed, scales, stream));
}

bsfp8_status scaled_gemm_granular(int64_t M, int64_t N, int64_t K, bsfp8_format a_fmt,
                                  const void* a, const void* a_scales, bsfp8_granularity a_g,
                                  bsfp8_format b_fmt, const void* b, const void* b_scales,
                                  bsfp8_granularity b_g, float alpha, const void* c, int64_t ldc,
                                  float beta, bsfp8_out out, void* d, int64_t ldd,
                                  hipStream_t stream) {
    const bool fp8 = is_fp8(a_fmt) && is_fp8(b_fmt);
    const bool mx = a_fmt == BSFP8_MXFP4 && b_fmt == BSFP8_MXFP4;
    if (!fp8 && !mx) return BSFP8_ERR_UNSUPPORTED;
    if (out != BSFP8_OUT_F32 && out != BSFP8_OUT_BF16 && out != BSFP8_OUT_F16)
        return BSFP8_ERR_UNSUPPORTED;
    // which kernel: per-tile FP8 (0), FP8 with scales constant along K (1), MXFP4 (2)
    int path;
    int tensor_mask = 0;
    if (mx) {
        if (a_g != BSFP8_GRAN_MX32 || b_g != BSFP8_GRAN_MX32) return BSFP8_ERR_UNSUPPORTED;
        path = 2;
    } else {
        const auto fp8_g = [](bsfp8_granularity g) {
            return g == BSFP8_GRAN_TILE || g == BSFP8_GRAN_ROW || g == BSFP8_GRAN_TENSOR;
        };
        if (!fp8_g(a_g) || !fp8_g(b_g)) return BSFP8_ERR_UNSUPPORTED;
        if (a_g != BSFP8_GRAN_TILE && b_g != BSFP8_GRAN_TILE) {
            path = 1;
        } else {
            // per-tile scales on one side: the other side's scale is per tile or
            // per tensor (in the K block product), or per row (a unit scale in the
            // product, and the row's scale on the FP32 sum at write-back)
            path = 0;
            tensor_mask = (a_g == BSFP8_GRAN_TENSOR ? 1 : 0) | (b_g == BSFP8_GRAN_TENSOR ? 2 : 0) |
                          (a_g == BSFP8_GRAN_ROW ? 1 | 4 : 0) | (b_g == BSFP8_GRAN_ROW ? 2 | 8 : 0);
        }
    }
    if (M < 0 || N < 0 || K < 0 || (K % 32) != 0) return BSFP8_ERR_INVALID_ARG;
    if (M > kI32Max || N > kI32Max || K > kI32Max) return BSFP8_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BSFP8_OK;
    const uintptr_t es = out == BSFP8_OUT_F32 ? 4 : 2;
    if (!d || ldd < N || !aligned(d, es)) return BSFP8_ERR_INVALID_ARG;
    if (beta != 0.0f && (!c || ldc < N || !aligned(c, es))) return BSFP8_ERR_INVALID_ARG;
    bsfp8::Epilogue ep{alpha, beta, beta != 0.0f ? c : nullptr, beta != 0.0f ? ldc : 0};
    if (K == 0) return from_hip(bsfp8::launch_fill(M, N, out, d, ldd, ep, stream));
    if (!a || !b || !a_scales || !b_scales) return BSFP8_ERR_INVALID_ARG;
    if (path == 0) {
        if (tensor_mask & 4) ep.row_scale = static_cast<const float*>(a_scales);
        if (tensor_mask & 8) ep.col_scale = static_cast<const float*>(b_scales);
    }
    if (!aligned(a, 16) || !aligned(b, 16)) return BSFP8_ERR_INVALID_ARG;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > kI32Max) return BSFP8_ERR_INVALID_ARG;
    const uint8_t* a8 = static_cast<const uint8_t*>(a);
    const uint8_t* b8 = static_cast<const uint8_t*>(b);
    // the MXFP4 kernels address a 32-row band of an operand (the skinny
    // kernel's tile) with 32-bit byte offsets: 32 K / 2 < 2^31
    if (path == 2 && K >= (int64_t(1) << 26)) return BSFP8_ERR_UNSUPPORTED;
    if (path == 2)
        return from_hip(bsfp8::launch_gemm_mxfp4(M, N, K, a8, static_cast<const uint8_t*>(a_scales), b8,
                                                 static_cast<const uint8_t*>(b_scales), out, d, ldd, ep,
                                                 stream));
    if (!aligned(a_scales, 4) || !aligned(b_scales, 4)) return BSFP8_ERR_INVALID_ARG;
    const float* sa = static_cast<const float*>(a_scales);
    const float* sb = static_cast<const float*>(b_scales);
    // the per-tile kernel addresses a 128-row band of an operand with 32-bit offsets
    if (path == 0 && K >= (int64_t(1) << 24)) return BSFP8_ERR_UNSUPPORTED;
    if (path == 0)
        return from_hip(bsfp8::launch_gemm_fp8(M, N, K, a_fmt, a8, sa, b_fmt, b8, sb, out, d, ldd, ep,
                                               stream, tensor_mask));
    // the K-constant kernel addresses a 256-row band of an operand with 32-bit offsets
    if (K >= (int64_t(1) << 23)) return BSFP8_ERR_UNSUPPORTED;
    return from_hip(bsfp8::launch_gemm_fp8_outer(M, N, K, a_fmt, a8, sa, a_g == BSFP8_GRAN_ROW ? 1 : 0,
                                                 b_fmt, b8, sb, b_g == BSFP8_GRAN_ROW ? 1 : 0, out, d,
                                                 ldd, ep, stream));
}

bsfp8_status scaled_gemm_mx(int64_t M, int64_t N, int64_t K, int block, bsfp8_mx_scale sfmt,
                            const void* a, const void* a_scales, const void* b,
                            const void* b_scales, float alpha, const void* c, int64_t ldc,
                            float beta, bsfp8_out out, void* d, int64_t ldd, hipStream_t stream) {
    if (block != 32 && block != 16 && block != 8) return BSFP8_ERR_UNSUPPORTED;
    if (sfmt != BSFP8_MX_E8M0 && sfmt != BSFP8_MX_F16 && sfmt != BSFP8_MX_BF16)
        return BSFP8_ERR_UNSUPPORTED;
    if (out != BSFP8_OUT_F32 && out != BSFP8_OUT_BF16 && out != BSFP8_OUT_F16)
        return BSFP8_ERR_UNSUPPORTED;
    if (block == 32 && sfmt == BSFP8_MX_E8M0)   // the hardware-scaled MXFP4 GEMM
        return scaled_gemm_granular(M, N, K, BSFP8_MXFP4, a, a_scales, BSFP8_GRAN_MX32, BSFP8_MXFP4,
                                    b, b_scales, BSFP8_GRAN_MX32, alpha, c, ldc, beta, out, d, ldd,
                                    stream);
    if (M < 0 || N < 0 || K < 0 || (K % 32) != 0) return BSFP8_ERR_INVALID_ARG;
    if (M > kI32Max || N > kI32Max || K > kI32Max) return BSFP8_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BSFP8_OK;
    const uintptr_t es = out == BSFP8_OUT_F32 ? 4 : 2;
    if (!d || ldd < N || !aligned(d, es)) return BSFP8_ERR_INVALID_ARG;
    if (beta != 0.0f && (!c || ldc < N || !aligned(c, es))) return BSFP8_ERR_INVALID_ARG;
    const bsfp8::Epilogue ep{alpha, beta, beta != 0.0f ? c : nullptr, beta != 0.0f ? ldc : 0};
    if (K == 0) return from_hip(bsfp8::launch_fill(M, N, out, d, ldd, ep, stream));
    if (!a || !b || !a_scales || !b_scales) return BSFP8_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16)) return BSFP8_ERR_INVALID_ARG;
    // the kernels address a 256-row band of an operand with 32-bit offsets
    if (K >= (int64_t(1) << 23)) return BSFP8_ERR_UNSUPPORTED;
    // a thread reads its block scales of a stage in one load of up to 8 bytes
    if (!aligned(a_scales, 8) || !aligned(b_scales, 8)) return BSFP8_ERR_INVALID_ARG;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > kI32Max) return BSFP8_ERR_INVALID_ARG;
    return from_hip(bsfp8::launch_gemm_mx(M, N, K, block, sfmt, static_cast<const uint8_t*>(a), a_scales,
                                          static_cast<const uint8_t*>(b), b_scales, out, d, ldd, ep,
                                          stream));
}

bsfp8_status scaled_gemm_quantize_a(int64_t M, int64_t N, int64_t K, const float* x, int64_t ldx,
                                    bsfp8_format a_fmt, bsfp8_format b_fmt, const void* b,
                                    const void* b_scales, bsfp8_granularity b_g, float alpha,
                                    const void* c, int64_t ldc, float beta, bsfp8_out out, void* d,
                                    int64_t ldd, uint8_t* a_codes, float* a_scales,
                                    hipStream_t stream) {
    if (!is_fp8(a_fmt) || !is_fp8(b_fmt)) return BSFP8_ERR_UNSUPPORTED;
    if (b_g != BSFP8_GRAN_TILE && b_g != BSFP8_GRAN_TENSOR) return BSFP8_ERR_UNSUPPORTED;
    if (out != BSFP8_OUT_F32 && out != BSFP8_OUT_BF16 && out != BSFP8_OUT_F16)
        return BSFP8_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K < 0 || (K % 32) != 0 || ldx < K) return BSFP8_ERR_INVALID_ARG;
    if (M > kI32Max || N > kI32Max || K > kI32Max) return BSFP8_ERR_INVALID_ARG;
    if ((a_codes == nullptr) != (a_scales == nullptr)) return BSFP8_ERR_INVALID_ARG;
    if (a_codes && (!aligned(a_codes, 4) || !aligned(a_scales, 4))) return BSFP8_ERR_INVALID_ARG;
    if (M == 0) return BSFP8_OK;
    if (K > 0) {
        if (!x || !aligned(x, 16) || (ldx % 4) != 0) return BSFP8_ERR_INVALID_ARG;
        // the kernel addresses a 128-row band of x with 32-bit byte offsets
        if (ldx >= (int64_t(1) << 22)) return BSFP8_ERR_UNSUPPORTED;
    }
    if (N == 0) {
        // no output tile carries the quantisation: the codes come from the quantiser itself
        if (a_codes && K > 0)
            return from_hip(bsfp8::launch_fp8_quantize(x, M, K, ldx, a_fmt, a_codes, a_scales, stream));
        return BSFP8_OK;
    }
    const uintptr_t es = out == BSFP8_OUT_F32 ? 4 : 2;
    if (!d || ldd < N || !aligned(d, es)) return BSFP8_ERR_INVALID_ARG;
    if (beta != 0.0f && (!c || ldc < N || !aligned(c, es))) return BSFP8_ERR_INVALID_ARG;
    const bsfp8::Epilogue ep{alpha, beta, beta != 0.0f ? c : nullptr, beta != 0.0f ? ldc : 0};
    if (K == 0) return from_hip(bsfp8::launch_fill(M, N, out, d, ldd, ep, stream));
    if (!b || !b_scales || !aligned(b, 16) || !aligned(b_scales, 4)) return BSFP8_ERR_INVALID_ARG;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > kI32Max) return BSFP8_ERR_INVALID_ARG;
    const uint8_t* b8 = static_cast<const uint8_t*>(b);
    const float* sb = static_cast<const float*>(b_scales);
    if (a_codes && tiles / ((M + 127) / 128) >= kOnlineMaxColumnTiles) {
        // A wide output re-quantises every A tile once per column of output
        // tiles; with somewhere to put the codes it is cheaper to quantise
        // once and run the per-tile GEMM on them (the same codes and the same
        // accumulation, so the same D).
        const hipError_t e = bsfp8::launch_fp8_quantize(x, M, K, ldx, a_fmt, a_codes, a_scales, stream);
        if (e != hipSuccess) return BSFP8_ERR_HIP;
        return from_hip(bsfp8::launch_gemm_fp8(M, N, K, a_fmt, a_codes, a_scales, b_fmt, b8, sb, out, d,
                                               ldd, ep, stream, b_g == BSFP8_GRAN_TENSOR ? 2 : 0));
    }
    const bsfp8::OnlineA qa{x, ldx, a_codes, a_scales};
    return from_hip(bsfp8::launch_gemm_fp8_online_a(M, N, K, a_fmt, qa, b_fmt,
                                                    b8, sb, b_g == BSFP8_GRAN_TENSOR ? 1 : 0, out, d, ldd,
                                                    ep, stream));
}

bsfp8_status scaled_gemm_ex(int64_t M, int64_t N, int64_t K, bsfp8_format a_fmt, const void* a,
                            const void* a_scales, bsfp8_format b_fmt, const void* b,
                            const void* b_scales, float alpha, const void* c, int64_t ldc,
                            float beta, bsfp8_out out, void* d, int64_t ldd,
                            hipStream_t stream) {
    const bsfp8_granularity g = a_fmt == BSFP8_MXFP4 ? BSFP8_GRAN_MX32 : BSFP8_GRAN_TILE;
    const bsfp8_granularity gb = b_fmt == BSFP8_MXFP4 ? BSFP8_GRAN_MX32 : BSFP8_GRAN_TILE;
    return scaled_gemm_granular(M, N, K, a_fmt, a, a_scales, g, b_fmt, b, b_scales, gb, alpha, c,
                                ldc, beta, out, d, ldd, stream);
}

bsfp8_status scaled_gemm(int64_t M, int64_t N, int64_t K, bsfp8_format a_fmt, const void* a,
                         const void* a_scales, bsfp8_format b_fmt, const void* b,
                         const void* b_scales, bsfp8_out out, void* d, int64_t ldd,
                         hipStream_t stream) {
    return scaled_gemm_ex(M, N, K, a_fmt, a, a_scales, b_fmt, b, b_scales, 1.0f, nullptr, 0,
                          0.0f, out, d, ldd, stream);
}

const char* bsfp8_status_string(bsfp8_status s) {
    switch (s) {
    case BSFP8_OK: return "BSFP8_OK";
    case BSFP8_ERR_INVALID_ARG: return "BSFP8_ERR_INVALID_ARG";
    case BSFP8_ERR_UNSUPPORTED: return "BSFP8_ERR_UNSUPPORTED";
    case BSFP8_ERR_HIP: return "BSFP8_ERR_HIP";
    default: return "BSFP8_ERR_UNKNOWN";
    }
}

int bsfp8_version(void) { return (0 << 16) | 5; }

}  // extern "C"
