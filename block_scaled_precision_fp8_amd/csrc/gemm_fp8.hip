// gemm_fp8.hip -- per-tile-scaled FP8 GEMM for gfx950 (CDNA4).
//
// D[m][n] = sum over 32-wide K blocks kb of  sa(m/128, kb) * sb(n/128, kb) * P_kb[m][n],
// P_kb = sum_{k in kb} qa[m][k] * qb[n][k]   (codes times codes, FP32).
//
// The scale product differs from one K block to the next ("Why grind FP8 GEMM
// on CDNA4", section 3.3 scales every 128 x 32 tile; "Rubin FP4 GEMM deep
// dive", section 2.2 applies each K block's scale product to that block's
// partial sum before accumulation).  Every K block's partial sum P_kb is
// therefore computed in a fresh MFMA accumulator and promoted into the FP32
// result with one VALU FMA per element, acc = fma(sigma_kb, P_kb, acc)
// (section 3.2 of the CDNA4 article alternates two accumulator groups; here
// the MFMA temporaries and the resident accumulators play those roles).
//
// Two operand paths, chosen by output type:
//  * bf16 output: v_mfma_f32_32x32x16_{fp8,bf8}_{fp8,bf8} on the codes.  These
//    instructions keep 13 bits below the largest product of a sum and truncate
//    the rest (the behaviour "FP8 MMA internals on Hopper" models for H100,
//    measured on gfx950), i.e. at most 2^-8 of sum |a b| per block: inside the
//    2^-7 bf16 tolerance.
//  * FP32 output: codes are widened exactly to bf16 while staged into LDS
//    (every E4M3/E5M2 value is a normal bf16) and multiplied with
//    v_mfma_f32_32x32x16_bf16, which keeps 24 alignment bits: inside 2^-19.
//
// Tiling: 128 x 128 output tile per workgroup (one A scale tile by one B scale
// tile, so sigma_kb is uniform across the workgroup), 4 waves of 64 x 64, each
// made of 2 x 2 MFMA 32 x 32 tiles.  A and B tiles are staged through LDS in
// two buffers of 128 rows x 128 bytes (+16 bytes of padding per row, which
// makes the 16-byte fragment reads of 8 consecutive rows cover all banks).
// The MFMA's row operand is B and its column operand is A, so each lane ends
// up holding 4 consecutive output columns: the epilogue writes 16-byte (FP32)
// or 8-byte (bf16) vectors.
#include "internal.h"

#include <utility>

namespace bsfp8 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int kRowBytes = 128;                // data bytes per LDS row per stage
constexpr int kStride = kRowBytes + 16;       // padded LDS row stride
constexpr int kOperandBytes = 128 * kStride;  // one operand tile
constexpr int kStageBytes = 2 * kOperandBytes;
constexpr int kLdsBytes = 2 * kStageBytes;    // double buffered: 73728 bytes

__device__ __forceinline__ uint64_t lo64(uint4 v) {
    return static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32);
}
__device__ __forceinline__ uint64_t hi64(uint4 v) {
    return static_cast<uint64_t>(v.z) | (static_cast<uint64_t>(v.w) << 32);
}

// src0 holds B codes (format BF), src1 holds A codes (format AF).
template <int AF, int BF>
__device__ __forceinline__ v16f mfma_codes(uint64_t x, uint64_t y, v16f c) {
    const long a = static_cast<long>(x), b = static_cast<long>(y);
    if constexpr (BF == BSFP8_E4M3 && AF == BSFP8_E4M3)
        return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
    else if constexpr (BF == BSFP8_E4M3 && AF == BSFP8_E5M2)
        return __builtin_amdgcn_mfma_f32_32x32x16_fp8_bf8(a, b, c, 0, 0, 0);
    else if constexpr (BF == BSFP8_E5M2 && AF == BSFP8_E4M3)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf8_fp8(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf8_bf8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_bf16(uint4 x, uint4 y, v16f c) {
    v8bf a, b;
    __builtin_memcpy(&a, &x, 16);
    __builtin_memcpy(&b, &y, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Four FP8 codes (one dword) -> four bf16 (two dwords), exactly: the hardware
// FP8 -> FP32 conversion is exact and an FP8 value's FP32 image has 16 zero
// low bits, so its upper half is the bf16 encoding of the same value.
template <int FMT>
__device__ __forceinline__ uint2 widen4(uint32_t w) {
    float f0, f1, f2, f3;
    if constexpr (FMT == BSFP8_E4M3) {
        auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
        auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
        f0 = lo[0]; f1 = lo[1]; f2 = hi[0]; f3 = hi[1];
    } else {
        auto lo = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), false);
        auto hi = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), true);
        f0 = lo[0]; f1 = lo[1]; f2 = hi[0]; f3 = hi[1];
    }
    uint2 r;
    r.x = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    r.y = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    return r;
}

template <int FMT>
__device__ __forceinline__ void widen16(uint4 v, uint4& lo, uint4& hi) {
    const uint2 a = widen4<FMT>(v.x), b = widen4<FMT>(v.y);
    const uint2 c = widen4<FMT>(v.z), d = widen4<FMT>(v.w);
    lo = make_uint4(a.x, a.y, b.x, b.y);
    hi = make_uint4(c.x, c.y, d.x, d.y);
}

template <int AF, int BF, int OUT, bool WIDE>
__global__ __launch_bounds__(kThreads, 2) void gemm_fp8_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sA,
    const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, int tiles_m, int tiles_n, int vec_ok) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

    constexpr int KPS = WIDE ? 64 : 128;     // K elements per stage (128 LDS bytes per row)
    constexpr int KBS = KPS / 32;            // K blocks per stage
    constexpr int CPR = KPS / 16;            // 16-byte global chunks per row per stage
    constexpr int RSTEP = kThreads / CPR;    // rows between one thread's chunks
    constexpr int NLD = 128 / RSTEP;         // chunks per thread per operand per stage

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;

    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int nkb = K >> 5;
    const int nst = (nkb + KBS - 1) / KBS;

    // Global -> register staging: thread `tid` moves chunk (tid % CPR) of rows
    // (tid / CPR) + RSTEP * i.  Rows past the matrix edge re-read the last row;
    // their results are never stored.
    const int crow = tid / CPR;
    const int cch = tid % CPR;
    const uint8_t* ga[NLD];
    const uint8_t* gb[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int ra = min(m0 + crow + RSTEP * i, M - 1);
        const int rb = min(n0 + crow + RSTEP * i, N - 1);
        ga[i] = A + static_cast<int64_t>(ra) * K + cch * 16;
        gb[i] = B + static_cast<int64_t>(rb) * K + cch * 16;
    }
    uint4 sa_reg[NLD], sb_reg[NLD];

    auto gload = [&](int s) {
        const int k0 = s * KPS;
        const bool ok = k0 + cch * 16 < K;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            sa_reg[i] = ok ? *reinterpret_cast<const uint4*>(ga[i] + k0) : make_uint4(0, 0, 0, 0);
            sb_reg[i] = ok ? *reinterpret_cast<const uint4*>(gb[i] + k0) : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* la = lds + buf * kStageBytes;
        uint8_t* lb = la + kOperandBytes;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int row = crow + RSTEP * i;
            if constexpr (!WIDE) {
                *reinterpret_cast<uint4*>(la + row * kStride + cch * 16) = sa_reg[i];
                *reinterpret_cast<uint4*>(lb + row * kStride + cch * 16) = sb_reg[i];
            } else {
                uint4 lo, hi;
                widen16<AF>(sa_reg[i], lo, hi);
                *reinterpret_cast<uint4*>(la + row * kStride + cch * 32) = lo;
                *reinterpret_cast<uint4*>(la + row * kStride + cch * 32 + 16) = hi;
                widen16<BF>(sb_reg[i], lo, hi);
                *reinterpret_cast<uint4*>(lb + row * kStride + cch * 32) = lo;
                *reinterpret_cast<uint4*>(lb + row * kStride + cch * 32 + 16) = hi;
            }
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

    const int frag_row = lane & 31;
    const int half = lane >> 5;
    const float* sa_row = sA + static_cast<int64_t>(tm) * nkb;
    const float* sb_row = sB + static_cast<int64_t>(tn) * nkb;

    auto compute_kb = [&](const uint8_t* la, const uint8_t* lb, int kb, int gkb) {
        const float sigma = sa_row[gkb] * sb_row[gkb];
        uint4 x0[2], x1[2], y0[2], y1[2];
        if constexpr (!WIDE) {
            // lane half h reads bytes 16h..16h+15 of the block: instruction 0 takes
            // the first 8, instruction 1 the next 8 (same mapping for A and B).
            const int off = kb * 32 + 16 * half;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                x0[t] = *reinterpret_cast<const uint4*>(lb + (wn * 64 + 32 * t + frag_row) * kStride + off);
                y0[t] = *reinterpret_cast<const uint4*>(la + (wm * 64 + 32 * t + frag_row) * kStride + off);
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
                    v16f p = v16f{};
                    p = mfma_codes<AF, BF>(lo64(x0[ti]), lo64(y0[tj]), p);
                    p = mfma_codes<AF, BF>(hi64(x0[ti]), hi64(y0[tj]), p);
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[ti][tj][r] = fmaf(sigma, p[r], acc[ti][tj][r]);
                }
        } else {
            // bf16: lane half h reads elements 16h..16h+15 (32 bytes) of the block.
            const int off = kb * 64 + 32 * half;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint8_t* px = lb + (wn * 64 + 32 * t + frag_row) * kStride + off;
                const uint8_t* py = la + (wm * 64 + 32 * t + frag_row) * kStride + off;
                x0[t] = *reinterpret_cast<const uint4*>(px);
                x1[t] = *reinterpret_cast<const uint4*>(px + 16);
                y0[t] = *reinterpret_cast<const uint4*>(py);
                y1[t] = *reinterpret_cast<const uint4*>(py + 16);
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
                    v16f p = v16f{};
                    p = mfma_bf16(x0[ti], y0[tj], p);
                    p = mfma_bf16(x1[ti], y1[tj], p);
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[ti][tj][r] = fmaf(sigma, p[r], acc[ti][tj][r]);
                }
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        if (s + 1 < nst) gload(s + 1);
        const uint8_t* la = lds + (s & 1) * kStageBytes;
        const uint8_t* lb = la + kOperandBytes;
        const int kb0 = s * KBS;
        if (kb0 + KBS <= nkb) {
#pragma unroll
            for (int kb = 0; kb < KBS; ++kb) compute_kb(la, lb, kb, kb0 + kb);
        } else {
            for (int kb = 0; kb < nkb - kb0; ++kb) compute_kb(la, lb, kb, kb0 + kb);
        }
        if (s + 1 < nst) lstore((s + 1) & 1);
        __syncthreads();
    }

    // Epilogue.  acc[ti][tj][r] is output row m = m0 + 64 wm + 32 tj + (lane % 32)
    // and column n = n0 + 64 wn + 32 ti + 8 (r / 4) + 4 (lane / 32) + r % 4.
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) {
            const int m = m0 + wm * 64 + tj * 32 + frag_row;
            if (m >= M) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 64 + ti * 32 + q * 8 + half * 4;
                const float v0 = acc[ti][tj][4 * q + 0], v1 = acc[ti][tj][4 * q + 1];
                const float v2 = acc[ti][tj][4 * q + 2], v3 = acc[ti][tj][4 * q + 3];
                if constexpr (OUT == BSFP8_OUT_F32) {
                    float* dp = static_cast<float*>(D) + static_cast<int64_t>(m) * ldd + n;
                    if (vec_ok && n + 3 < N) {
                        *reinterpret_cast<float4*>(dp) = make_float4(v0, v1, v2, v3);
                    } else {
                        if (n + 0 < N) dp[0] = v0;
                        if (n + 1 < N) dp[1] = v1;
                        if (n + 2 < N) dp[2] = v2;
                        if (n + 3 < N) dp[3] = v3;
                    }
                } else {
                    uint16_t* dp = static_cast<uint16_t*>(D) + static_cast<int64_t>(m) * ldd + n;
                    const uint32_t b0 = f32_to_bf16_rne(v0), b1 = f32_to_bf16_rne(v1);
                    const uint32_t b2 = f32_to_bf16_rne(v2), b3 = f32_to_bf16_rne(v3);
                    if (vec_ok && n + 3 < N) {
                        *reinterpret_cast<uint2*>(dp) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
                    } else {
                        if (n + 0 < N) dp[0] = static_cast<uint16_t>(b0);
                        if (n + 1 < N) dp[1] = static_cast<uint16_t>(b1);
                        if (n + 2 < N) dp[2] = static_cast<uint16_t>(b2);
                        if (n + 3 < N) dp[3] = static_cast<uint16_t>(b3);
                    }
                }
            }
        }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_byte;
typedef __attribute__((address_space(3))) void lds_void;

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <int OFF>
__device__ __forceinline__ void lds_read16(u32x4& v, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LDS: per buffer, A then B, 128 rows x 128 bytes each, unpadded (filled by
// direct global-to-LDS loads); row R keeps 16-byte chunk g at g ^ ((R >> 1) & 7).
constexpr int kDRow = 128;
constexpr int kDOperand = 128 * kDRow;      // 16 KB
constexpr int kDStage = 2 * kDOperand;      // 32 KB
constexpr int kDLds = 2 * kDStage;          // 64 KB: two workgroups per CU

template <int AF, int BF>
__global__ __launch_bounds__(kThreads, 2) void gemm_fp8_bf16_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sA,
    const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, int tiles_m, int tiles_n, int vec_ok) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kDLds];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;
    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int nkb = K >> 5;
    const int nst = (nkb + 3) >> 2;          // 128 K per stage
    const int last = nst - 1;

    // direct loads: instruction i (0..3) of wave w fills rows 32 i + 8 w .. + 7
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A), 0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B), 0, N * K, 0x00020000);
    const int drow = 8 * wave + (lane >> 3);
    const int dchunk = (lane & 7) ^ ((drow >> 1) & 7);
    const uint32_t dma_a = static_cast<uint32_t>(m0 + drow) * K + dchunk * 16;
    const uint32_t dma_b = static_cast<uint32_t>(n0 + drow) * K + dchunk * 16;
    const uint32_t row_step = 32u * static_cast<uint32_t>(K);
    auto dma_one = [&](auto J, int stage, int buf) {
        constexpr int j = J;
        constexpr int i = j >> 1;
        const int so = min(stage, last) * 128;
        if constexpr ((j & 1) == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs_a, (lds_void*)(lds + buf * kDStage + (32 * i + 8 * wave) * kDRow), 16,
                dma_a + i * row_step, so, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs_b, (lds_void*)(lds + buf * kDStage + kDOperand + (32 * i + 8 * wave) * kDRow), 16,
                dma_b + i * row_step, so, 0, 0);
    };

    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    const int sw = (frag_row >> 1) & 7;
    // read base per buffer and block: chunk 2 kb + half of rows wm*64 + 32 t + r
    uint32_t rd_a[2][4], rd_b[2][4];
#pragma unroll
    for (int bf = 0; bf < 2; ++bf)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const uint32_t pos = static_cast<uint32_t>(((2 * kb + half) ^ sw) * 16);
            rd_a[bf][kb] = lds0 + bf * kDStage + (wm * 64 + frag_row) * kDRow + pos;
            rd_b[bf][kb] = lds0 + bf * kDStage + kDOperand + (wn * 64 + frag_row) * kDRow + pos;
        }

    // scales of a stage: 4 floats of A's tile row and 4 of B's, loaded one stage ahead
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(sA), 0, static_cast<int>(tiles_m) * nkb * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(sB), 0, static_cast<int>(tiles_n) * nkb * 4, 0x00020000);
    const uint32_t so_a = static_cast<uint32_t>(tm) * nkb * 4;
    const uint32_t so_b = static_cast<uint32_t>(tn) * nkb * 4;
    u32x4 nsa, nsb;
    auto load_scales = [&](int stage) {
        const int so = min(stage, last) * 16;
        asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(nsa) : "v"(so_a), "s"(rs_sa), "s"(so) : "memory");
        asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(nsb) : "v"(so_b), "s"(rs_sb), "s"(so) : "memory");
    };

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
    u32x4 fx[2][2], fy[2][2];    // [set][t]

    static_for<8>([&](auto J) { dma_one(J, 0, 0); });
    load_scales(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    static_for<2>([&](auto t) {
        lds_read16<t * 32 * kDRow>(fx[0][t], rd_b[0][0]);
        lds_read16<t * 32 * kDRow>(fy[0][t], rd_a[0][0]);
    });
    static_for<8>([&](auto J) { dma_one(J, 1, 1); });

    // full stages run unconditionally; a partial last stage (K not a multiple
    // of 128) is finished by the tail below
    const int nfull = nkb >> 2;
    for (int s = 0; s < nfull; ++s) {
        const int cb = s & 1;
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // this stage's scales
        u32x4 ca = nsa, cbv = nsb;
        asm volatile("" : "+v"(ca), "+v"(cbv));
        float sig[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) sig[k] = __uint_as_float(ca[k]) * __uint_as_float(cbv[k]);
        load_scales(s + 1);

        auto block = [&](auto KB) {
            constexpr int kb = KB;
            constexpr int nkb_ = (kb + 1) & 3;
            const int rb = kb == 3 ? cb ^ 1 : cb;
            u32x4 (&f)[2] = fx[kb & 1];
            u32x4 (&g)[2] = fy[kb & 1];
            if constexpr (kb == 3) {
                asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            } else {
                lds_wait();
            }
            // prefetch the next block's fragments
            static_for<2>([&](auto t) {
                lds_read16<t * 32 * kDRow>(fx[(kb + 1) & 1][t], rb ? rd_b[1][nkb_] : rd_b[0][nkb_]);
                lds_read16<t * 32 * kDRow>(fy[(kb + 1) & 1][t], rb ? rd_a[1][nkb_] : rd_a[0][nkb_]);
            });
            if constexpr (kb == 3) static_for<8>([&](auto J) { dma_one(J, s + 2, cb); });
            // the MFMAs below may only start after the prefetch is issued
            asm volatile("" : "+v"(f[0]), "+v"(f[1]), "+v"(g[0]), "+v"(g[1]));
            {
                const float sigma = sig[kb];
#pragma unroll
                for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                    for (int tj = 0; tj < 2; ++tj) {
                        const uint64_t xl = static_cast<uint64_t>(f[ti][0]) | (static_cast<uint64_t>(f[ti][1]) << 32);
                        const uint64_t xh = static_cast<uint64_t>(f[ti][2]) | (static_cast<uint64_t>(f[ti][3]) << 32);
                        const uint64_t yl = static_cast<uint64_t>(g[tj][0]) | (static_cast<uint64_t>(g[tj][1]) << 32);
                        const uint64_t yh = static_cast<uint64_t>(g[tj][2]) | (static_cast<uint64_t>(g[tj][3]) << 32);
                        v16f p = v16f{};
                        p = mfma_codes<AF, BF>(xl, yl, p);
                        p = mfma_codes<AF, BF>(xh, yh, p);
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[ti][tj][r] = fmaf(sigma, p[r], acc[ti][tj][r]);
                    }
            }
            // close the block: its promotions finish before the next block's reads
            asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]));
        };
        block(std::integral_constant<int, 0>{});
        block(std::integral_constant<int, 1>{});
        block(std::integral_constant<int, 2>{});
        block(std::integral_constant<int, 3>{});
    }
    if (nfull < nst) {
        // partial stage: its data and block-0 fragments are already in place
        const int cb = nfull & 1;
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        u32x4 ca = nsa, cbv = nsb;
        asm volatile("" : "+v"(ca), "+v"(cbv));
        const int nk = nkb - 4 * nfull;
        for (int kb = 0; kb < nk; ++kb) {
            lds_wait();
            u32x4 x[2], y[2];
            if (kb == 0) {
                x[0] = fx[0][0]; x[1] = fx[0][1]; y[0] = fy[0][0]; y[1] = fy[0][1];
            } else {
                const uint32_t ra = (cb ? rd_a[1][0] : rd_a[0][0]) + ((((2 * kb + half) ^ sw) - (half ^ sw)) * 16);
                const uint32_t rb = (cb ? rd_b[1][0] : rd_b[0][0]) + ((((2 * kb + half) ^ sw) - (half ^ sw)) * 16);
                lds_read16<0>(x[0], rb);
                lds_read16<32 * kDRow>(x[1], rb);
                lds_read16<0>(y[0], ra);
                lds_read16<32 * kDRow>(y[1], ra);
                lds_wait();
            }
            // the MFMAs consume the fragments only after the wait above
            asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(y[0]), "+v"(y[1]));
            const float sigma = __uint_as_float(ca[kb]) * __uint_as_float(cbv[kb]);
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
                    const uint64_t xl = static_cast<uint64_t>(x[ti][0]) | (static_cast<uint64_t>(x[ti][1]) << 32);
                    const uint64_t xh = static_cast<uint64_t>(x[ti][2]) | (static_cast<uint64_t>(x[ti][3]) << 32);
                    const uint64_t yl = static_cast<uint64_t>(y[tj][0]) | (static_cast<uint64_t>(y[tj][1]) << 32);
                    const uint64_t yh = static_cast<uint64_t>(y[tj][2]) | (static_cast<uint64_t>(y[tj][3]) << 32);
                    v16f p = v16f{};
                    p = mfma_codes<AF, BF>(xl, yl, p);
                    p = mfma_codes<AF, BF>(xh, yh, p);
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[ti][tj][r] = fmaf(sigma, p[r], acc[ti][tj][r]);
                }
        }
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    // Epilogue through LDS (free now): 128 rows x 256 bytes of bf16; 16-byte
    // chunk c of row R sits at c ^ (R & 15).  Each 64-lane store then covers
    // 4 whole rows instead of 32 rows x 16 bytes.
    __syncthreads();
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int R = wm * 64 + tj * 32 + frag_row;
                const int c = wn * 8 + ti * 4 + q;
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                const bf16x4 v = {(__bf16)acc[ti][tj][4 * q + 0], (__bf16)acc[ti][tj][4 * q + 1],
                                  (__bf16)acc[ti][tj][4 * q + 2], (__bf16)acc[ti][tj][4 * q + 3]};
                *reinterpret_cast<bf16x4*>(lds + R * 256 + ((c ^ (R & 15)) << 4) + 8 * half) = v;
            }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int R = wave * 32 + i * 4 + (lane >> 4);
        const int c = lane & 15;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + R * 256 + ((c ^ (R & 15)) << 4));
        const int m = m0 + R, n = n0 + c * 8;
        if (m >= M) continue;
        uint16_t* dp = static_cast<uint16_t*>(D) + static_cast<int64_t>(m) * ldd + n;
        if (vec_ok && n + 8 <= N) {
            *reinterpret_cast<uint4*>(dp) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (n + j < N) dp[j] = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
        }
    }
}

template <int AF, int BF>
hipError_t launch_typed(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                        const uint8_t* b, const float* sb, int out, void* d, int64_t ldd,
                        hipStream_t stream) {
    const int tiles_m = static_cast<int>((M + BM - 1) / BM);
    const int tiles_n = static_cast<int>((N + BN - 1) / BN);
    const dim3 grid(static_cast<uint32_t>(tiles_m) * static_cast<uint32_t>(tiles_n));
    const int align = out == BSFP8_OUT_F32 ? 16 : 8;
    const int vec_ok = (ldd % 4 == 0) && (reinterpret_cast<uintptr_t>(d) % align == 0);
    if (out == BSFP8_OUT_F32)
        hipLaunchKernelGGL((gemm_fp8_kernel<AF, BF, BSFP8_OUT_F32, true>), grid, dim3(kThreads), 0,
                           stream, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K),
                           a, sa, b, sb, d, ldd, tiles_m, tiles_n, vec_ok);
    else
        hipLaunchKernelGGL((gemm_fp8_bf16_kernel<AF, BF>), grid, dim3(kThreads),
                           0, stream, static_cast<int>(M), static_cast<int>(N),
                           static_cast<int>(K), a, sa, b, sb, d, ldd, tiles_m, tiles_n,
                           static_cast<int>((ldd % 8 == 0) && (reinterpret_cast<uintptr_t>(d) % 16 == 0)));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                           const float* a_scales, int b_fmt, const uint8_t* b,
                           const float* b_scales, int out, void* d, int64_t ldd,
                           hipStream_t stream) {
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E4M3)
        return launch_typed<BSFP8_E4M3, BSFP8_E4M3>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, stream);
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E5M2)
        return launch_typed<BSFP8_E4M3, BSFP8_E5M2>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, stream);
    if (a_fmt == BSFP8_E5M2 && b_fmt == BSFP8_E4M3)
        return launch_typed<BSFP8_E5M2, BSFP8_E4M3>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, stream);
    return launch_typed<BSFP8_E5M2, BSFP8_E5M2>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, stream);
}

}  // namespace bsfp8
