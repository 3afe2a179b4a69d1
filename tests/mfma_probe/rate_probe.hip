// rate_probe.hip -- test instrument: sustained issue rate of the gfx950 matrix
// instructions the GEMMs use, and the shader clock while they run.
//
// Part of the test suite, not of the library.  It measures what bounds the
// per-tile FP8 GEMM ("Why grind FP8 GEMM on CDNA4", section 3.2: per-block
// promotion, and section 5.5: matrix-core utilisation as the first counter to
// read) independently of any GEMM's data movement: every operand lives in
// registers, so the only work is the matrix instructions themselves and, in the
// promotion pattern, the FP32 multiply-adds that apply one scale product per
// 32-wide K block.
//
// Each wave loads its operand registers once from `src` (9216 dwords: 64 lanes
// x 8 dwords of A, then of B, for the chains; then four such pairs, one per
// 32 x 32 tile, for the promotion pattern), runs `iters` iterations of a fixed pattern, and
// records the shader-clock counter (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) around the loop.  Their ratio is the shader clock
// while the pattern ran.  Operand values are the caller's (random codes or
// zeros), so the power draw of real data can be compared with that of zeros.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Instruction selector (the `instr` argument).  FLOPs per instruction in
// rate_flops() below.
enum RateInstr {
    kR_Fp8K16 = 0,     // v_mfma_f32_32x32x16_fp8_fp8         (K = 16, one 32-wide block = 2 instructions)
    kR_ScaleFp8 = 1,   // v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 with unit E8M0 scales (K = 64, two blocks)
    kR_ScaleFp4 = 2,   // v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 with unit E8M0 scales
    kR_Bf16K16 = 3,    // v_mfma_f32_32x32x16_bf16
    kR_Fp8K32x16 = 4,  // v_mfma_f32_16x16x32_fp8_fp8          (16 x 16 tile, K = 32: one block)
    kR_NumInstr = 5
};

// Pattern selector (the `pattern` argument).
enum RatePattern {
    kP_Chains = 0,     // four independent accumulator chains: the bare instruction rate
    kP_Promote = 1,    // the per-tile GEMM's inner block: per 32-wide K block and per
                       // 32 x 32 tile, a fresh accumulator P (two K = 16 instructions,
                       // or one 16 x 16 x 32 per 16 x 16 quarter), then
                       // acc = fma(sigma, P, acc) for each of its elements
    kP_Interleave = 2, // the same work software-pipelined: each tile's FMAs are issued
                       // between the next tile's instructions, one instruction then 8
                       // FMAs (16 x 16 x 32: one then 4), so that the matrix core and
                       // the VALU of one wave work at the same time
    kP_NumPattern = 3
};

__device__ __forceinline__ v16f mfma32(int instr, const uint32_t (&a)[8], const uint32_t (&b)[8], v16f c) {
    if (instr == kR_Fp8K16) {
        const long x = static_cast<long>(a[0] | (static_cast<uint64_t>(a[1]) << 32));
        const long y = static_cast<long>(b[0] | (static_cast<uint64_t>(b[1]) << 32));
        return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(x, y, c, 0, 0, 0);
    }
    if (instr == kR_Bf16K16) {
        v8bf x, y;
        __builtin_memcpy(&x, a, 16);
        __builtin_memcpy(&y, b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
    }
    v8i x, y;
    __builtin_memcpy(&x, a, 32);
    __builtin_memcpy(&y, b, 32);
    if (instr == kR_ScaleFp4)
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 4, 4, 0, 127, 0, 127);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ v4f mfma16(const uint32_t (&a)[8], const uint32_t (&b)[8], int off, v4f c) {
    const long x = static_cast<long>(a[off] | (static_cast<uint64_t>(a[off + 1]) << 32));
    const long y = static_cast<long>(b[off] | (static_cast<uint64_t>(b[off + 1]) << 32));
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(x, y, c, 0, 0, 0);
}

// Opaque to the optimiser: the values do not change, but the compiler may not
// assume so, which keeps loop-invariant products inside the loop.
template <int N>
__device__ __forceinline__ void opaque(uint32_t (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

template <int INSTR, int PATTERN>
__global__ __launch_bounds__(256) void rate_kernel(int iters, float sigma, const uint32_t* __restrict__ src,
                                                   uint64_t* __restrict__ times, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = static_cast<int>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
    uint32_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = src[lane * 8 + i];
        b[i] = src[512 + lane * 8 + i];
    }
    float total = 0.0f;
    uint64_t t0, r0, t1, r1;
    if constexpr (PATTERN == kP_Chains) {
        v16f c0 = v16f{}, c1 = v16f{}, c2 = v16f{}, c3 = v16f{};
        v4f e0 = v4f{}, e1 = v4f{}, e2 = v4f{}, e3 = v4f{};
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
        for (int it = 0; it < iters; ++it) {
            if constexpr (INSTR == kR_Fp8K32x16) {
                e0 = mfma16(a, b, 0, e0); e1 = mfma16(a, b, 2, e1);
                e2 = mfma16(a, b, 4, e2); e3 = mfma16(a, b, 6, e3);
            } else {
                c0 = mfma32(INSTR, a, b, c0); c1 = mfma32(INSTR, a, b, c1);
                c2 = mfma32(INSTR, a, b, c2); c3 = mfma32(INSTR, a, b, c3);
            }
        }
        if constexpr (INSTR == kR_Fp8K32x16) asm volatile("" : "+v"(e0), "+v"(e1), "+v"(e2), "+v"(e3));
        else asm volatile("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
        t1 = __builtin_amdgcn_s_memtime();
        r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
        for (int r = 0; r < 16; ++r) total += c0[r] + c1[r] + c2[r] + c3[r];
#pragma unroll
        for (int r = 0; r < 4; ++r) total += e0[r] + e1[r] + e2[r] + e3[r];
    } else if constexpr (PATTERN == kP_Interleave) {
        v16f acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = v16f{};
        uint32_t xs[4][8], ys[4][8];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xs[t][i] = src[1024 + 2048 * t + lane * 8 + i];
                ys[t][i] = src[1024 + 2048 * t + 512 + lane * 8 + i];
            }
        // a tile's product in a fresh accumulator (the same instructions as
        // the promotion pattern)
        auto product = [&](int t) {
            opaque(xs[t]);
            opaque(ys[t]);
            v16f p;
            if constexpr (INSTR == kR_Fp8K32x16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v4f e = mfma16(xs[t], ys[t], 2 * q, v4f{});
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[4 * q + r] = e[r];
                }
            } else if constexpr (INSTR == kR_Fp8K16 || INSTR == kR_Bf16K16) {
                p = mfma32(INSTR, xs[t], ys[t], v16f{});
                p = mfma32(INSTR, ys[t], xs[t], p);
            } else {
                p = mfma32(INSTR, xs[t], ys[t], v16f{});
            }
            return p;
        };
        constexpr int kInstr = INSTR == kR_Fp8K32x16 ? 4 : (INSTR == kR_Fp8K16 || INSTR == kR_Bf16K16) ? 2 : 1;
        constexpr int kFmaPer = 16 / kInstr;
        v16f prev = product(3);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
        for (int it = 0; it < iters; ++it) {
            // tile t's instructions, then the FMAs of the tile before it
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const v16f p = product(t);
                v16f& a = acc[(t + 3) & 3];
#pragma unroll
                for (int r = 0; r < 16; ++r) a[r] = __builtin_fmaf(sigma, prev[r], a[r]);
                prev = p;
#pragma unroll
                for (int g = 0; g < kInstr; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // one matrix instruction
                    __builtin_amdgcn_sched_group_barrier(0x002, kFmaPer, 0);   // then its share of FMAs
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[3][r] = __builtin_fmaf(sigma, prev[r], acc[3][r]);
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
        t1 = __builtin_amdgcn_s_memtime();
        r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) total += acc[t][r];
    } else {
        // four 32 x 32 tiles, as one wave of the per-tile GEMM (64 x 64) holds
        v16f acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = v16f{};
        // every tile has operand registers of its own, loaded once, so that no
        // two tiles' products can be merged
        uint32_t xs[4][8], ys[4][8];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xs[t][i] = src[1024 + 2048 * t + lane * 8 + i];
                ys[t][i] = src[1024 + 2048 * t + 512 + lane * 8 + i];
            }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t (&x)[8] = xs[t];
                uint32_t (&y)[8] = ys[t];
                opaque(x);
                opaque(y);
                v16f p;
                if constexpr (INSTR == kR_Fp8K32x16) {
                    // a 32 x 32 tile as four 16 x 16 quarters, one instruction each
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4f e = mfma16(x, y, 2 * q, v4f{});
#pragma unroll
                        for (int r = 0; r < 4; ++r) p[4 * q + r] = e[r];
                    }
                } else if constexpr (INSTR == kR_Fp8K16 || INSTR == kR_Bf16K16) {
                    // one 32-wide block = two K = 16 instructions into a fresh accumulator
                    p = mfma32(INSTR, x, y, v16f{});
                    p = mfma32(INSTR, y, x, p);
                } else {
                    // one K = 64 instruction (two blocks; not exact per block, rate only)
                    p = mfma32(INSTR, x, y, v16f{});
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] = __builtin_fmaf(sigma, p[r], acc[t][r]);
            }
        }
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
        t1 = __builtin_amdgcn_s_memtime();
        r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) total += acc[t][r];
    }
    sink[static_cast<int64_t>(wave) * 64 + lane] = total;
    if (lane == 0) {
        times[2 * static_cast<int64_t>(wave)] = t1 - t0;
        times[2 * static_cast<int64_t>(wave) + 1] = r1 - r0;
    }
}

template <int PATTERN>
hipError_t launch_pattern(int instr, int nwg, int iters, float sigma, const uint32_t* src, uint64_t* times,
                          float* sink, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(nwg)), block(256);
    switch (instr) {
    case kR_Fp8K16: hipLaunchKernelGGL((rate_kernel<kR_Fp8K16, PATTERN>), grid, block, 0, stream, iters, sigma, src, times, sink); break;
    case kR_ScaleFp8: hipLaunchKernelGGL((rate_kernel<kR_ScaleFp8, PATTERN>), grid, block, 0, stream, iters, sigma, src, times, sink); break;
    case kR_ScaleFp4: hipLaunchKernelGGL((rate_kernel<kR_ScaleFp4, PATTERN>), grid, block, 0, stream, iters, sigma, src, times, sink); break;
    case kR_Bf16K16: hipLaunchKernelGGL((rate_kernel<kR_Bf16K16, PATTERN>), grid, block, 0, stream, iters, sigma, src, times, sink); break;
    default: hipLaunchKernelGGL((rate_kernel<kR_Fp8K32x16, PATTERN>), grid, block, 0, stream, iters, sigma, src, times, sink); break;
    }
    return hipGetLastError();
}

}  // namespace

extern "C" {

// FLOPs of the matrix work one wave does per loop iteration of (instr, pattern)
// (2 x multiply-adds of the instructions issued; the promotion FMAs are not
// counted), or 0 for an unknown selector.
double mfma_rate_flops_per_iter(int instr, int pattern) {
    if (instr < 0 || instr >= kR_NumInstr || pattern < 0 || pattern >= kP_NumPattern) return 0.0;
    const double k16 = 2.0 * 32 * 32 * 16, k64 = 2.0 * 32 * 32 * 64, q = 2.0 * 16 * 16 * 32;
    const bool is64 = instr == kR_ScaleFp8 || instr == kR_ScaleFp4;
    if (pattern == kP_Chains) return 4.0 * (instr == kR_Fp8K32x16 ? q : is64 ? k64 : k16);
    // promotion patterns, four tiles per iteration: two K = 16 instructions,
    // four 16 x 16 x 32, or one K = 64
    return 4.0 * (instr == kR_Fp8K32x16 ? 4.0 * q : is64 ? k64 : 2.0 * k16);
}

// Launch `nwg` workgroups of four waves; each wave runs `iters` iterations of
// (instr, pattern) on the operands in src (device, 9216 dwords: lane l's A
// registers at 8 l .. 8 l + 7, its B registers at 512 + 8 l ..., then for the
// promotion pattern tile t's at 1024 + 2048 t + 8 l and 1024 + 2048 t + 512 + 8 l).  times
// (device, 2 uint64 per wave) receives the shader-clock cycles and the 100 MHz
// real-time ticks of each wave's loop; sink (device, 64 floats per wave)
// receives each lane's accumulator sum.  Returns 0 on success, 1 for a bad
// argument, 2 for a launch error.
int mfma_rate_launch(int instr, int pattern, int nwg, int iters, float sigma, const uint32_t* src,
                     uint64_t* times, float* sink, hipStream_t stream) {
    if (instr < 0 || instr >= kR_NumInstr || pattern < 0 || pattern >= kP_NumPattern) return 1;
    if (nwg <= 0 || nwg > (1 << 20) || iters < 0 || !src || !times || !sink) return 1;
    const hipError_t e =
        pattern == kP_Chains    ? launch_pattern<kP_Chains>(instr, nwg, iters, sigma, src, times, sink, stream)
        : pattern == kP_Promote ? launch_pattern<kP_Promote>(instr, nwg, iters, sigma, src, times, sink, stream)
                                : launch_pattern<kP_Interleave>(instr, nwg, iters, sigma, src, times, sink, stream);
    return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
