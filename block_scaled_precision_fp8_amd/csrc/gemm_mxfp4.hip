// gemm_mxfp4.hip -- MXFP4 GEMM for gfx950 (CDNA4).
//
// D[m][n] = sum_kb 2^(ea[m][kb] + eb[n][kb]) * sum_{k in kb} e2m1_a[m][k] * e2m1_b[n][k]
// ("Rubin FP4 GEMM deep dive", sections 2.2 and 3.1: 32-element K blocks, each
// with its own E8M0 scale on both operands, scales applied to the block sums).
// The power-of-two block scales are applied inside the matrix core by
// v_mfma_scale_f32_32x32x64_f8f6f4 (format E2M1 on both sides): lane l of an
// operand supplies 32 consecutive K values (16 packed bytes) of row l % 32 for
// K block l / 32 of the instruction, together with that row's E8M0 byte for
// the same block.  No per-block VALU work is needed, so the FP32 accumulators
// stay in the matrix core's registers for the whole K loop.
//
// Tiling as for the FP8 kernel: 128 x 128 output tile per workgroup, 4 waves of
// 64 x 64 (2 x 2 MFMA tiles), A and B staged through padded LDS rows of 128
// bytes (256 K values) in two buffers; B is the MFMA row operand so each lane
// holds 4 consecutive output columns for vector stores.
#include "internal.h"

namespace bsfp8 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int kStride = 128 + 16;
constexpr int kOperandBytes = 128 * kStride;
constexpr int kStageBytes = 2 * kOperandBytes;
constexpr int kLdsBytes = 2 * kStageBytes;
constexpr int KPS = 256;        // K elements per stage (128 packed bytes per row)
// The 256 x 256 kernel is used once it has at least this many tiles.
constexpr int64_t kBigTileThreshold = 64;

__device__ __forceinline__ v16f mfma_fp4(uint4 x, uint4 y, uint32_t sx, uint32_t sy, v16f c) {
    v8i a = {static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z),
             static_cast<int>(x.w), 0, 0, 0, 0};
    v8i b = {static_cast<int>(y.x), static_cast<int>(y.y), static_cast<int>(y.z),
             static_cast<int>(y.w), 0, 0, 0, 0};
    // format 4 = E2M1 for both operands; scale byte 0 of each scale register.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0,
                                                           static_cast<int>(sx), 0,
                                                           static_cast<int>(sy));
}

// Store four consecutive output columns n..n+3 of row m (masked at the right edge).
template <int OUT>
__device__ __forceinline__ void store4(void* D, int64_t ldd, int m, int n, int N, int vec_ok,
                                       float v0, float v1, float v2, float v3) {
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

template <int OUT>
__global__ __launch_bounds__(kThreads, 2) void gemm_mxfp4_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, int tiles_m, int tiles_n, int vec_ok) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;

    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int kbytes = K >> 1;       // packed bytes per row
    const int nkb = K >> 5;          // scale blocks per row
    const int nst = (K + KPS - 1) / KPS;

    // staging: 128 rows x 128 bytes per operand = 1024 chunks, 4 per thread
    const int crow = tid >> 3;
    const int cch = tid & 7;
    const uint8_t* ga[4];
    const uint8_t* gb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = min(m0 + crow + 32 * i, M - 1);
        const int rb = min(n0 + crow + 32 * i, N - 1);
        ga[i] = A + static_cast<int64_t>(ra) * kbytes + cch * 16;
        gb[i] = B + static_cast<int64_t>(rb) * kbytes + cch * 16;
    }
    uint4 ra_[4], rb_[4];
    auto gload = [&](int s) {
        const int b0 = s * (KPS / 2);
        const bool ok = b0 + cch * 16 < kbytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra_[i] = ok ? *reinterpret_cast<const uint4*>(ga[i] + b0) : make_uint4(0, 0, 0, 0);
            rb_[i] = ok ? *reinterpret_cast<const uint4*>(gb[i] + b0) : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* la = lds + buf * kStageBytes;
        uint8_t* lb = la + kOperandBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = crow + 32 * i;
            *reinterpret_cast<uint4*>(la + row * kStride + cch * 16) = ra_[i];
            *reinterpret_cast<uint4*>(lb + row * kStride + cch * 16) = rb_[i];
        }
    };

    const int frag_row = lane & 31;
    const int half = lane >> 5;
    // scale rows this lane reads: A rows (for the column operand) and B rows (row operand)
    const uint8_t* sa_p[2];
    const uint8_t* sb_p[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ra = min(m0 + wm * 64 + 32 * t + frag_row, M - 1);
        const int rb = min(n0 + wn * 64 + 32 * t + frag_row, N - 1);
        sa_p[t] = sA + static_cast<int64_t>(ra) * nkb;
        sb_p[t] = sB + static_cast<int64_t>(rb) * nkb;
    }

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

    // one K step = 64 K values = 32 packed bytes per row = 2 scale blocks
    auto compute_step = [&](const uint8_t* la, const uint8_t* lb, int ks, int gstep) {
        const int off = ks * 32 + 16 * half;
        const int blk = 2 * gstep + half;   // this lane's scale block
        uint4 x[2], y[2];
        uint32_t sx[2], sy[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            x[t] = *reinterpret_cast<const uint4*>(lb + (wn * 64 + 32 * t + frag_row) * kStride + off);
            y[t] = *reinterpret_cast<const uint4*>(la + (wm * 64 + 32 * t + frag_row) * kStride + off);
            sx[t] = sb_p[t][blk];
            sy[t] = sa_p[t][blk];
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int tj = 0; tj < 2; ++tj)
                acc[ti][tj] = mfma_fp4(x[ti], y[tj], sx[ti], sy[tj], acc[ti][tj]);
    };

    const int nsteps = K >> 6;   // K / 64 (K is a multiple of 32; an odd block count is handled below)
    const bool odd_block = (nkb & 1) != 0;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        if (s + 1 < nst) gload(s + 1);
        const uint8_t* la = lds + (s & 1) * kStageBytes;
        const uint8_t* lb = la + kOperandBytes;
        const int g0 = s * (KPS / 64);
        if (g0 + KPS / 64 <= nsteps) {
#pragma unroll
            for (int ks = 0; ks < KPS / 64; ++ks) compute_step(la, lb, ks, g0 + ks);
        } else {
            for (int ks = 0; ks < nsteps - g0; ++ks) compute_step(la, lb, ks, g0 + ks);
            if (odd_block) {
                // last 32-wide block: the upper lane half's K values are zero
                // (staged as zeros past the row end) and its scale byte must stay
                // finite, so it reuses block nkb - 1.
                const int ks = nsteps - g0;
                const int off = ks * 32 + 16 * half;
                uint4 x[2], y[2];
                uint32_t sx[2], sy[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    x[t] = *reinterpret_cast<const uint4*>(lb + (wn * 64 + 32 * t + frag_row) * kStride + off);
                    y[t] = *reinterpret_cast<const uint4*>(la + (wm * 64 + 32 * t + frag_row) * kStride + off);
                    if (half) { x[t] = make_uint4(0, 0, 0, 0); y[t] = make_uint4(0, 0, 0, 0); }
                    sx[t] = sb_p[t][nkb - 1];
                    sy[t] = sa_p[t][nkb - 1];
                }
#pragma unroll
                for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                    for (int tj = 0; tj < 2; ++tj)
                        acc[ti][tj] = mfma_fp4(x[ti], y[tj], sx[ti], sy[tj], acc[ti][tj]);
            }
        }
        if (s + 1 < nst) lstore((s + 1) & 1);
        __syncthreads();
    }

#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) {
            const int m = m0 + wm * 64 + tj * 32 + frag_row;
            if (m >= M) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 64 + ti * 32 + q * 8 + half * 4;
                store4<OUT>(D, ldd, m, n, N, vec_ok, acc[ti][tj][4 * q + 0], acc[ti][tj][4 * q + 1],
                            acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]);
            }
        }
}

// ---------------------------------------------------------------------------
// Large-tile variant for K a multiple of 256: 256 x 256 output tile, 4 waves of
// 128 x 128 (4 x 4 MFMA tiles, 256 FP32 accumulators per lane held in the
// accumulation registers), one workgroup per CU.  A K step of 64 reads 8
// fragments of 1 KB per wave for 16 MFMAs, half the LDS traffic per FLOP of
// the 128 x 128 tiling; the 256-wide edge halves the L2 traffic per FLOP.
// Codes and E8M0 scales arrive through buffer loads (rows past the matrix
// edge read as zero) one stage ahead of use.
// ---------------------------------------------------------------------------
constexpr int kBigOperandBytes = 256 * kStride;
constexpr int kBigStageBytes = 2 * kBigOperandBytes;
constexpr int kBigLdsBytes = 2 * kBigStageBytes;     // 147456 bytes

template <int OUT>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp4_big_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, int tiles_m, int tiles_n, int vec_ok) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kBigLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;

    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
    const int m0 = tm * 256;
    const int n0 = tn * 256;
    const int kbytes = K >> 1;
    const int nkb = K >> 5;
    const int nst = K >> 8;          // K is a multiple of 256

    // staging: 256 rows x 128 bytes per operand per stage, 8 chunks per thread
    const int crow = tid >> 3;
    const int cch = tid & 7;
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A), 0, M * kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B), 0, N * kbytes, 0x00020000);
    const int voff_a = (m0 + crow) * kbytes + cch * 16;
    const int voff_b = (n0 + crow) * kbytes + cch * 16;
    const int row_step = 32 * kbytes;
    uint4 ra[8], rb[8];

    // scales: the 4 A rows and 4 B rows this lane feeds to the MFMAs, 8 blocks per stage
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sA), 0, M * nkb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sB), 0, N * nkb, 0x00020000);
    // one lane offset per operand; the row step (32 rows) and stage step go in SGPRs
    const int soff_a = (m0 + wm * 128 + frag_row) * nkb;
    const int soff_b = (n0 + wn * 128 + frag_row) * nkb;
    const int srow_step = 32 * nkb;
    uint2 sca[4], scb[4], nsca[4], nscb[4];

    auto gload = [&](int s) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            auto va = __builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_a, s * 128 + i * row_step, 0);
            auto vb = __builtin_amdgcn_raw_buffer_load_b128(rs_b, voff_b, s * 128 + i * row_step, 0);
            __builtin_memcpy(&ra[i], &va, 16);
            __builtin_memcpy(&rb[i], &vb, 16);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            auto xa = __builtin_amdgcn_raw_buffer_load_b64(rs_sa, soff_a, s * 8 + t * srow_step, 0);
            auto xb = __builtin_amdgcn_raw_buffer_load_b64(rs_sb, soff_b, s * 8 + t * srow_step, 0);
            __builtin_memcpy(&nsca[t], &xa, 8);
            __builtin_memcpy(&nscb[t], &xb, 8);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* la = lds + buf * kBigStageBytes;
        uint8_t* lb = la + kBigOperandBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = crow + 32 * i;
            *reinterpret_cast<uint4*>(la + row * kStride + cch * 16) = ra[i];
            *reinterpret_cast<uint4*>(lb + row * kStride + cch * 16) = rb[i];
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    // byte (2 ks + half) of a stage's 8 scale bytes
    auto pick = [&](uint2 v, int ks) -> uint32_t {
        const uint32_t w = ks < 2 ? v.x : v.y;
        return (w >> (8 * (2 * (ks & 1) + half))) & 0xFFu;
    };

    gload(0);
    lstore(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) { sca[t] = nsca[t]; scb[t] = nscb[t]; }
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        if (s + 1 < nst) gload(s + 1);
        const uint8_t* la = lds + (s & 1) * kBigStageBytes;
        const uint8_t* lb = la + kBigOperandBytes;
        // fragments of K step ks + 1 are read while the MFMAs of step ks run
        struct Frag { uint4 x[4], y[4]; uint32_t sx[4], sy[4]; };
        auto load_frag = [&](Frag& f, int ks) {
            const int off = ks * 32 + 16 * half;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f.x[t] = *reinterpret_cast<const uint4*>(lb + (wn * 128 + 32 * t + frag_row) * kStride + off);
                f.y[t] = *reinterpret_cast<const uint4*>(la + (wm * 128 + 32 * t + frag_row) * kStride + off);
                f.sx[t] = pick(scb[t], ks);
                f.sy[t] = pick(sca[t], ks);
            }
        };
        Frag fr[2];
        load_frag(fr[0], 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) load_frag(fr[(ks + 1) & 1], ks + 1);
            if (ks == 3 && s + 1 < nst) {
                // The next stage's staged data goes to the other LDS buffer here:
                // after three K steps of MFMAs have covered the global-load latency
                // and before the last step's MFMAs.  MFMA builtins carry no memory
                // dependence, so the compiler would move these writes (and their
                // wait for the loads) above the MFMAs; the empty asm statements tie
                // the staged registers to every accumulator as left by the previous
                // steps, which pins the order.
                uint32_t key = 0;
                asm volatile(""
                             : "+v"(key)
                             : "a"(acc[0][0]), "a"(acc[0][1]), "a"(acc[0][2]), "a"(acc[0][3]),
                               "a"(acc[1][0]), "a"(acc[1][1]), "a"(acc[1][2]), "a"(acc[1][3]),
                               "a"(acc[2][0]), "a"(acc[2][1]), "a"(acc[2][2]), "a"(acc[2][3]),
                               "a"(acc[3][0]), "a"(acc[3][1]), "a"(acc[3][2]), "a"(acc[3][3]));
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    uint32_t ta = ra[i].x, tb = rb[i].x;
                    asm volatile("" : "+v"(ta), "+v"(tb) : "v"(key));
                    ra[i].x = ta;
                    rb[i].x = tb;
                }
                lstore((s + 1) & 1);
            }
            const Frag& f = fr[ks & 1];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int tj = 0; tj < 4; ++tj)
                    acc[ti][tj] = mfma_fp4(f.x[ti], f.y[tj], f.sx[ti], f.sy[tj], acc[ti][tj]);
            if (ks + 1 < 4) {
                // interleave the next step's 8 fragment reads with this step's 16 MFMAs
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
                }
            }
        }
        if (s + 1 < nst) {
#pragma unroll
            for (int t = 0; t < 4; ++t) { sca[t] = nsca[t]; scb[t] = nscb[t]; }
        }
        __syncthreads();
    }

#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            const int m = m0 + wm * 128 + tj * 32 + frag_row;
            if (m >= M) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 128 + ti * 32 + q * 8 + half * 4;
                store4<OUT>(D, ldd, m, n, N, vec_ok, acc[ti][tj][4 * q + 0], acc[ti][tj][4 * q + 1],
                            acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]);
            }
        }
}

}  // namespace

hipError_t launch_gemm_mxfp4(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                             const uint8_t* a_scales, const uint8_t* b, const uint8_t* b_scales,
                             int out, void* d, int64_t ldd, hipStream_t stream) {
    const int align = out == BSFP8_OUT_F32 ? 16 : 8;
    const int vec_ok = (ldd % 4 == 0) && (reinterpret_cast<uintptr_t>(d) % align == 0);
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    const bool fits32 = M * (K / 2) < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31);
    if (K % 256 == 0 && big_tiles >= kBigTileThreshold && fits32) {
        const int tm = static_cast<int>((M + 255) / 256), tn = static_cast<int>((N + 255) / 256);
        const dim3 g(static_cast<uint32_t>(tm) * static_cast<uint32_t>(tn));
        if (out == BSFP8_OUT_F32)
            hipLaunchKernelGGL(gemm_mxfp4_big_kernel<BSFP8_OUT_F32>, g, dim3(kThreads), 0, stream,
                               static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a,
                               a_scales, b, b_scales, d, ldd, tm, tn, vec_ok);
        else
            hipLaunchKernelGGL(gemm_mxfp4_big_kernel<BSFP8_OUT_BF16>, g, dim3(kThreads), 0, stream,
                               static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a,
                               a_scales, b, b_scales, d, ldd, tm, tn, vec_ok);
        return hipGetLastError();
    }
    const int tiles_m = static_cast<int>((M + BM - 1) / BM);
    const int tiles_n = static_cast<int>((N + BN - 1) / BN);
    const dim3 grid(static_cast<uint32_t>(tiles_m) * static_cast<uint32_t>(tiles_n));
    if (out == BSFP8_OUT_F32)
        hipLaunchKernelGGL(gemm_mxfp4_kernel<BSFP8_OUT_F32>, grid, dim3(kThreads), 0, stream,
                           static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a,
                           a_scales, b, b_scales, d, ldd, tiles_m, tiles_n, vec_ok);
    else
        hipLaunchKernelGGL(gemm_mxfp4_kernel<BSFP8_OUT_BF16>, grid, dim3(kThreads), 0, stream,
                           static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a,
                           a_scales, b, b_scales, d, ldd, tiles_m, tiles_n, vec_ok);
    return hipGetLastError();
}

}  // namespace bsfp8
