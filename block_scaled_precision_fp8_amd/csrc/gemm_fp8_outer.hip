// gemm_fp8_outer.hip -- FP8 GEMM with scales that are constant along K (gfx950).
//
// With per-row scales on A, per-column scales on B or one scale per tensor
// ("Why grind FP8 GEMM on CDNA4", section 3.3 weighs these granularities), the
// scale product of output (m, n) is the same for every K block:
//     D[m][n] = sA[m] sB[n] sum_k qA[m][k] qB[n][k],
// so the whole K sum stays in the matrix core and the scales multiply once, at
// write-back, as an outer product.  Without the per-32-K promotion that
// per-tile scales need, the kernel can use v_mfma_f32_32x32x64_f8f6f4, whose
// FP8 rate is about 1.75 times that of the K = 16 FP8 instructions (16-bit
// outputs).  FP32 output needs more than that instruction's 13 fraction bits
// per group of 8 products: there the codes are widened to bf16 and multiplied
// by v_mfma_f32_32x32x16_bf16, as in the per-tile kernel.
//
// Tiling: 256 x 256 output tile per workgroup, 4 waves of 128 x 128 (4 x 4
// MFMA 32 x 32 tiles, 256 FP32 accumulators per lane in the accumulation
// registers), one workgroup per CU.  K advances in stages of 64: a stage is 256
// rows x 64 bytes of A and of B (32 KB), brought by direct global-to-LDS loads
// into one of four LDS buffers three stages before it is used.  Row R keeps its
// 16-byte chunk g at position g ^ ((R >> 2) & 3), so the 16 lanes of a fragment
// read phase (16 consecutive rows, one chunk) hit 16 distinct bank groups.
// Operand fragments: for the K = 64 instruction with 8-bit elements, lane
// (row r, half h) supplies K values 16 h .. 16 h + 15 in registers 0-3 and
// 32 + 16 h .. 32 + 16 h + 15 in registers 4-7 (measured with the test probe).
// The main loop is volatile inline assembly, as in the MXFP4 kernel, so that
// loads, fragment reads and MFMAs interleave in program order.
#include "big_tile.h"

namespace bsfp8 {

namespace {

using namespace big_tile;
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 256;
constexpr int kRowBytes = 64;                        // one stage of K per row
constexpr int kOperandBytes = 256 * kRowBytes;       // 16 KB
constexpr int kStageBytes = 2 * kOperandBytes;       // 32 KB
constexpr int kBuffers = 4;
constexpr int kLdsBytes = kBuffers * kStageBytes;    // 128 KB
// after the stage buffers: the tile's 256 row scales of A, then its 256
// column scales of B (2 KB), staged once at the start so that the epilogue
// reads them from LDS instead of waiting on global loads per row tile
constexpr int kScaleLds = kLdsBytes;
constexpr int kLdsTotal = kLdsBytes + 2 * 256 * 4;
// stages loaded before the first wait; the rest of the first four follow it,
// so that stage 0's loads do not queue behind three more stages' worth
#ifndef BSFP8_OUTER_PROLOGUE_STAGES
#define BSFP8_OUTER_PROLOGUE_STAGES 2
#endif
constexpr int kPrologueStages = BSFP8_OUTER_PROLOGUE_STAGES;

template <int FMT>
constexpr int mfma_fmt() { return FMT == BSFP8_E4M3 ? 0 : 1; }

// acc += x^T y for one 32 x 32 x 64 step; x is the row operand (format CB), y
// the column operand (format BG).
template <int CB, int BG>
__device__ __forceinline__ void mfma_fp8_k64(v16f& acc, const u32x8& x, const u32x8& y) {
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0 cbsz:%3 blgp:%4"
                 : "+a"(acc)
                 : "v"(x), "v"(y), "i"(CB), "i"(BG));
}

// The epilogue's per-element scale: sA of the element's row times sB of its
// column (step 0 broadcasts one scale per tensor); zero outside the matrix.
// The tile's scales are in LDS (ss: 256 of A, then 256 of B, tile-relative).
// Row-operand tile ti covers tile columns b_base + 32 ti + 8 q + e (q, e < 4)
// of this lane; its 16 column scales are read when the epilogue reaches ti.
struct OuterScale {
    const float* ss;
    int b_base;
    float sa[4], sb[16];
    __device__ OuterScale(const float* s, int a_base, int bb) : ss(s), b_base(bb) {
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) sa[tj] = ss[a_base + 32 * tj];
    }
    __device__ void load(int ti) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sb[r] = ss[256 + b_base + 32 * ti + 8 * (r >> 2) + (r & 3)];
    }
    __device__ float operator()(int, int tj, int r, float v) const { return (sa[tj] * sb[r]) * v; }
};

// Eight FP8 codes (two dwords) -> eight bf16 (four dwords), exactly: every
// E4M3 and E5M2 value is a normal bf16.
template <int FMT>
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 a, b, c, d;
    if constexpr (FMT == BSFP8_E4M3) {
        a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
        c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
        d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    } else {
        a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, 1.0f, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, 1.0f, true);
        c = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, 1.0f, false);
        d = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, 1.0f, true);
    }
    return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                 __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
}

// acc += x^T y for one 32 x 32 x 16 bf16 step.
__device__ __forceinline__ void mfma_bf16_k16(v16f& acc, const u32x4& x, const u32x4& y) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
}

template <int AF, int BF, int OUT, bool STAGE16>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_outer_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sA, int sa_step,
    const uint8_t* __restrict__ B, const float* __restrict__ sB, int sb_step, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsTotal];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;

    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
    const int m0 = tm * 256;
    const int n0 = tn * 256;
    const int nst = (K + 63) >> 6;

    // Buffer resources start at the tile's first row and end after its last
    // row inside the matrix, so rows past the edge read as zero and every
    // range-checked offset stays below 256 K < 2^31.
    const int rows_a = min(256, M - m0);
    const int rows_b = min(256, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A) + static_cast<int64_t>(m0) * K, 0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B) + static_cast<int64_t>(n0) * K, 0, rows_b * K, 0x00020000);

    // Direct loads: load j (0..7) of wave w fills rows 16 g .. 16 g + 15 of
    // operand j & 1 (A, B) with g = 4 (j >> 1) + w; lane l takes row
    // 16 g + l / 4 and the global chunk that belongs at position l % 4.  A chunk
    // past the end of K is given an out-of-range offset (it reads as zero).
    const int drow = lane >> 2;
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    // Stages at or past the end of K (the padding of the last group of four)
    // read as zero throughout.
    const uint32_t dma_row = static_cast<uint32_t>((16 * wave + drow) * K + dchunk * 16);
    const uint32_t dma_grp = static_cast<uint32_t>(64 * K);       // 4 row groups further
    auto dma_one = [&](auto J, int stage, auto BUF) {
        constexpr int j = J;
        constexpr int buf = BUF;
        constexpr int gi = j >> 1;           // row group 4 gi + wave
        const bool in_k = stage * 64 + dchunk * 16 < K;
        const uint32_t vo = in_k ? dma_row + gi * dma_grp : 0x80000000u;
        lds_void* dst = (lds_void*)(lds + buf * kStageBytes + (j & 1) * kOperandBytes + (4 * gi + wave) * 1024);
        if constexpr ((j & 1) == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, dst, 16, vo, stage * 64, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, dst, 16, vo, stage * 64, 0, 0);
    };

    // Fragment reads: lane (frag_row r, half h) reads chunks h (registers 0-3)
    // and 2 + h (registers 4-7) of rows wm 128 + 32 t + r (A) and wn 128 + 32 t +
    // r (B).  Buffers 0 and 1 are addressed from base set 0, 2 and 3 from set 1;
    // (buffer & 1) and t are immediate offsets.
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    const int sw = (frag_row >> 2) & 3;
    const uint32_t lo = static_cast<uint32_t>((half ^ sw) * 16);
    const uint32_t hi = static_cast<uint32_t>(((2 + half) ^ sw) * 16);
    uint32_t ra_lo[2], ra_hi[2], rb_lo[2], rb_hi[2];
#pragma unroll
    for (int set = 0; set < 2; ++set) {
        const uint32_t base = lds0 + set * 2 * kStageBytes;
        ra_lo[set] = base + (wm * 128 + frag_row) * kRowBytes + lo;
        ra_hi[set] = base + (wm * 128 + frag_row) * kRowBytes + hi;
        rb_lo[set] = base + kOperandBytes + (wn * 128 + frag_row) * kRowBytes + lo;
        rb_hi[set] = base + kOperandBytes + (wn * 128 + frag_row) * kRowBytes + hi;
    }

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    struct Frag { u32x4 xl[4], xh[4], yl[4], yh[4]; };
    Frag fr[2];
    // read piece R (0..15) of the fragments of the stage held in buffer BUF
    auto read_one = [&](auto R, Frag& dst, auto BUF) {
        constexpr int r = R;
        constexpr int buf = BUF;
        constexpr int t = r >> 2;
        constexpr int which = r & 3;
        constexpr int set = buf >> 1;
        constexpr int off = (buf & 1) * kStageBytes + t * 32 * kRowBytes;
        if constexpr (which == 0) lds_read16<off>(dst.xl[t], rb_lo[set]);
        if constexpr (which == 1) lds_read16<off>(dst.xh[t], rb_hi[set]);
        if constexpr (which == 2) lds_read16<off>(dst.yl[t], ra_lo[set]);
        if constexpr (which == 3) lds_read16<off>(dst.yh[t], ra_hi[set]);
    };

    constexpr int CB = mfma_fmt<BF>();    // the row operand is B
    constexpr int BG = mfma_fmt<AF>();

    // The tile's scales: thread t loads A row m0 + t and B column n0 + t
    // (indices past the edge clamped, the value then replaced by zero); they
    // are stored to LDS below, once the stage loads are on their way.
    const float sc_a = sA[static_cast<int64_t>(min(m0 + tid, M - 1)) * sa_step];
    const float sc_b = sB[static_cast<int64_t>(min(n0 + tid, N - 1)) * sb_step];
    // Prologue: stages 0-3 on their way into buffers 0-3 (the first
    // kPrologueStages before the wait for stage 0, the others after it);
    // stage 0's fragments into registers once it has landed.
    static_for<kPrologueStages>([&](auto S) { static_for<8>([&](auto J) { dma_one(J, S, S); }); });
    {
        float* ss = reinterpret_cast<float*>(lds + kScaleLds);
        ss[tid] = m0 + tid < M ? sc_a : 0.0f;
        ss[256 + tid] = n0 + tid < N ? sc_b : 0.0f;
    }
    asm volatile("s_waitcnt vmcnt(%0)" :: "i"(8 * (kPrologueStages - 1)) : "memory");
    static_for<4 - kPrologueStages>([&](auto S) {
        constexpr auto st = std::integral_constant<int, kPrologueStages + S>{};
        static_for<8>([&](auto J) { dma_one(J, st, st); });
    });
    lds_wait_barrier();
    static_for<16>([&](auto R) { read_one(R, fr[0], std::integral_constant<int, 0>{}); });

    // Stage s lives in buffer s % 4 and its fragments in set s % 2; the loop
    // runs whole groups of four stages so that both are compile-time.
    const int ngroups = (nst + 3) >> 2;
    for (int gi = 0; gi < ngroups; ++gi) {
        static_for<4>([&](auto U) {
            constexpr int u = U;
            const int s = 4 * gi + u;
            // stage s + 1 has landed once only the loads of stages s + 2 and
            // s + 3 are outstanding; the barrier publishes it, and it also
            // means every wave has finished reading buffer u (stage s's
            // fragments are in registers), which stage s + 4 then refills
            asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
            lds_wait_barrier();
            const Frag& f = fr[u & 1];
            Frag& g = fr[(u + 1) & 1];
            constexpr auto nbuf = std::integral_constant<int, (u + 1) & 3>{};
            if constexpr (OUT != BSFP8_OUT_F32) {
                static_for<16>([&](auto J) {
                    constexpr int j = J;
                    constexpr int ti = j >> 2, tj = j & 3;
                    const u32x8 x = __builtin_shufflevector(f.xl[ti], f.xh[ti], 0, 1, 2, 3, 4, 5, 6, 7);
                    const u32x8 y = __builtin_shufflevector(f.yl[tj], f.yh[tj], 0, 1, 2, 3, 4, 5, 6, 7);
                    mfma_fp8_k64<CB, BG>(acc[ti][tj], x, y);
                    read_one(J, g, nbuf);
                    if constexpr ((j & 1) == 0) dma_one(std::integral_constant<int, j / 2>{}, s + 4, U);
                });
            } else {
                // FP32 output: the FP8 instructions keep 13 fraction bits per
                // group of 8 products, too few for FP32 accuracy; the codes are
                // widened exactly to bf16 and multiplied by the bf16 instruction
                // (24 fraction bits).  Each lane's 32 codes of a step form four
                // groups of 8 (K positions in the same order on both operands,
                // so every product still pairs equal K).
                static_for<4>([&](auto I) {
                    constexpr int i = I;
                    u32x4 xw[4], yw[4];
                    static_for<4>([&](auto T) {
                        constexpr int t = T;
                        const u32x4& xs = i < 2 ? f.xl[t] : f.xh[t];
                        const u32x4& ys = i < 2 ? f.yl[t] : f.yh[t];
                        xw[t] = widen8<BF>(xs[2 * (i & 1)], xs[2 * (i & 1) + 1]);
                        yw[t] = widen8<AF>(ys[2 * (i & 1)], ys[2 * (i & 1) + 1]);
                    });
                    // the conversions' results must settle before the MFMAs read them
                    asm volatile("s_nop 4"
                                 : "+v"(xw[0]), "+v"(xw[1]), "+v"(xw[2]), "+v"(xw[3]),
                                   "+v"(yw[0]), "+v"(yw[1]), "+v"(yw[2]), "+v"(yw[3]));
                    static_for<16>([&](auto J) {
                        constexpr int j = J;
                        constexpr int ti = j >> 2, tj = j & 3;
                        constexpr int n = 16 * i + j;       // 0..63 in the step
                        mfma_bf16_k16(acc[ti][tj], xw[ti], yw[tj]);
                        if constexpr (n % 4 == 0) read_one(std::integral_constant<int, n / 4>{}, g, nbuf);
                        if constexpr (n % 8 == 0) dma_one(std::integral_constant<int, n / 8>{}, s + 4, U);
                    });
                });
            }
        });
    }
    // no direct load may still be writing LDS when the epilogue reuses it, and
    // the last step's fragment reads, which have no consumer, are named after
    // the wait so that their registers are not reused while in flight
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        asm volatile("" :: "v"(fr[q].xl[0]), "v"(fr[q].xl[1]), "v"(fr[q].xl[2]), "v"(fr[q].xl[3]),
                           "v"(fr[q].xh[0]), "v"(fr[q].xh[1]), "v"(fr[q].xh[2]), "v"(fr[q].xh[3]));
        asm volatile("" :: "v"(fr[q].yl[0]), "v"(fr[q].yl[1]), "v"(fr[q].yl[2]), "v"(fr[q].yl[3]),
                           "v"(fr[q].yh[0]), "v"(fr[q].yh[1]), "v"(fr[q].yh[2]), "v"(fr[q].yh[3]));
    }
    // MFMA results must settle before the accumulation registers are read.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                   "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]),
                   "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                   "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));

    OuterScale sc(reinterpret_cast<const float*>(lds + kScaleLds), wm * 128 + frag_row, wn * 128 + 4 * half);
    epilogue<OUT, STAGE16>(acc, lds, wave, lane, m0, n0, M, N, D, ldd, ep, vec_ok, sc);
}

template <int AF, int BF, int OUT>
hipError_t launch_out(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa, int sa_step,
                      const uint8_t* b, const float* sb, int sb_step, void* d, int64_t ldd,
                      const Epilogue& ep, hipStream_t stream) {
    const int vec = vec16_ok(OUT, d, ldd, ep);
    const int tm = static_cast<int>((M + 255) / 256), tn = static_cast<int>((N + 255) / 256);
    const dim3 grid(static_cast<uint32_t>(tm) * static_cast<uint32_t>(tn));
    if constexpr (OUT != BSFP8_OUT_F32) {
        if (ep.beta == 0.0f) {
            hipLaunchKernelGGL((gemm_fp8_outer_kernel<AF, BF, OUT, true>), grid, dim3(kThreads), 0, stream,
                               static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, sa, sa_step,
                               b, sb, sb_step, d, ldd, ep, tm, tn, vec);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_fp8_outer_kernel<AF, BF, OUT, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, sa, sa_step,
                       b, sb, sb_step, d, ldd, ep, tm, tn, vec);
    return hipGetLastError();
}

template <int AF, int BF>
hipError_t launch_typed(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa, int sa_step,
                        const uint8_t* b, const float* sb, int sb_step, int out, void* d, int64_t ldd,
                        const Epilogue& ep, hipStream_t stream) {
    if (out == BSFP8_OUT_F32)
        return launch_out<AF, BF, BSFP8_OUT_F32>(M, N, K, a, sa, sa_step, b, sb, sb_step, d, ldd, ep, stream);
    if (out == BSFP8_OUT_BF16)
        return launch_out<AF, BF, BSFP8_OUT_BF16>(M, N, K, a, sa, sa_step, b, sb, sb_step, d, ldd, ep, stream);
    return launch_out<AF, BF, BSFP8_OUT_F16>(M, N, K, a, sa, sa_step, b, sb, sb_step, d, ldd, ep, stream);
}

}  // namespace

hipError_t launch_gemm_fp8_outer(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                                 const float* a_scales, int a_step, int b_fmt, const uint8_t* b,
                                 const float* b_scales, int b_step, int out, void* d, int64_t ldd,
                                 const Epilogue& ep, hipStream_t stream) {
    // few rows: the skinny per-tile kernel streams B with far more workgroups
    if (skinny_outer_fits(M))
        return launch_gemm_fp8_skinny_outer(M, N, K, a_fmt, a, a_scales, a_step, b_fmt, b, b_scales, b_step,
                                            out, d, ldd, ep, stream);
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E4M3)
        return launch_typed<BSFP8_E4M3, BSFP8_E4M3>(M, N, K, a, a_scales, a_step, b, b_scales, b_step, out, d, ldd, ep, stream);
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E5M2)
        return launch_typed<BSFP8_E4M3, BSFP8_E5M2>(M, N, K, a, a_scales, a_step, b, b_scales, b_step, out, d, ldd, ep, stream);
    if (a_fmt == BSFP8_E5M2 && b_fmt == BSFP8_E4M3)
        return launch_typed<BSFP8_E5M2, BSFP8_E4M3>(M, N, K, a, a_scales, a_step, b, b_scales, b_step, out, d, ldd, ep, stream);
    return launch_typed<BSFP8_E5M2, BSFP8_E5M2>(M, N, K, a, a_scales, a_step, b, b_scales, b_step, out, d, ldd, ep, stream);
}

}  // namespace bsfp8
