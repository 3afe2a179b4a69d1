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
//  * bf16 / FP16 output: v_mfma_f32_32x32x16_{fp8,bf8}_{fp8,bf8} on the codes.  These
//    instructions align each group of 8 products to 13 fraction bits below the
//    group's largest exponent sum and cut the rest toward zero (the behaviour
//    "FP8 MMA internals on Hopper" models for H100, measured on gfx950), i.e.
//    at most 7 * 2^-13 of sum |a b| per block: inside the 2^-7 tolerance of
//    the 16-bit outputs.
//  * FP32 output: each fragment is widened exactly to bf16 (every E4M3/E5M2
//    value is a normal bf16) right before v_mfma_f32_32x32x16_bf16, which keeps
//    24 fraction bits per group of 8: about 2^-20.4 of sum |a b| per block.
// Only these K = 16 instructions keep each 32-wide block's sum apart; the
// K = 64 F8F6F4 instructions would merge two blocks whose scale products are
// unrelated FP32 numbers.
//
// Tiling: 128 x 128 output tile per workgroup (one A scale tile by one B scale
// tile, so sigma_kb is uniform across the workgroup), 4 waves of 64 x 64, each
// made of 2 x 2 MFMA 32 x 32 tiles, two workgroups per CU.  The MFMA's row
// operand is B and its column operand is A, so each lane holds 4 consecutive
// output columns.
//
// Data movement:
//  * A and B are staged one stage (128 K = 4 blocks) ahead with direct
//    global-to-LDS loads, into unpadded 128-byte LDS rows; 16-byte chunk g of
//    row R is stored at position g ^ ((R >> 1) & 7), so the 16 lanes of a
//    fragment-read phase hit 16 distinct 4-bank groups.
//  * The fragments of block kb + 1 are read (ordered inline assembly) before
//    block kb's MFMAs, which are tied to the prefetch so the compiler cannot
//    hoist them above it.  The stage barrier sits before a stage's last block,
//    so the next stage's first fragments load under that block's MFMAs.
//  * The output tile leaves through LDS, so every store writes whole rows.
#include "fp8_codec.h"

#include <type_traits>
#include <utility>

namespace bsfp8 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;

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


// Eight FP8 codes (two dwords) -> eight bf16, exactly (every E4M3 and E5M2
// value is a normal bf16; unit scale).  A and B fragments go through the same
// mapping, so the K indices of the two operands still pair up.
template <int FMT>
__device__ __forceinline__ v8bf widen8(uint32_t w0, uint32_t w1) {
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
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
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

// Product of one 32 x 32 MFMA tile over one 32-wide K block.  Lane half h
// holds K values 16h .. 16h+15 of its row in x (B, format BF) and y (A,
// format AF); the first instruction takes the first 8, the second the next 8.
//  * bf16 / FP16 output: the FP8 codes go straight into the FP8 MFMA.
//  * FP32 output: the codes are widened exactly to bf16 and multiplied with the
//    bf16 MFMA, which keeps 24 fraction bits instead of 13.
template <int AF, int BF, int OUT>
__device__ __forceinline__ v16f tile_product(const u32x4& x, const u32x4& y) {
    v16f p = v16f{};
    if constexpr (OUT != BSFP8_OUT_F32) {
        const uint64_t xl = static_cast<uint64_t>(x[0]) | (static_cast<uint64_t>(x[1]) << 32);
        const uint64_t xh = static_cast<uint64_t>(x[2]) | (static_cast<uint64_t>(x[3]) << 32);
        const uint64_t yl = static_cast<uint64_t>(y[0]) | (static_cast<uint64_t>(y[1]) << 32);
        const uint64_t yh = static_cast<uint64_t>(y[2]) | (static_cast<uint64_t>(y[3]) << 32);
        p = mfma_codes<AF, BF>(xl, yl, p);
        p = mfma_codes<AF, BF>(xh, yh, p);
    } else {
        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen8<BF>(x[0], x[1]), widen8<AF>(y[0], y[1]), p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen8<BF>(x[2], x[3]), widen8<AF>(y[2], y[3]), p, 0, 0, 0);
    }
    return p;
}
// Half H of tile_product for 16-bit outputs: the instruction over K 16 H ..
// 16 H + 15 of the block, accumulating into p.
template <int AF, int BF, int H>
__device__ __forceinline__ v16f product_half(const u32x4& x, const u32x4& y, v16f p) {
    const uint64_t xv = static_cast<uint64_t>(x[2 * H]) | (static_cast<uint64_t>(x[2 * H + 1]) << 32);
    const uint64_t yv = static_cast<uint64_t>(y[2 * H]) | (static_cast<uint64_t>(y[2 * H + 1]) << 32);
    return mfma_codes<AF, BF>(xv, yv, p);
}
template <int H>
__device__ __forceinline__ void promote_half(v16f& a, float sg, const v16f& p) {
#pragma unroll
    for (int r = 8 * H; r < 8 * H + 8; ++r) a[r] = fmaf(sg, p[r], a[r]);
}

// QA: the A operand arrives in FP32 and is quantised inside the kernel on its
// way to LDS ("Why grind FP8 GEMM on CDNA4", section 4.2 converts and scales
// while loading; section 3.3 overlaps the online scale computation with the
// loads).  The workgroup then has 8 waves: waves 0-3 run the GEMM exactly as
// without QA (B still arrives by direct loads), waves 4-7 quantise A.  Each
// SIMD runs one GEMM wave and one quantiser wave, so the quantisation's VALU
// work interleaves with the other wave's MFMAs, and the GEMM waves keep their
// whole register budget.
//
// Quantiser thread q = tid - 256 (xc = q % 32, xr = q / 32) holds 16-byte chunk
// xc of the stage's 512-byte FP32 row segments of rows xr + 8 i, i = 0..15:
// each load instruction of a wave reads two whole row segments, and all 64
// values of a thread belong to the tile of K block xc / 8 (the quantiser's own
// layout).  Two register sets alternate.  Between the stage barriers s - 1 and
// s the quantiser waves
//   1. issue the loads of stage s + 2's values,
//   2. form stage s + 1's tile scales from the maxima published before barrier
//      s - 1, and store them in LDS for the GEMM waves,
//   3. encode stage s + 1's values into LDS buffer (s + 1) % 2 (free since
//      barrier s - 1; the GEMM waves read it after barrier s),
//   4. reduce the tile maxima of stage s + 2's values (lane shuffles, then one
//      value per wave in LDS), to be combined after barrier s.
// The codes are those of fp8_quantize; tn == 0 workgroups can also store them.
constexpr int kQThreads = 512;
// __syncthreads() calls in the epilogue, matched by the quantiser waves
constexpr int kEpilogueBarriers = 2;

template <int AF, int BF, int OUT, bool QA>
__global__ __launch_bounds__(QA ? kQThreads : kThreads, QA ? 1 : 2) void gemm_fp8_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sA,
    const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok, int tensor_mask, OnlineA qa) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kDLds];
    __shared__ float red[2][4][4];      // QA: [stage parity][quantiser wave][K block] tile maxima
    __shared__ float sa_lds[2][4];      // QA: [stage parity][K block] A tile scales
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
    const int nfull = nkb >> 2;              // full stages; a partial last stage follows

    if constexpr (QA) {
        if (wave >= 4) {
            const int q = tid - 256;
            const int cw = wave - 4;
            const int xc = q & 31;
            const int xr = q >> 5;
            const int xkb = xc >> 3;
            const int rows_here = min(BM, M - m0);
            // FP32 A rows of this tile; every offset is range checked (the
            // resource starts at the tile's first row, so offsets stay below
            // 128 ldx 4 < 2^31)
            const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(qa.x + static_cast<int64_t>(m0) * qa.ldx), 0,
                rows_here * static_cast<int>(qa.ldx) * 4, 0x00020000);
            const uint32_t x_off0 = static_cast<uint32_t>((xr * static_cast<int>(qa.ldx) + xc * 4) * 4);
            const uint32_t x_row8 = static_cast<uint32_t>(32 * qa.ldx);
            const bool write_a = qa.codes != nullptr && tn == 0;
            float4 xa[16], xb[16];
            // stage `stage`'s values (clamped to the last stage); rows past M
            // and columns past K read as zero
            auto load = [&](float4 (&v)[16], int stage) {
                const int st = min(stage, last);
                const bool col_ok = st * 128 + xc * 4 < K;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const bool ok = col_ok && xr + 8 * i < rows_here;
                    const uint32_t vo = ok ? x_off0 + i * x_row8 + st * 512 : 0x80000000u;
                    const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs_x, static_cast<int>(vo), 0, 0);
                    v[i] = make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]),
                                       __uint_as_float(w[2]), __uint_as_float(w[3]));
                }
            };
            // this wave's tile maxima of v into red[par] (the 16 lanes of a
            // wave that hold one tile differ in lane bits 0, 1, 2 and 5)
            auto publish = [&](const float4 (&v)[16], int par) {
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) m = fmaxf(m, abs_max4(v[i]));
                m = fmaxf(m, __shfl_xor(m, 1));
                m = fmaxf(m, __shfl_xor(m, 2));
                m = fmaxf(m, __shfl_xor(m, 4));
                m = fmaxf(m, __shfl_xor(m, 32));
                if ((lane & 0x27) == 0) red[par][cw][xkb] = m;
            };
            // this lane's tile scale of stage `stage` from red[stage % 2]; the
            // four scales also go to sa_lds for the GEMM waves (and to
            // qa.scales in write_a workgroups)
            auto form = [&](int stage) {
                constexpr float F = fp8_max<AF>();
                const int par = stage & 1;
                const float am = fmaxf(fmaxf(red[par][0][xkb], red[par][1][xkb]),
                                       fmaxf(red[par][2][xkb], red[par][3][xkb]));
                float sc = am / F;
                if (sc == 0.0f) sc = 1.0f;
                if (cw == 0 && (lane & 0x27) == 0) {
                    sa_lds[par][xkb] = sc;
                    if (write_a && stage <= last && stage * 4 + xkb < nkb)
                        qa.scales[static_cast<int64_t>(tm) * nkb + stage * 4 + xkb] = sc;
                }
                return sc;
            };
            // encode v (stage `stage`) into LDS buffer stage % 2: the code
            // dword of item i is row R = xr + 8 i, bytes 4 xc .. 4 xc + 3 of
            // the stage, i.e. in 16-byte chunk xc / 4, stored at
            // (xc / 4) ^ ((R >> 1) & 7) like the direct loads of B
            auto encode = [&](const float4 (&v)[16], int stage, float sc) {
                uint32_t w[16];
                if (__all(sc >= kNearScaleMin)) {
                    const Fp8QuotientNear qt(sc);
#pragma unroll
                    for (int i = 0; i < 16; ++i) w[i] = fp8_codes4<AF>(qt, v[i]);
                } else {
                    const Fp8Quotient qt(sc);
#pragma unroll
                    for (int i = 0; i < 16; ++i) w[i] = fp8_codes4<AF>(qt, v[i]);
                }
                const int buf = stage & 1;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int R = xr + 8 * i;
                    const int off = buf * kDStage + R * kDRow + (((xc >> 2) ^ ((R >> 1) & 7)) << 4) + (xc & 3) * 4;
                    *reinterpret_cast<uint32_t*>(lds + off) = w[i];
                }
                if (write_a && stage <= last) {
                    const int col = stage * 128 + xc * 4;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int R = xr + 8 * i;
                        if (R < rows_here && col < K)
                            *reinterpret_cast<uint32_t*>(qa.codes + static_cast<int64_t>(m0 + R) * K + col) = w[i];
                    }
                }
            };
            auto barrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
            // between stage barriers s - 1 and s: cur holds stage s + 1, nxt
            // receives stage s + 2
            auto step = [&](float4 (&cur)[16], float4 (&nxt)[16], int s) {
                load(nxt, s + 2);
                encode(cur, s + 1, form(s + 1));
                publish(nxt, s & 1);
                barrier();
            };
            // the GEMM waves' two prologue barriers
            load(xa, 0);
            publish(xa, 0);
            barrier();
            load(xb, 1);
            encode(xa, 0, form(0));
            publish(xb, 1);
            barrier();
            for (int s = 0; s < nfull; s += 2) {
                step(xb, xa, s);
                if (s + 1 < nfull) step(xa, xb, s + 1);
            }
#pragma unroll
            for (int i = 0; i < kEpilogueBarriers; ++i) __syncthreads();
            return;
        }
    }

    // direct loads: instruction i (0..3) of wave w fills rows 32 i + 8 w .. + 7.
    // The buffer resources start at the tile's first row and cover its rows,
    // so every offset stays below 128 K < 2^31 (K < 2^24) however large the
    // operand, and rows past M or N fail the range check and read as zero.
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A) + (QA ? 0 : static_cast<int64_t>(m0) * K), 0,
        QA ? 0 : min(BM, M - m0) * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B) + static_cast<int64_t>(n0) * K, 0, min(BN, N - n0) * K, 0x00020000);
    const int drow = 8 * wave + (lane >> 3);
    const int dchunk = (lane & 7) ^ ((drow >> 1) & 7);
    const uint32_t dma_a = static_cast<uint32_t>(drow) * K + dchunk * 16;
    const uint32_t dma_b = static_cast<uint32_t>(drow) * K + dchunk * 16;
    const uint32_t row_step = 32u * static_cast<uint32_t>(K);
    // direct loads of a stage: A (without QA) and B, alternating.  The stage's
    // K offset rides in the scalar offset, which the range check does not
    // cover.  A full stage lies inside every row; in a partial last stage (K
    // not a multiple of 128) the chunks at or past K are CHECKED: they get an
    // out-of-range VGPR offset and read as zero without touching memory.
    const int kend = K - dchunk * 16;       // chunk at stage offset so is inside K iff so < kend
    auto dma_one = [&](auto J, int stage, int buf, auto CHECKED) {
        constexpr int j = J;
        constexpr int i = j >> 1;
        const int so = min(stage, last) * 128;
        if constexpr ((j & 1) == 0) {
            if constexpr (!QA) {
                uint32_t vo = dma_a + i * row_step;
                if constexpr (CHECKED) vo = so < kend ? vo : 0x80000000u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs_a, (lds_void*)(lds + buf * kDStage + (32 * i + 8 * wave) * kDRow), 16, vo, so, 0, 0);
            }
        } else {
            uint32_t vo = dma_b + i * row_step;
            if constexpr (CHECKED) vo = so < kend ? vo : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs_b, (lds_void*)(lds + buf * kDStage + kDOperand + (32 * i + 8 * wave) * kDRow), 16, vo, so,
                0, 0);
        }
    };
    auto dma_stage = [&](int stage, int buf, auto CHECKED) {
        static_for<8>([&](auto J) { dma_one(J, stage, buf, CHECKED); });
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
    // (with QA, A's come from the quantiser waves through LDS)
    // An operand with one scale per tensor (bit 0 of tensor_mask: A, bit 1: B)
    // has a one-float scale array: its stage loads read past that float as
    // zero and are not used; sa0 / sb0 stand in for them.
    const bool a_tensor = !QA && (tensor_mask & 1) != 0;
    const bool b_tensor = (tensor_mask & 2) != 0;
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(sA), 0, QA ? 0 : a_tensor ? 4 : static_cast<int>(tiles_m) * nkb * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(sB), 0, b_tensor ? 4 : static_cast<int>(tiles_n) * nkb * 4, 0x00020000);
    const uint32_t so_a = a_tensor ? 0u : static_cast<uint32_t>(tm) * nkb * 4;
    const uint32_t so_b = b_tensor ? 0u : static_cast<uint32_t>(tn) * nkb * 4;
    // (bit 2 / bit 3: that side's scales are per row and applied at write-back)
    float sa0 = 0.0f;
    if constexpr (!QA) sa0 = (tensor_mask & 4) ? 1.0f : sA[0];
    const float sb0 = (tensor_mask & 8) ? 1.0f : sB[0];
    auto sigma = [&](uint32_t a_bits, uint32_t b_bits) {
        return (a_tensor ? sa0 : __uint_as_float(a_bits)) * (b_tensor ? sb0 : __uint_as_float(b_bits));
    };
    u32x4 nsa = u32x4{}, nsb;
    // A full stage's four scales lie inside the tile row, and the stage offset
    // rides in the scalar offset.  In a partial last stage (K / 32 not a
    // multiple of 4) the four scales would reach past the row, and for the
    // last tile row past the array: CHECKED loads put the stage offset in the
    // range-checked VGPR offset instead, and a dwordx4 load is checked per
    // dword, so the scales past the array read as zero without touching
    // memory.  A per-tensor side keeps its offset at zero: its load covers the
    // one-float array and three dwords that read as zero.
    auto load_scales = [&](int stage, auto CHECKED) {
        const int so = min(stage, last) * 16;
        const int so_sa = a_tensor ? 0 : so;
        const int so_sb = b_tensor ? 0 : so;
        if constexpr (CHECKED) {
            const uint32_t va = so_a + so_sa, vb = so_b + so_sb;
            if constexpr (!QA)
                asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(nsa) : "v"(va), "s"(rs_sa) : "memory");
            asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(nsb) : "v"(vb), "s"(rs_sb) : "memory");
        } else {
            if constexpr (!QA)
                asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(nsa) : "v"(so_a), "s"(rs_sa), "s"(so_sa) : "memory");
            asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(nsb) : "v"(so_b), "s"(rs_sb), "s"(so_sb) : "memory");
        }
    };
    constexpr std::true_type kChecked{};
    constexpr std::false_type kUnchecked{};

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
    u32x4 fx[2][2], fy[2][2];    // [set][t]
    // the last tile's product of the previous block, promoted during the next
    // block (a zero product with a zero scale before the first)
    v16f pend = v16f{};
    float pend_sig = 0.0f;
    auto promote = [](v16f& a, float sg, const v16f& p) {
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = fmaf(sg, p[r], a[r]);
    };
    // MFMA instructions per 32-wide block of the wave's four 32 x 32 tiles
    constexpr int kMfmaPerBlock = 8;

    // the prologue's loads are checked (stage 0 or 1 may be the partial one)
    dma_stage(0, 0, kChecked);
    load_scales(0, kChecked);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // with QA, a second barrier: stage 0's A codes and scales are in LDS
    if constexpr (QA) asm volatile("s_barrier" ::: "memory");
    static_for<2>([&](auto t) {
        lds_read16<t * 32 * kDRow>(fx[0][t], rd_b[0][0]);
        lds_read16<t * 32 * kDRow>(fy[0][t], rd_a[0][0]);
    });
    dma_stage(1, 1, kChecked);

    // Full stages run unconditionally; a partial last stage (K not a multiple
    // of 128) is finished by the tail below.  A stage loads the scales of the
    // next stage and the codes of the one after; only the last two full stages
    // can load the partial stage, so only they run the checked loads.
    auto run_stage = [&](int s, auto CHECKED) {
        const int cb = s & 1;
        // this stage's scales: issued one stage ago, followed by the direct
        // loads of the next stage (8 of them, 4 with QA)
        if constexpr (QA) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        u32x4 ca = nsa, cbv = nsb;
        asm volatile("" : "+v"(ca), "+v"(cbv));
        float sig[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (QA) sig[k] = sa_lds[cb][k] * (b_tensor ? sb0 : __uint_as_float(cbv[k]));
            else sig[k] = sigma(ca[k], cbv[k]);
        }
        load_scales(s + 1, CHECKED);

        auto block = [&](auto KB) {
            constexpr int kb = KB;
            constexpr int nkb_ = (kb + 1) & 3;
            const int rb = kb == 3 ? cb ^ 1 : cb;
            u32x4 (&f)[2] = fx[kb & 1];
            u32x4 (&g)[2] = fy[kb & 1];
            if constexpr (kb == 3) {
                // the next stage's direct loads are in (only its scales, one
                // load, or two without QA, may be outstanding)
                if constexpr (QA) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            } else {
                lds_wait();
            }
            // prefetch the next block's fragments
            static_for<2>([&](auto t) {
                lds_read16<t * 32 * kDRow>(fx[(kb + 1) & 1][t], rb ? rd_b[1][nkb_] : rd_b[0][nkb_]);
                lds_read16<t * 32 * kDRow>(fy[(kb + 1) & 1][t], rb ? rd_a[1][nkb_] : rd_a[0][nkb_]);
            });
            if constexpr (kb == 3) dma_stage(s + 2, cb, CHECKED);
            // the MFMAs below may only start after the prefetch is issued
            asm volatile("" : "+v"(f[0]), "+v"(f[1]), "+v"(g[0]), "+v"(g[1]));
            // Software-pipelined promotion: each tile's product is promoted
            // while the next tile's MFMAs run (the last tile's, while the
            // next block's first MFMAs run), one MFMA then 8 FMAs, so that the
            // matrix core and the VALU work at the same time.  Every
            // accumulator still receives its blocks in K order.
            const float sig_kb = sig[kb];
            if constexpr (OUT == BSFP8_OUT_F32) {
                const v16f p0 = tile_product<AF, BF, OUT>(f[0], g[0]);
                promote(acc[1][1], pend_sig, pend);
                const v16f p1 = tile_product<AF, BF, OUT>(f[0], g[1]);
                promote(acc[0][0], sig_kb, p0);
                const v16f p2 = tile_product<AF, BF, OUT>(f[1], g[0]);
                promote(acc[0][1], sig_kb, p1);
                pend = tile_product<AF, BF, OUT>(f[1], g[1]);
                promote(acc[1][0], sig_kb, p2);
#pragma unroll
                for (int i = 0; i < kMfmaPerBlock; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 64 / kMfmaPerBlock, 0);  // then its FMAs
                }
            } else {
                // the same order fixed by scheduling barriers: left free, the
                // compiler placed FMAs right behind the MFMA whose result they
                // read, holding the wave's next MFMA back
                // tile product q of x, y while the previous tile's product pp
                // is promoted into pa
                auto tile_slots = [&](v16f& q, const u32x4& x, const u32x4& y, v16f& pa, float ps,
                                      const v16f& pp) {
                    __builtin_amdgcn_sched_barrier(0);
                    q = product_half<AF, BF, 0>(x, y, v16f{});
                    __builtin_amdgcn_sched_barrier(0);
                    promote_half<0>(pa, ps, pp);
                    __builtin_amdgcn_sched_barrier(0);
                    q = product_half<AF, BF, 1>(x, y, q);
                    __builtin_amdgcn_sched_barrier(0);
                    promote_half<1>(pa, ps, pp);
                    __builtin_amdgcn_sched_barrier(0);
                };
                v16f q0, q1, q2, q3;
                tile_slots(q0, f[0], g[0], acc[1][1], pend_sig, pend);
                tile_slots(q1, f[0], g[1], acc[0][0], sig_kb, q0);
                tile_slots(q2, f[1], g[0], acc[0][1], sig_kb, q1);
                tile_slots(q3, f[1], g[1], acc[1][0], sig_kb, q2);
                pend = q3;
            }
            pend_sig = sig_kb;
        };
        block(std::integral_constant<int, 0>{});
        block(std::integral_constant<int, 1>{});
        block(std::integral_constant<int, 2>{});
        block(std::integral_constant<int, 3>{});
    };
    const int nfast = nfull < nst ? max(0, nfull - 2) : nfull;
    int s0 = 0;
    for (; s0 < nfast; ++s0) run_stage(s0, kUnchecked);
    for (; s0 < nfull; ++s0) run_stage(s0, kChecked);
    // the last full block's pending tile
    promote(acc[1][1], pend_sig, pend);
    if (nfull < nst) {
        // partial stage: its data and block-0 fragments are already in place
        const int cb = nfull & 1;
        if constexpr (QA) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
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
            float sig_kb;
            if constexpr (QA) sig_kb = sa_lds[cb][kb] * (b_tensor ? sb0 : __uint_as_float(cbv[kb]));
            else sig_kb = sigma(ca[kb], cbv[kb]);
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
                    const v16f p = tile_product<AF, BF, OUT>(x[ti], y[tj]);
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[ti][tj][r] = fmaf(sig_kb, p[r], acc[ti][tj][r]);
                }
        }
    }
    // the last stage's scale loads and fragment reads may have no consumer:
    // naming them after the wait keeps their registers from being reused
    // while they are in flight
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    asm volatile("" :: "v"(nsa), "v"(nsb), "v"(fx[0][0]), "v"(fx[0][1]), "v"(fx[1][0]), "v"(fx[1][1]),
                       "v"(fy[0][0]), "v"(fy[0][1]), "v"(fy[1][0]), "v"(fy[1][1]));

    // Epilogue through LDS (free now): the tile is written in the MFMA layout
    // and read back by rows, so that each 64-lane store covers whole output
    // rows instead of 32 rows x 16 bytes.  16-byte chunk c of LDS row R sits at
    // c ^ (R & 15), which keeps the scattered writes and the row reads free of
    // bank conflicts.
    __syncthreads();
    if constexpr (OUT != BSFP8_OUT_F32) {
        if (ep.beta == 0.0f && !ep.row_scale && !ep.col_scale) {
            // 16-bit output without C: alpha * acc converted while staged
            // (128 rows x 256 bytes), a store covers 4 rows
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int R = wm * 64 + tj * 32 + frag_row;
                        const int c = wn * 8 + ti * 4 + q;
                        const uint32_t h0 = to_half_bits<OUT>(ep.alpha * acc[ti][tj][4 * q + 0]);
                        const uint32_t h1 = to_half_bits<OUT>(ep.alpha * acc[ti][tj][4 * q + 1]);
                        const uint32_t h2 = to_half_bits<OUT>(ep.alpha * acc[ti][tj][4 * q + 2]);
                        const uint32_t h3 = to_half_bits<OUT>(ep.alpha * acc[ti][tj][4 * q + 3]);
                        *reinterpret_cast<uint2*>(lds + R * 256 + ((c ^ (R & 15)) << 4) + 8 * half) =
                            make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
                    }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int R = wave * 32 + i * 4 + (lane >> 4);
                const int c = lane & 15;
                const uint4 w = *reinterpret_cast<const uint4*>(lds + R * 256 + ((c ^ (R & 15)) << 4));
                store_half8(D, ldd, m0 + R, n0 + c * 8, M, N, vec_ok, w);
            }
            return;
        }
    }
    // General case: the FP32 tile (128 rows x 512 bytes, the whole 64 KB);
    // alpha, beta * C and the output conversion are applied in the row phase.
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int R = wm * 64 + tj * 32 + frag_row;
                const int c = wn * 16 + ti * 8 + q * 2 + half;
                *reinterpret_cast<float4*>(lds + R * 512 + ((c ^ (R & 15)) << 4)) =
                    make_float4(acc[ti][tj][4 * q + 0], acc[ti][tj][4 * q + 1],
                                acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]);
            }
    __syncthreads();
    if constexpr (OUT == BSFP8_OUT_F32) {
        // 4 values per lane: a store covers 2 rows
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
            const int R = wave * 32 + i * 2 + (lane >> 5);
            const int c = lane & 31;
            const float4 v = *reinterpret_cast<const float4*>(lds + R * 512 + ((c ^ (R & 15)) << 4));
            const float a4[4] = {v.x, v.y, v.z, v.w};
            finish_row_chunk<OUT, 4>(D, ldd, ep, m0 + R, n0 + c * 4, M, N, vec_ok, a4);
        }
    } else {
        // 8 values per lane: a store covers 4 rows
#pragma unroll 4
        for (int i = 0; i < 8; ++i) {
            const int R = wave * 32 + i * 4 + (lane >> 4);
            const int c = (lane & 15) * 2;
            const float4 v0 = *reinterpret_cast<const float4*>(lds + R * 512 + ((c ^ (R & 15)) << 4));
            const float4 v1 = *reinterpret_cast<const float4*>(lds + R * 512 + (((c + 1) ^ (R & 15)) << 4));
            const float a8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            finish_row_chunk<OUT, 8>(D, ldd, ep, m0 + R, n0 + c * 4, M, N, vec_ok, a8);
        }
    }
}

// Skinny form (few output rows, so few 128 x 128 tiles: the two-pass kernel
// would keep only a handful of CUs streaming B).  One workgroup per 32 x 32
// output tile, N / 32 of them per 32 rows; its four waves split K into four
// contiguous ranges of 4-block chunks and each computes the tile's partial sum
// over its range with the same per-block product and promotion as the main
// kernel (tile_product, acc = fma(sigma_kb, P_kb, acc)).  Each load
// instruction reads whole 128-byte row segments (8 rows x 128 bytes), which
// pass through the wave's own LDS area into the MFMA layout (lane (r, h) takes
// the 16 codes K 16 h .. 16 h + 15 of row r of a block); kDepth chunks are in
// flight.  Range-checked buffer loads: rows past M or N and blocks past the
// wave's range read as zero and their sigma is zero.  The four partial sums are
// added in a fixed order through LDS, so the result does not depend on
// timing; wave 0 writes the tile.
// OUTER: scales constant along K (per row of A or per tensor, per column of B
// or per tensor; a_step / b_step are 1 or 0): the blocks are summed unscaled
// and the scale product multiplies the sum once, at write-back, as in the
// K-constant kernel.
constexpr int kSkinnyDepth = 2;              // chunks of 4 blocks in flight per wave
constexpr int kSkinnyWaves = 4;              // waves per workgroup, splitting K
constexpr int64_t kSkinnyMaxM = 64;          // rows up to which the skinny form is used
constexpr int64_t kSkinnyMaxTiles = 32;      // ... and 128 x 128 tiles below which it is too

template <int AF, int BF, int OUT, bool OUTER>
__global__ __launch_bounds__(64 * kSkinnyWaves, 8 / kSkinnyWaves) void gemm_fp8_skinny_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sA,
    const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok, int tensor_mask, int a_step,
    int b_step) {
    __shared__ v16f part[kSkinnyWaves - 1][64];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kSkinnyWaves][2][32 * 128];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Workgroups go to the 8 XCDs round-robin by launch index.  The row tiles
    // of one column tile are launched 8 apart, so they run on the same XCD at
    // about the same time and read that tile's B rows through one L2.  The
    // column tiles are padded to a multiple of 8; padding workgroups exit.
    const int grp = static_cast<int>(blockIdx.x) / (8 * tiles_m);
    const int rem = static_cast<int>(blockIdx.x) - grp * 8 * tiles_m;
    const int tm = rem >> 3, tn = grp * 8 + (rem & 7);
    if (tn >= tiles_n) return;
    const int m0 = tm * 32, n0 = tn * 32;
    const int nkb = K >> 5;
    // K is split into chunks of 4 blocks (128 bytes of each row); each wave
    // takes a contiguous range of chunks
    const int nch = (nkb + 3) >> 2;
    const int cper = (nch + kSkinnyWaves - 1) / kSkinnyWaves;
    const int c0 = min(wave * cper, nch), c1 = min(c0 + cper, nch);
    const int kb1 = min(4 * c1, nkb);

    // operand rows of this tile (the resources start at its first row, so
    // offsets stay below 32 K)
    const int rows_a = min(32, M - m0), rows_b = min(32, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A) + static_cast<int64_t>(m0) * K, 0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B) + static_cast<int64_t>(n0) * K, 0, rows_b * K, 0x00020000);
    const int r = lane & 31, h = lane >> 5;
    // sigma of block kb (zero past the wave's range)
    const bool a_tensor = (tensor_mask & 1) != 0, b_tensor = (tensor_mask & 2) != 0;
    const float* sa_row = sA + (a_tensor ? 0 : static_cast<int64_t>(m0 >> 7) * nkb);
    const float* sb_row = sB + (b_tensor ? 0 : static_cast<int64_t>(n0 >> 7) * nkb);
    // (bit 2 / bit 3: that side's scales are per row and applied at
    // write-back; bits 0 / 1 are then set as well, so index 0 is in range).
    // Branch-free: both scales are loaded from a clamped index and selected,
    // since conditional loads here compiled to a branch per block.
    const bool a_unit = (tensor_mask & 4) != 0, b_unit = (tensor_mask & 8) != 0;
    auto sigma = [&](int kb) {
        if constexpr (OUTER) return kb < kb1 ? 1.0f : 0.0f;
        const int kc = max(0, min(kb, nkb - 1));
        float la = sa_row[a_tensor ? 0 : kc], lb = sb_row[b_tensor ? 0 : kc];
        // the empty asm uses both loads, so that they are not moved into branches
        asm volatile("" : "+s"(la), "+s"(lb));
        const float sa = a_unit ? 1.0f : la;
        const float sb = b_unit ? 1.0f : lb;
        return kb < kb1 ? sa * sb : 0.0f;
    };
    // Loads read whole 128-byte row segments: lane l takes 16-byte piece l & 7
    // of row (l >> 3) + 8 i, so each instruction covers 8 rows x 128 bytes.
    // The wave stages the chunk in its own LDS area (piece g of row R at
    // g ^ (R & 7)) and reads the MFMA fragments back: lane (r, h) takes bytes
    // 32 b + 16 h .. + 15 of row r for block b of the chunk.
    const int lr = lane >> 3, lg = lane & 7;
    uint8_t* st_a = stage[wave][0];
    uint8_t* st_b = stage[wave][1];
    u32x4 ga[kSkinnyDepth][4], gb[kSkinnyDepth][4];
    auto fetch = [&](auto SLOT, int c) {
        constexpr int j = SLOT;
        const bool ok = c < c1 && 4 * c + (lg >> 1) < nkb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = ok ? static_cast<uint32_t>((lr + 8 * i) * K + 128 * c + 16 * lg) : 0x80000000u;
            const auto wa = __builtin_amdgcn_raw_buffer_load_b128(rs_a, static_cast<int>(o), 0, 0);
            const auto wb = __builtin_amdgcn_raw_buffer_load_b128(rs_b, static_cast<int>(o), 0, 0);
            ga[j][i] = u32x4{wa[0], wa[1], wa[2], wa[3]};
            gb[j][i] = u32x4{wb[0], wb[1], wb[2], wb[3]};
        }
    };
    v16f acc = v16f{};
    static_for<kSkinnyDepth>([&](auto J) { fetch(J, c0 + J); });
    for (int c = c0; c < c1; c += kSkinnyDepth) {
        static_for<kSkinnyDepth>([&](auto J) {
            constexpr int j = J;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = lr + 8 * i;
                const int pos = row * 128 + 16 * (lg ^ (row & 7));
                *reinterpret_cast<u32x4*>(st_a + pos) = ga[j][i];
                *reinterpret_cast<u32x4*>(st_b + pos) = gb[j][i];
            }
            fetch(J, c + j + kSkinnyDepth);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int pos = r * 128 + 16 * ((2 * b + h) ^ (r & 7));
                const u32x4 xa = *reinterpret_cast<const u32x4*>(st_a + pos);
                const u32x4 xb = *reinterpret_cast<const u32x4*>(st_b + pos);
                const float sgb = sigma(4 * (c + j) + b);
                const v16f p = tile_product<AF, BF, OUT>(xb, xa);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = fmaf(sgb, p[e], acc[e]);
            }
        });
    }
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    // the partial sums of waves 1, 2, ..., added in that order
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w) {
        const v16f q = part[w][lane];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += q[e];
    }
    // lane (r, h) holds row m0 + r, columns n0 + 8 q + 4 h + e in acc[4 q + e]
    float s_m = 1.0f;
    if constexpr (OUTER) s_m = sA[static_cast<int64_t>(min(m0 + r, M - 1)) * a_step];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float a4[4] = {acc[4 * q + 0], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        if constexpr (OUTER) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = min(n0 + 8 * q + 4 * h + e, N - 1);
                a4[e] = (s_m * sB[static_cast<int64_t>(n) * b_step]) * a4[e];
            }
        }
        finish_row_chunk<OUT, 4>(D, ldd, ep, m0 + r, n0 + 8 * q + 4 * h, M, N, vec_ok, a4);
    }
}

// The skinny form for scales constant along K (called by the K-constant GEMM's
// launcher for up to kSkinnyMaxM rows).
template <int AF, int BF>
hipError_t launch_skinny_outer_typed(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                                     int a_step, const uint8_t* b, const float* sb, int b_step, int out,
                                     void* d, int64_t ldd, const Epilogue& ep, hipStream_t stream) {
    const int tm = static_cast<int>((M + 31) / 32), tn = static_cast<int>((N + 31) / 32);
    const uint32_t wgs = static_cast<uint32_t>((tn + 7) / 8) * 8u * static_cast<uint32_t>(tm);
    const int vec = vec16_ok(out, d, ldd, ep);
    const int Mi = static_cast<int>(M), Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    if (out == BSFP8_OUT_F32)
        hipLaunchKernelGGL((gemm_fp8_skinny_kernel<AF, BF, BSFP8_OUT_F32, true>), dim3(wgs), dim3(64 * kSkinnyWaves), 0,
                           stream, Mi, Ni, Ki, a, sa, b, sb, d, ldd, ep, tm, tn, vec, 0, a_step, b_step);
    else if (out == BSFP8_OUT_BF16)
        hipLaunchKernelGGL((gemm_fp8_skinny_kernel<AF, BF, BSFP8_OUT_BF16, true>), dim3(wgs), dim3(64 * kSkinnyWaves), 0,
                           stream, Mi, Ni, Ki, a, sa, b, sb, d, ldd, ep, tm, tn, vec, 0, a_step, b_step);
    else
        hipLaunchKernelGGL((gemm_fp8_skinny_kernel<AF, BF, BSFP8_OUT_F16, true>), dim3(wgs), dim3(64 * kSkinnyWaves), 0,
                           stream, Mi, Ni, Ki, a, sa, b, sb, d, ldd, ep, tm, tn, vec, 0, a_step, b_step);
    return hipGetLastError();
}

template <int AF, int BF, int OUT, bool QA>
hipError_t launch_out(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                      const uint8_t* b, const float* sb, void* d, int64_t ldd,
                      const Epilogue& ep, int tensor_mask, const OnlineA& qa, hipStream_t stream) {
    if constexpr (!QA) {
        if (M <= kSkinnyMaxM || ((M + 127) / 128) * ((N + 127) / 128) < kSkinnyMaxTiles) {
            const int tm = static_cast<int>((M + 31) / 32), tn = static_cast<int>((N + 31) / 32);
            const uint32_t wgs = static_cast<uint32_t>((tn + 7) / 8) * 8u * static_cast<uint32_t>(tm);
            hipLaunchKernelGGL((gemm_fp8_skinny_kernel<AF, BF, OUT, false>), dim3(wgs), dim3(64 * kSkinnyWaves), 0,
                               stream, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, sa,
                               b, sb, d, ldd, ep, tm, tn, vec16_ok(OUT, d, ldd, ep), tensor_mask, 0, 0);
            return hipGetLastError();
        }
    }
    const int tiles_m = static_cast<int>((M + BM - 1) / BM);
    const int tiles_n = static_cast<int>((N + BN - 1) / BN);
    const dim3 grid(static_cast<uint32_t>(tiles_m) * static_cast<uint32_t>(tiles_n));
    hipLaunchKernelGGL((gemm_fp8_kernel<AF, BF, OUT, QA>), grid, dim3(QA ? kQThreads : kThreads), 0, stream,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, sa, b, sb,
                       d, ldd, ep, tiles_m, tiles_n, vec16_ok(OUT, d, ldd, ep), tensor_mask, qa);
    return hipGetLastError();
}

template <int AF, int BF, bool QA>
hipError_t launch_typed(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                        const uint8_t* b, const float* sb, int out, void* d, int64_t ldd,
                        const Epilogue& ep, int tm, const OnlineA& qa, hipStream_t stream) {
    if (out == BSFP8_OUT_F32)
        return launch_out<AF, BF, BSFP8_OUT_F32, QA>(M, N, K, a, sa, b, sb, d, ldd, ep, tm, qa, stream);
    if (out == BSFP8_OUT_BF16)
        return launch_out<AF, BF, BSFP8_OUT_BF16, QA>(M, N, K, a, sa, b, sb, d, ldd, ep, tm, qa, stream);
    return launch_out<AF, BF, BSFP8_OUT_F16, QA>(M, N, K, a, sa, b, sb, d, ldd, ep, tm, qa, stream);
}

template <bool QA>
hipError_t launch_formats(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                          const float* a_scales, int b_fmt, const uint8_t* b, const float* b_scales,
                          int out, void* d, int64_t ldd, const Epilogue& ep, int tensor_mask,
                          const OnlineA& qa, hipStream_t stream) {
    // problems with enough 256 x 256 tiles take the large-tile kernel (half the
    // L2-to-LDS bytes per FLOP); the others the 128 x 128 or skinny kernels
    if (!QA && M > kSkinnyMaxM && gemm_fp8_big_fits(M, N, K))
        return launch_gemm_fp8_big(M, N, K, a_fmt, a, a_scales, b_fmt, b, b_scales, out, d, ldd, ep,
                                   tensor_mask, stream);
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E4M3)
        return launch_typed<BSFP8_E4M3, BSFP8_E4M3, QA>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, tensor_mask, qa, stream);
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E5M2)
        return launch_typed<BSFP8_E4M3, BSFP8_E5M2, QA>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, tensor_mask, qa, stream);
    if (a_fmt == BSFP8_E5M2 && b_fmt == BSFP8_E4M3)
        return launch_typed<BSFP8_E5M2, BSFP8_E4M3, QA>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, tensor_mask, qa, stream);
    return launch_typed<BSFP8_E5M2, BSFP8_E5M2, QA>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, tensor_mask, qa, stream);
}

}  // namespace

hipError_t launch_gemm_fp8(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                           const float* a_scales, int b_fmt, const uint8_t* b,
                           const float* b_scales, int out, void* d, int64_t ldd,
                           const Epilogue& ep, hipStream_t stream, int tensor_mask) {
    const OnlineA none{nullptr, 0, nullptr, nullptr};
    return launch_formats<false>(M, N, K, a_fmt, a, a_scales, b_fmt, b, b_scales, out, d, ldd, ep,
                                 tensor_mask, none, stream);
}

bool skinny_outer_fits(int64_t M) { return M <= kSkinnyMaxM; }

hipError_t launch_gemm_fp8_skinny_outer(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                                        const float* a_scales, int a_step, int b_fmt, const uint8_t* b,
                                        const float* b_scales, int b_step, int out, void* d, int64_t ldd,
                                        const Epilogue& ep, hipStream_t stream) {
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E4M3)
        return launch_skinny_outer_typed<BSFP8_E4M3, BSFP8_E4M3>(M, N, K, a, a_scales, a_step, b, b_scales, b_step, out, d, ldd, ep, stream);
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E5M2)
        return launch_skinny_outer_typed<BSFP8_E4M3, BSFP8_E5M2>(M, N, K, a, a_scales, a_step, b, b_scales, b_step, out, d, ldd, ep, stream);
    if (a_fmt == BSFP8_E5M2 && b_fmt == BSFP8_E4M3)
        return launch_skinny_outer_typed<BSFP8_E5M2, BSFP8_E4M3>(M, N, K, a, a_scales, a_step, b, b_scales, b_step, out, d, ldd, ep, stream);
    return launch_skinny_outer_typed<BSFP8_E5M2, BSFP8_E5M2>(M, N, K, a, a_scales, a_step, b, b_scales, b_step, out, d, ldd, ep, stream);
}

hipError_t launch_gemm_fp8_online_a(int64_t M, int64_t N, int64_t K, int a_fmt, const OnlineA& qa,
                                    int b_fmt, const uint8_t* b, const float* b_scales,
                                    int b_tensor, int out, void* d, int64_t ldd,
                                    const Epilogue& ep, hipStream_t stream) {
    return launch_formats<true>(M, N, K, a_fmt, nullptr, nullptr, b_fmt, b, b_scales, out, d, ldd,
                                ep, b_tensor ? 2 : 0, qa, stream);
}

}  // namespace bsfp8
