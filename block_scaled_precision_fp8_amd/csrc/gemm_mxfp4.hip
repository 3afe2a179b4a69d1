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
#include "big_tile.h"

namespace bsfp8 {

namespace {

using namespace big_tile;
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

// byte Q of each scale register
template <int Q = 0>
__device__ __forceinline__ v16f mfma_fp4(uint4 x, uint4 y, uint32_t sx, uint32_t sy, v16f c) {
    v8i a = {static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z),
             static_cast<int>(x.w), 0, 0, 0, 0};
    v8i b = {static_cast<int>(y.x), static_cast<int>(y.y), static_cast<int>(y.z),
             static_cast<int>(y.w), 0, 0, 0, 0};
    // format 4 = E2M1 for both operands
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, Q, static_cast<int>(sx), Q,
                                                           static_cast<int>(sy));
}

// SUB: E8M0 scale blocks per 32 K values (1: MXFP4; 2, 4: blocks of 16, 8,
// one MFMA per block with the lane's other A values zeroed, as in the large
// kernel below).
template <int OUT, int SUB = 1>
__global__ __launch_bounds__(kThreads, 2) void gemm_mxfp4_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
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
    const int nkb = K >> 5;          // 32-wide K blocks per row
    const int nsb = nkb * SUB;       // scale bytes per row
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
        sa_p[t] = sA + static_cast<int64_t>(ra) * nsb;
        sb_p[t] = sB + static_cast<int64_t>(rb) * nsb;
    }
    // the lane's SUB scale bytes of 32-wide block kb (one aligned load)
    auto scale_word = [&](const uint8_t* p, int kb) -> uint32_t {
        if constexpr (SUB == 1) return p[kb];
        else if constexpr (SUB == 2) return *reinterpret_cast<const uint16_t*>(p + 2 * kb);
        else return *reinterpret_cast<const uint32_t*>(p + 4 * kb);
    };
    // SUB MFMAs per tile pair: block q of the lane's 32 values (A's other
    // values zero) under scale byte q of each operand
    auto mfma_sub = [&](v16f& c, const uint4& xv, const uint4& yv, uint32_t sx, uint32_t sy) {
        if constexpr (SUB == 1) {
            c = mfma_fp4(xv, yv, sx, sy, c);
        } else {
            static_for<SUB>([&](auto Q) {
                constexpr int q = Q;
                const uint32_t w[4] = {yv.x, yv.y, yv.z, yv.w};
                uint32_t z[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) z[i] = (i * SUB / 4 == q) ? w[i] : 0u;
                c = mfma_fp4<q>(xv, make_uint4(z[0], z[1], z[2], z[3]), sx, sy, c);
            });
        }
    };

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
            sx[t] = scale_word(sb_p[t], blk);
            sy[t] = scale_word(sa_p[t], blk);
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int tj = 0; tj < 2; ++tj)
                mfma_sub(acc[ti][tj], x[ti], y[tj], sx[ti], sy[tj]);
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
                    sx[t] = scale_word(sb_p[t], nkb - 1);
                    sy[t] = scale_word(sa_p[t], nkb - 1);
                }
#pragma unroll
                for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                    for (int tj = 0; tj < 2; ++tj)
                        mfma_sub(acc[ti][tj], x[ti], y[tj], sx[ti], sy[tj]);
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
                const float a4[4] = {acc[ti][tj][4 * q + 0], acc[ti][tj][4 * q + 1],
                                     acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]};
                finish_row_chunk<OUT, 4>(D, ldd, ep, m, n, M, N, vec_ok, a4);
            }
        }
}

// ---------------------------------------------------------------------------
// Large-tile variant for K a multiple of 256: 256 x 256 output tile, 4 waves of
// 128 x 128 (4 x 4 MFMA tiles, 256 FP32 accumulators per lane held in the
// accumulation registers), one workgroup per CU.  A K step of 64 reads 8
// fragments of 1 KB per wave for 16 MFMAs, half the LDS traffic per FLOP of
// the 128 x 128 tiling; the 256-wide edge halves the L2 traffic per FLOP.
// Codes go straight from global memory to LDS (direct loads, rows past the
// matrix edge read as zero) one stage ahead of use; the E8M0 scales go the
// same way a period of 4 stages ahead, into 32 KB of LDS beside the codes.
//
// The same kernel serves E2M1 blocks of 16 K values with E8M0 scales (SUB = 2
// scale blocks per 32 K; "Rubin FP4 GEMM deep dive", section 5.3 for the
// smaller blocks).  The instruction takes one scale per lane and 32 K values,
// so each 32-K half of a lane is split in two: one MFMA multiplies the first
// 16 values of the A operand (the other 16 zero) under both operands' scales
// of the first block, a second one the last 16 under the second block's
// scales.  Zero codes add nothing, so every block keeps its own exact
// power-of-two scale, at two FP4 instructions per 64 K: half the FP4 rate,
// twice that of the bf16 instruction the dequantising kernels use.
// ---------------------------------------------------------------------------

// E2M1 x E2M1 MFMA with E8M0 block scales; byte SEL of each scale register is used.
template <int SEL>
__device__ __forceinline__ void mfma_fp4_sel(v16f& acc, const u32x4& x, const u32x4& y, uint32_t sx,
                                             uint32_t sy) {
    asm volatile(
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%5,0] "
        "op_sel_hi:[%6,%6,0] cbsz:4 blgp:4"
        : "+a"(acc)
        : "v"(x), "v"(y), "v"(sx), "v"(sy), "i"(SEL & 1), "i"(SEL >> 1));
}
// The same for an operand that the compiler assembles with VALU moves just
// before (an A chunk with some dwords zeroed): the two wait states in front
// cover the VALU-write to MFMA-read dependency, which the compiler does not
// track for inline assembly.
template <int SEL>
__device__ __forceinline__ void mfma_fp4_sel_w(v16f& acc, const u32x4& x, const u32x4& y, uint32_t sx,
                                               uint32_t sy) {
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%5,0] "
        "op_sel_hi:[%6,%6,0] cbsz:4 blgp:4"
        : "+a"(acc)
        : "v"(x), "v"(y), "v"(sx), "v"(sy), "i"(SEL & 1), "i"(SEL >> 1));
}
// Gather, for each of the 4 K steps of a stage, this lane's scale byte (block
// 2 ks + half of the stage's 8 blocks) into byte ks of one register.  The
// trailing wait states cover the VALU-write to MFMA-read dependency.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ void lds_read8(u32x2& v, uint32_t addr) {
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_read4(uint32_t& v, uint32_t addr) {
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
__device__ __forceinline__ void gather_scales(uint32_t& w0, uint32_t& w1, uint32_t& w2, uint32_t& w3,
                                              const u32x2& s0, const u32x2& s1, const u32x2& s2,
                                              const u32x2& s3, uint32_t sel) {
    asm volatile(
        "v_perm_b32 %0, %5, %4, %12\n\t"
        "v_perm_b32 %1, %7, %6, %12\n\t"
        "v_perm_b32 %2, %9, %8, %12\n\t"
        "v_perm_b32 %3, %11, %10, %12\n\t"
        "s_nop 4"
        : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
        : "v"(s0.x), "v"(s0.y), "v"(s1.x), "v"(s1.y), "v"(s2.x), "v"(s2.y), "v"(s3.x),
          "v"(s3.y), "v"(sel));
}
// Blocks of 16: a row's 16 scale bytes of a stage, byte 4 ks + 2 half + sub
// for the block of K step ks, lane half and sub-block sub; gather byte
// 2 half + sub of each of the four words into byte ks of lo (sub 0) and hi
// (sub 1).  sel is 0x05010400 + 0x02020202 * half.
__device__ __forceinline__ void gather_scales16(uint32_t& lo, uint32_t& hi, const u32x4& s, uint32_t sel) {
    uint32_t p01, p23;
    asm volatile(
        "v_perm_b32 %2, %5, %4, %8\n\t"
        "v_perm_b32 %3, %7, %6, %8\n\t"
        "v_perm_b32 %0, %3, %2, %9\n\t"
        "v_perm_b32 %1, %3, %2, %10\n\t"
        "s_nop 4"
        : "=&v"(lo), "=&v"(hi), "=&v"(p01), "=&v"(p23)
        : "v"(s.x), "v"(s.y), "v"(s.z), "v"(s.w), "v"(sel), "v"(0x05040100u), "v"(0x07060302u));
}

// Large-tile LDS layout: per buffer, A then B, each 256 rows of 128 bytes
// (unpadded, so that direct global-to-LDS loads can fill them).  Row R keeps
// its 16-byte chunk g at position g ^ ((R >> 1) & 7): the 16 lanes of a
// fragment-read phase (16 consecutive rows, one chunk) then hit 16 distinct
// 4-bank groups.
constexpr int kDmaRowBytes = 128;
constexpr int kDmaOperandBytes = 256 * kDmaRowBytes;     // 32 KB
constexpr int kDmaStageBytes = 2 * kDmaOperandBytes;     // 64 KB
constexpr int kDmaLdsBytes = 2 * kDmaStageBytes;         // 128 KB
typedef __attribute__((address_space(3))) void lds_void;
// The large-tile kernel's scales go through LDS as well, after the codes: a
// period of 4 stages (1024 K; 2 stages with blocks of 16) takes 32 scale
// bytes of each of the tile's 256 A rows and 256 B rows, 16 KB, in two
// buffers (160 KB of LDS in all).
constexpr int kScalePeriodBytes = 16 * 1024;
constexpr int kScaleLdsOffset = kDmaLdsBytes;
constexpr int kBigLdsBytes = kDmaLdsBytes + 2 * kScalePeriodBytes;

// STAGE16: 16-bit output with beta == 0, converted while staged (one pass).
// It is a template parameter rather than a branch on beta so that each
// instantiation holds only one epilogue: with both, the 256 live accumulators
// at the branch spilled to scratch.  SUB: E8M0 scale blocks per 32 K values
// (1: MXFP4, 2: blocks of 16).
template <int OUT, bool STAGE16, int SUB>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp4_big_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
    static_assert(SUB == 1 || SUB == 2 || SUB == 4, "blocks of 32, 16 or 8 K values");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kBigLdsBytes];

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
    const int nsb = (K >> 5) * SUB;  // scale bytes per row
    const int nst = K >> 8;          // K is a multiple of 256
    const int last = nst - 1;

    // Direct loads: instruction i of wave w fills LDS rows 32 i + 8 w .. + 7 of
    // one operand (1 KB, 16 bytes per lane in lane order); lane l takes row
    // 8 w + l / 8 (+ 32 i) and the global chunk that belongs at position l % 8.
    // The row is part of the range-checked VGPR offset (rows past the matrix
    // edge load zeros); the scalar offset carries only the stage's K offset.
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A), 0, M * kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B), 0, N * kbytes, 0x00020000);
    const int drow = 8 * wave + (lane >> 3);
    const int dchunk = (lane & 7) ^ ((drow >> 1) & 7);
    const uint32_t dma_a = static_cast<uint32_t>(m0 + drow) * kbytes + dchunk * 16;
    const uint32_t dma_b = static_cast<uint32_t>(n0 + drow) * kbytes + dchunk * 16;
    const uint32_t row_step = 32u * static_cast<uint32_t>(kbytes);
    // direct load j (0..15) of a stage: A for even j, B for odd j, rows 32 (j / 2) + ...
    auto dma_one = [&](auto J, int stage, int buf) {
        constexpr int j = J;
        constexpr int i = j >> 1;
        const int so = min(stage, last) * 128;
        if constexpr ((j & 1) == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs_a, (lds_void*)(lds + buf * kDmaStageBytes + (32 * i + 8 * wave) * kDmaRowBytes), 16,
                dma_a + i * row_step, so, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs_b, (lds_void*)(lds + buf * kDmaStageBytes + kDmaOperandBytes +
                                  (32 * i + 8 * wave) * kDmaRowBytes), 16,
                dma_b + i * row_step, so, 0, 0);
    };
    auto dma_stage = [&](int stage, int buf) {
        static_for<16>([&](auto J) { dma_one(J, stage, buf); });
    };

    // Fragment reads: lane (frag_row r, half h) reads chunk 2 ks + h of rows
    // wm*128 + 32 t + r (A) and wn*128 + 32 t + r (B); t is an immediate offset.
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    const int sw = (frag_row >> 1) & 7;
    uint32_t rd_a[2][4], rd_b[2][4];
#pragma unroll
    for (int bf = 0; bf < 2; ++bf)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint32_t pos = static_cast<uint32_t>(((2 * ks + half) ^ sw) * 16);
            rd_a[bf][ks] = lds0 + bf * kDmaStageBytes + (wm * 128 + frag_row) * kDmaRowBytes + pos;
            rd_b[bf][ks] = lds0 + bf * kDmaStageBytes + kDmaOperandBytes +
                           (wn * 128 + frag_row) * kDmaRowBytes + pos;
        }

    // Scales: this lane feeds rows wm*128 + 32 t + frag_row of A and
    // wn*128 + 32 t + frag_row of B; a stage covers 8 SUB scale blocks (bytes)
    // per row.  A scale row of K / 32 SUB bytes holds a whole 16-byte load
    // only every few rows, and a load into registers of one lane's bytes
    // touches 32 rows (32 cache lines) per instruction, which holds the single
    // wave per SIMD back for long.  So the scales are staged in LDS by direct
    // loads of 32 rows x 32 bytes (a period of 4 / SUB stages), 4 per wave and
    // period, a period ahead of use, and read with ds_read_b64 (ds_read_b128
    // for blocks of 16).  Load j (0..15) of a period covers operand j / 8 (A,
    // then B), rows 32 (j % 8) .. + 31 of the tile; lane l brings 16 bytes,
    // half l / 32 of the period's 32 bytes of row l % 32, and lands at
    // (l / 32) * 512 + (l % 32) * 16 of the load's 1 KB.  Offsets are
    // range-checked (VGPR offset only): rows past M or N and bytes past the
    // scale array read as zero, bytes past a row's end read the next row and
    // are never used.
    constexpr int kPeriod = 4 / SUB;     // stages per scale period
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sA), 0, M * nsb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sB), 0, N * nsb, 0x00020000);
    const uint32_t srow_step = 32u * static_cast<uint32_t>(nsb);
    const int lastp = (nst - 1) / kPeriod;
    // this wave's loads q = 0..3 of a period are j = 4 wave + q: operand
    // wave / 2, rows 128 (wave % 2) + 32 q + lane % 32
    const uint32_t sdma = static_cast<uint32_t>((wave < 2 ? m0 : n0) + 128 * (wave & 1) + (lane & 31)) * nsb +
                          (lane >> 5) * 16;
    auto scale_dma = [&](int period, int q) {
        const uint32_t vo = sdma + q * srow_step + min(period, lastp) * 32;
        lds_void* dst = (lds_void*)(lds + kScaleLdsOffset + (period & 1) * kScalePeriodBytes +
                                    (4 * wave + q) * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wave < 2 ? rs_sa : rs_sb, dst, 16, vo, 0, 0, 0);
    };
    // a stage's scale bytes of a row within the period's buffers: 8 (16) bytes
    // at the stage's byte offset 8 SUB (stage % period) of the row's 32
    auto scale_stage_offset = [&](int stage) -> uint32_t {
        if constexpr (SUB == 1)
            return ((stage >> 2) & 1) * kScalePeriodBytes + ((stage >> 1) & 1) * 512 + (stage & 1) * 8;
        else
            return ((stage >> 1) & 1) * kScalePeriodBytes + (stage & 1) * 512;
    };
    // reads of a stage's scales: A tile t is load j = 4 wm + t, B tile t is
    // j = 8 + 4 wn + t; the stage's offset is added per stage, t is an
    // immediate offset
    const uint32_t srd_a = lds0 + kScaleLdsOffset + (4 * wm) * 1024 + frag_row * 16;
    const uint32_t srd_b = lds0 + kScaleLdsOffset + (8 + 4 * wn) * 1024 + frag_row * 16;
    const uint32_t perm_sel = SUB == 1 ? 0x06040200u + 0x01010101u * static_cast<uint32_t>(half)
                                       : 0x05010400u + 0x02020202u * static_cast<uint32_t>(half);
    // Blocks of 8: a stage is one period, and K step ks of lane half h needs
    // the 4 scale bytes of blocks 8 ks + 4 h .. + 3, which are dword 2 ks + h of
    // the row's 32 bytes: one ds_read_b32 per tile and step, byte q selected
    // by the MFMA's op_sel for block q of the lane's 32 values.  Offsets: the
    // stage's buffer (s % 2) 16384, (ks / 2) 512 + (ks % 2) 8, tile t 1024.
    const uint32_t srd4_a = srd_a + 4 * half, srd4_b = srd_b + 4 * half;
    uint32_t ssa[2][4], ssb[2][4];   // [set][tile]
    auto read_step_scales = [&](auto BUF, auto KS, int set, auto T) {
        constexpr int off = BUF * kScalePeriodBytes + (KS >> 1) * 512 + (KS & 1) * 8 + T * 1024;
        lds_read4<off>(ssa[set][T], srd4_a);
        lds_read4<off>(ssb[set][T], srd4_b);
    };
    using SV = std::conditional_t<SUB == 1, u32x2, u32x4>;
    SV nsa[4], nsb4[4];
    auto read_sv = [&](SV& v, uint32_t addr, auto OFF) {
        if constexpr (SUB == 1)
            lds_read8<OFF>(v, addr);
        else
            lds_read16<OFF>(v, addr);
    };
    auto read_scales = [&](int stage) {
        const uint32_t so = scale_stage_offset(stage);
        const uint32_t ra = srd_a + so, rb = srd_b + so;
        static_for<4>([&](auto T) {
            constexpr int t = T;
            read_sv(nsa[t], ra, std::integral_constant<int, t * 1024>{});
            read_sv(nsb4[t], rb, std::integral_constant<int, t * 1024>{});
        });
    };
    // scale read T (0..7: A tile T / 2 for even T, B tile T / 2 for odd T) of a stage
    auto read_scale_one = [&](uint32_t ra, uint32_t rb, auto T) {
        constexpr int t = T;
        if constexpr (t & 1)
            read_sv(nsb4[t >> 1], rb, std::integral_constant<int, (t >> 1) * 1024>{});
        else
            read_sv(nsa[t >> 1], ra, std::integral_constant<int, (t >> 1) * 1024>{});
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    // Fragments of one K step: B (x) and A (y) 16-byte chunks.  With blocks
    // of 16 or 8 each MFMA gets a copy of the A chunk with one block's dwords
    // kept and the others zeroed (built by the compiler from the whole chunk;
    // reading the halves separately into zero-padded registers measured 1%
    // slower and conflicted in LDS).
    struct Frag { u32x4 x[4], y[4]; };
    Frag fr[2];
    // A fragment T of a K step into g from LDS address addr (+ the tile's offset)
    auto read_y = [&](Frag& g, uint32_t addr, auto T) {
        constexpr int t = T;
        lds_read16<t * 32 * kDmaRowBytes>(g.y[t], addr);
    };

    // Prologue: stage 0 into buffer 0, the first period's scales and the
    // first half of stage 1 (loads 0..7; stage 0's step 0 issues the rest)
    // into buffer 1 all in flight before the first wait (vmcnt counts in issue
    // order: stage 0 and the scales are in once at most stage 1's 8 direct
    // loads are outstanding), then stage 0's first fragments and scales into
    // registers.
    dma_stage(0, 0);
    static_for<4>([&](auto q) { scale_dma(0, q); });
    static_for<8>([&](auto J) { dma_one(J, 1, 1); });
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    lds_wait_barrier();
    static_for<4>([&](auto t) {
        lds_read16<t * 32 * kDmaRowBytes>(fr[0].x[t], rd_b[0][0]);
        read_y(fr[0], rd_a[0][0], t);
    });
    if constexpr (SUB == 4)
        static_for<4>([&](auto t) {
            read_step_scales(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, 0, t);
        });
    else
        read_scales(0);

    // Stage s uses buffer s % 2.  The loop runs pairs of stages so that the
    // buffer, and with it every LDS address of the stage, is a compile-time
    // choice (run-time selects had kept both buffers' read addresses live:
    // 128 VGPRs instead of 212, and 2-4% faster).
    auto run_stage = [&](int s, auto CB) {
        constexpr int cb = CB;
        // this stage's scales and first fragments were read during the last
        // stage's step 3 (or the prologue)
        lds_wait();
        uint32_t wa[4], wb[4], wah[SUB == 2 ? 4 : 1], wbh[SUB == 2 ? 4 : 1];
        if constexpr (SUB == 4) {
            // read one K step ahead instead
        } else if constexpr (SUB == 1) {
            gather_scales(wa[0], wa[1], wa[2], wa[3], nsa[0], nsa[1], nsa[2], nsa[3], perm_sel);
            gather_scales(wb[0], wb[1], wb[2], wb[3], nsb4[0], nsb4[1], nsb4[2], nsb4[3], perm_sel);
        } else {
            static_for<4>([&](auto T) {
                constexpr int t = T;
                gather_scales16(wa[t], wah[t], nsa[t], perm_sel);
                gather_scales16(wb[t], wbh[t], nsb4[t], perm_sel);
            });
        }
        // stage s + 1's scale reads (step 3)
        const uint32_t sso = scale_stage_offset(s + 1);
        const uint32_t sra = srd_a + sso, srb = srd_b + sso;

        // One K step (64 K values): 16 MFMAs (32 with blocks of 16, 64 with
        // blocks of 8) on fragment set KS & 1 with the fragment reads (and,
        // for blocks of 8, the scale reads) of the next step in their shadows.  Step 3 follows the barrier that publishes stage
        // s + 1: it reads that stage's first fragments and scales and issues
        // the first 8 direct loads of stage s + 2 into this stage's buffer,
        // which no wave reads any more; step 0 of the next stage issues the
        // other 8, and this wave's share of the next period's scales.  With
        // one wave per SIMD, a memory instruction between two MFMAs holds the
        // matrix core until it issues, and the loads back up once they ask
        // more of L2 than it delivers to a CU: one direct load every 32
        // MFMA-cycles, over two steps, keeps a stage's 64 KB under that rate
        // (16 loads in one step measured 5-7% slower).
        auto kstep = [&](auto KS) {
            constexpr int ks = KS;
            constexpr int nks = (ks + 1) & 3;
            constexpr int NM = 16 * SUB;          // MFMAs of the step
            constexpr int LD = 2 * SUB;           // MFMAs per direct load
            const Frag& f = fr[ks & 1];
            Frag& g = fr[(ks + 1) & 1];
            const int rb = ks == 3 ? cb ^ 1 : cb;
            const uint32_t ra_addr = rb ? rd_a[1][nks] : rd_a[0][nks];
            const uint32_t rb_addr = rb ? rd_b[1][nks] : rd_b[0][nks];
            static_for<NM>([&](auto J) {
                constexpr int j = J;
                constexpr int jj = j & 15;
                constexpr int ti = jj >> 2, tj = jj & 3;
                if constexpr (SUB == 1) {
                    mfma_fp4_sel<ks>(acc[ti][tj], f.x[ti], f.y[tj], wb[ti], wa[tj]);
                } else if constexpr (SUB == 4) {
                    // block q = j / 16 of each lane's 32 values: dword q of A kept
                    constexpr int q = j >> 4;
                    u32x4 yq = {0u, 0u, 0u, 0u};
                    yq[q] = f.y[tj][q];
                    mfma_fp4_sel_w<q>(acc[ti][tj], f.x[ti], yq, ssb[ks & 1][ti], ssa[ks & 1][tj]);
                } else {
                    // block j / 16 of each lane's 32 values: dwords 2 (j / 16), + 1 of A kept
                    constexpr int q = j >> 4;
                    u32x4 yq = {0u, 0u, 0u, 0u};
                    yq[2 * q] = f.y[tj][2 * q];
                    yq[2 * q + 1] = f.y[tj][2 * q + 1];
                    if constexpr (q == 0)
                        mfma_fp4_sel_w<ks>(acc[ti][tj], f.x[ti], yq, wb[ti], wa[tj]);
                    else
                        mfma_fp4_sel_w<ks>(acc[ti][tj], f.x[ti], yq, wbh[ti], wah[tj]);
                }
                // the next step's fragment reads, then (step 3) the next
                // stage's scale reads, one after each MFMA
                if constexpr (j < 8) {
                    constexpr int t = j >> 1;
                    if constexpr (j & 1)
                        read_y(g, ra_addr, std::integral_constant<int, t>{});
                    else
                        lds_read16<t * 32 * kDmaRowBytes>(g.x[t], rb_addr);
                } else if constexpr (SUB == 4 && j < 12) {
                    // the next step's scales: its stage's buffer
                    read_step_scales(std::integral_constant<int, (ks == 3 ? cb ^ 1 : cb)>{},
                                     std::integral_constant<int, nks>{}, (ks + 1) & 1,
                                     std::integral_constant<int, j - 8>{});
                } else if constexpr (SUB != 4 && ks == 3 && j < 16) {
                    read_scale_one(sra, srb, std::integral_constant<int, j - 8>{});
                }
                if constexpr (ks == 0 && j % 8 == 0 && j >= 8 && j < 8 + 8 * SUB)
                    scale_dma((s / kPeriod) + 1, SUB * (s % kPeriod) + (j - 8) / 8);
                if constexpr (ks == 3 && j % LD == LD - 1)
                    dma_one(std::integral_constant<int, (j / LD)>{}, s + 2, cb);
                if constexpr (ks == 0 && j % LD == LD - 1)
                    dma_one(std::integral_constant<int, (8 + j / LD)>{}, s + 1, cb ^ 1);
            });
        };
        kstep(std::integral_constant<int, 0>{});
        lds_wait();
        kstep(std::integral_constant<int, 1>{});
        lds_wait();
        kstep(std::integral_constant<int, 2>{});
        // stage s + 1 has landed (its second half was issued in step 0), and
        // so have this stage's scale loads: publish them (the last reads of
        // the scale buffer that the next period's loads refill were waited for
        // before an earlier barrier)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_wait_barrier();
        kstep(std::integral_constant<int, 3>{});
    };
    int s0 = 0;
    for (; s0 + 1 < nst; s0 += 2) {
        run_stage(s0, std::integral_constant<int, 0>{});
        run_stage(s0 + 1, std::integral_constant<int, 1>{});
    }
    if (s0 < nst) run_stage(s0, std::integral_constant<int, 0>{});
    // no direct load may still be writing LDS when the workgroup ends, and no
    // register load may still be in flight when its register is reused: the
    // last stage's scale loads and fragment reads have no consumer, so they
    // are named after the wait to keep their registers
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    asm volatile("" :: "v"(fr[0].x[0]), "v"(fr[0].x[1]), "v"(fr[0].x[2]), "v"(fr[0].x[3]),
                       "v"(fr[0].y[0]), "v"(fr[0].y[1]), "v"(fr[0].y[2]), "v"(fr[0].y[3]));
    asm volatile("" :: "v"(fr[1].x[0]), "v"(fr[1].x[1]), "v"(fr[1].x[2]), "v"(fr[1].x[3]),
                       "v"(fr[1].y[0]), "v"(fr[1].y[1]), "v"(fr[1].y[2]), "v"(fr[1].y[3]));
    if constexpr (SUB == 4)
        asm volatile("" :: "v"(ssa[0][0]), "v"(ssa[0][1]), "v"(ssa[0][2]), "v"(ssa[0][3]),
                           "v"(ssb[0][0]), "v"(ssb[0][1]), "v"(ssb[0][2]), "v"(ssb[0][3]));
    else
        asm volatile("" :: "v"(nsa[0]), "v"(nsa[1]), "v"(nsa[2]), "v"(nsa[3]),
                           "v"(nsb4[0]), "v"(nsb4[1]), "v"(nsb4[2]), "v"(nsb4[3]));
    // MFMA results must settle before the accumulation registers are read.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                   "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]),
                   "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                   "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));

    NoScale none;
    big_tile::epilogue<OUT, STAGE16>(acc, lds, wave, lane, m0, n0, M, N, D, ldd, ep, vec_ok, none);
}

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// Large-tile variant for K a multiple of 32 but not of 256: the same tile and
// MFMAs as gemm_mxfp4_big_kernel, with K staged in a ring of four 128-K
// buffers.  Chunks (32-element blocks) past K load as zero through
// range-checked offsets, and so do their scale bytes (a scale row of K / 32
// bytes need not start on a 4-byte boundary: each row's 8 bytes of a 256-K step
// are cut out of an aligned 12-byte load).  Every load is spread over the K
// steps, at most one memory instruction after each MFMA.  On K a multiple of
// 256 this form measured 10% slower than the two-buffer kernel (8192^3), which
// therefore keeps those.
//
// Ring LDS layout: 4 buffers of 32 KB, each A then B, 256 rows of 64
// bytes (unpadded, so that direct loads can fill them).  Row R keeps its
// 16-byte chunk g at position g ^ ((R >> 2) & 3): the 16 lanes of a
// fragment-read phase (16 consecutive rows, one chunk) then hit 16 distinct
// 4-bank groups.
constexpr int kRingRow = 64;
constexpr int kRingOperand = 256 * kRingRow;           // 16 KB
constexpr int kRingBuffer = 2 * kRingOperand;          // 32 KB
constexpr int kRingLds = 4 * kRingBuffer;              // 128 KB

// STAGE16: 16-bit output with beta == 0, converted while staged (one pass).
// It is a template parameter rather than a branch on beta so that each
// instantiation holds only one epilogue: with both, the 256 live accumulators
// at the branch spilled to scratch.
template <int OUT, bool STAGE16>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp4_ring_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kRingLds];

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
    const int nh = (nkb + 3) >> 2;       // 128-K buffers, the last one partial
    const int nss = (nkb + 7) >> 3;      // 256-K scale steps
    const int nrounds = (nh + 3) >> 2;   // trips around the 4-buffer ring

    // Direct loads: load i (0..3) of wave w fills LDS rows 64 w + 16 i .. + 15
    // of one operand in one buffer (1 KB, 16 bytes per lane in lane order);
    // lane l takes row 64 w + 16 i + l / 4 and the global chunk that belongs
    // at position l % 4, whose swizzle (row >> 2) & 3 = (l >> 4) & 3 is the
    // same for every i and w.  The row is in the range-checked VGPR offset
    // (rows past the matrix edge load zeros), the buffer's K offset in the
    // scalar offset; a chunk past K (block 4 h + chunk >= K / 32) gets an
    // out-of-range VGPR offset.
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A), 0, M * kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B), 0, N * kbytes, 0x00020000);
    const int drow = 64 * wave + (lane >> 2);
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    const uint32_t dma_a = static_cast<uint32_t>(m0 + drow) * kbytes + dchunk * 16;
    const uint32_t dma_b = static_cast<uint32_t>(n0 + drow) * kbytes + dchunk * 16;
    const uint32_t row16 = 16u * static_cast<uint32_t>(kbytes);
    // load I (0..3 A, 4..7 B) of K buffer h into ring buffer BUF
    auto dma_one = [&](auto I, auto BUF, int h) {
        constexpr int q = I;
        constexpr int buf = BUF;
        constexpr int i = q & 3;
        uint32_t oob = 4 * h + dchunk < nkb ? 0u : 0x80000000u;
        asm volatile("" : "+v"(oob));
        const uint32_t vo = ((q < 4 ? dma_a : dma_b) + i * row16) | oob;
        lds_void* dst = (lds_void*)(lds + buf * kRingBuffer + (q < 4 ? 0 : kRingOperand) +
                                    (64 * wave + 16 * i) * kRingRow);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 4 ? rs_a : rs_b, dst, 16, vo, h * kRingRow, 0, 0);
    };

    // Fragment reads: lane (frag_row r, half h) reads chunk 2 q + h of rows
    // wm*128 + 32 t + r (A) and wn*128 + 32 t + r (B) for K step q (0, 1) of
    // a buffer; t and the buffer are immediate offsets from one of two bases
    // (buffers 0, 1 and buffers 2, 3), so that they stay below 64 KB.
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    const int sw = (frag_row >> 2) & 3;
    uint32_t rd_a[2][2], rd_b[2][2];     // [hi][q]
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t pos = static_cast<uint32_t>(((2 * q + half) ^ sw) * 16);
            rd_a[hi][q] = lds0 + hi * 2 * kRingBuffer + (wm * 128 + frag_row) * kRingRow + pos;
            rd_b[hi][q] = lds0 + hi * 2 * kRingBuffer + kRingOperand + (wn * 128 + frag_row) * kRingRow + pos;
        }

    // Scales: this lane feeds rows wm*128 + 32 t + frag_row of A and
    // wn*128 + 32 t + frag_row of B; 256 K cover 8 scale bytes of a row, at
    // byte offset row * K / 32 + 8 S.  The 12 bytes from the dword below it are
    // loaded (the whole offset range-checked: rows past the edge and steps past
    // K read as zero) and the 8 cut out with v_alignbyte; bytes of blocks past
    // K are cleared.
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sA), 0, M * nkb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sB), 0, N * nkb, 0x00020000);
    const uint32_t soff_a = static_cast<uint32_t>(m0 + wm * 128 + frag_row) * nkb;
    const uint32_t soff_b = static_cast<uint32_t>(n0 + wn * 128 + frag_row) * nkb;
    // (the byte shift of row t, (soff + t * srow_step) & 3, is recomputed where
    // it is used rather than kept in registers)
    const uint32_t srow_step = 32u * static_cast<uint32_t>(nkb);
    const uint32_t perm_sel = 0x06040200u + 0x01010101u * static_cast<uint32_t>(half);
    u32x3 nsa[2][4], nsb[2][4];     // [256-K step parity][t]
    auto scale_ld = [](u32x3& dst, uint32_t vo, __amdgpu_buffer_rsrc_t rs) {
        asm volatile("buffer_load_dwordx3 %0, %1, %2, 0 offen" : "=v"(dst) : "v"(vo), "s"(rs) : "memory");
    };
    // the scale load of row t (A for OP 0, B for OP 1) for 256-K step S into set SET
    auto scale_one = [&](auto OP, auto SET, int t, int S) {
        uint32_t vo = ((OP ? soff_b : soff_a) + t * srow_step + S * 8) & ~3u;
        vo = S < nss ? vo : 0x80000000u;
        asm volatile("" : "+v"(vo));
        if constexpr (OP)
            scale_ld(nsb[SET][t], vo, rs_sb);
        else
            scale_ld(nsa[SET][t], vo, rs_sa);
    };
    // the 8 scale bytes of a row out of its 12 loaded bytes
    auto cut8 = [](const u32x3& w, uint32_t sh) {
        return u32x2{__builtin_amdgcn_alignbyte(w.y, w.x, sh), __builtin_amdgcn_alignbyte(w.z, w.y, sh)};
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto scales_all = [&](auto SET, int S) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            scale_one(I0{}, SET, t, S);
            scale_one(I1{}, SET, t, S);
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    struct Frag { u32x4 x[4], y[4]; };
    Frag fr[2];

    // Prologue: buffers 0, 1, 2 and the A half of buffer 3 in flight, with the
    // scales of the first two 256-K steps; then buffer 0's first fragments.
    // (vmcnt counts in issue order: buffer 0 and the first scales are in once
    // at most the 28 loads issued after them are outstanding.)
    static_for<8>([&](auto I) { dma_one(I, I0{}, 0); });
    scales_all(I0{}, 0);
    static_for<8>([&](auto I) { dma_one(I, I1{}, 1); });
    static_for<8>([&](auto I) { dma_one(I, std::integral_constant<int, 2>{}, 2); });
    scales_all(I1{}, 1);
    static_for<4>([&](auto I) { dma_one(I, std::integral_constant<int, 3>{}, 3); });
    asm volatile("s_waitcnt vmcnt(28)" ::: "memory");
    lds_wait_barrier();
    static_for<4>([&](auto t) {
        lds_read16<t * 32 * kRingRow>(fr[0].x[t], rd_b[0][0]);
        lds_read16<t * 32 * kRingRow>(fr[0].y[t], rd_a[0][0]);
    });

    // Round r visits ring buffers 0..3 = K buffers h = 4 r .. 4 r + 3, two K
    // steps each.  In the first K step of buffer h the B half of buffer h + 3
    // is loaded (its ring slot, h - 1's, is free since the barrier inside
    // h - 1), in the second the A half of buffer h + 4 (into h's own slot, free
    // since the barrier just before); each K step also loads two scale rows of
    // the 256-K step two ahead.  Per K step the loads issue in the order 4
    // direct loads, 2 scale loads, so that:
    //  * the barrier inside buffer h (publishing buffer h + 1, whose B half
    //    was issued 4 K steps earlier) may leave 2 + 4 * 6 = 26 loads in flight;
    //  * the scales of a 256-K step, whose last loads were issued in the last
    //    K step two steps back, are in once at most 4 * 6 = 24 are.
    uint32_t wa[4], wb[4];
    for (int r = 0; r < nrounds; ++r) {
        static_for<4>([&](auto BUF) {
            constexpr int b = BUF;
            constexpr int set = b >> 1;          // parity of the 256-K step
            const int h = 4 * r + b;
            if constexpr ((b & 1) == 0) {
                const int S = h >> 1;
                asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
                u32x3 ra[4], rb3[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) { ra[t] = nsa[set][t]; rb3[t] = nsb[set][t]; }
                asm volatile("" : "+v"(ra[0]), "+v"(ra[1]), "+v"(ra[2]), "+v"(ra[3]),
                                  "+v"(rb3[0]), "+v"(rb3[1]), "+v"(rb3[2]), "+v"(rb3[3]));
                // bytes of blocks at or past K / 32 (the last step's) are cleared
                const int vb = nkb - 8 * S;
                const uint32_t mlo = vb >= 4 ? 0xFFFFFFFFu : vb <= 0 ? 0u : (1u << (8 * vb)) - 1u;
                const uint32_t mhi = vb >= 8 ? 0xFFFFFFFFu : vb <= 4 ? 0u : (1u << (8 * (vb - 4))) - 1u;
                u32x2 ca[4], cbv[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    ca[t] = cut8(ra[t], (soff_a + t * srow_step) & 3u);
                    cbv[t] = cut8(rb3[t], (soff_b + t * srow_step) & 3u);
                    ca[t].x &= mlo; ca[t].y &= mhi;
                    cbv[t].x &= mlo; cbv[t].y &= mhi;
                }
                gather_scales(wa[0], wa[1], wa[2], wa[3], ca[0], ca[1], ca[2], ca[3], perm_sel);
                gather_scales(wb[0], wb[1], wb[2], wb[3], cbv[0], cbv[1], cbv[2], cbv[3], perm_sel);
            }
            static_for<2>([&](auto Q) {
                constexpr int q = Q;
                constexpr int k = 2 * b + q;             // K step within the round
                constexpr int ks = 2 * (b & 1) + q;      // K step within the 256-K step
                constexpr int nb = q == 0 ? b : (b + 1) & 3;
                constexpr int nq = q ^ 1;
                const Frag& f = fr[k & 1];
                Frag& g = fr[(k + 1) & 1];
                const uint32_t ra = rd_a[nb >> 1][nq];
                const uint32_t rb = rd_b[nb >> 1][nq];
                constexpr int boff = (nb & 1) * kRingBuffer;
                if constexpr (q == 0) lds_wait();
                static_for<16>([&](auto J) {
                    constexpr int j = J;
                    constexpr int ti = j >> 2, tj = j & 3;
                    mfma_fp4_sel<ks>(acc[ti][tj], f.x[ti], f.y[tj], wb[ti], wa[tj]);
                    if constexpr ((j & 1) == 0) {
                        constexpr int t = j >> 2;
                        if constexpr ((j & 2) == 0)
                            lds_read16<boff + t * 32 * kRingRow>(g.x[t], rb);
                        else
                            lds_read16<boff + t * 32 * kRingRow>(g.y[t], ra);
                    } else if constexpr (j < 8) {
                        constexpr int i = j >> 1;
                        if constexpr (q == 0)
                            dma_one(std::integral_constant<int, 4 + i>{}, std::integral_constant<int, (b + 3) & 3>{}, h + 3);
                        else
                            dma_one(std::integral_constant<int, i>{}, std::integral_constant<int, b>{}, h + 4);
                    } else if constexpr (j == 9) {
                        scale_one(I0{}, std::integral_constant<int, set>{}, ks, (h >> 1) + 2);
                    } else if constexpr (j == 11) {
                        scale_one(I1{}, std::integral_constant<int, set>{}, ks, (h >> 1) + 2);
                    }
                });
                if constexpr (q == 0) {
                    // buffer h + 1 has landed; publish it (and free buffer h)
                    asm volatile("s_waitcnt vmcnt(26)" ::: "memory");
                    lds_wait_barrier();
                }
            });
        });
    }
    // no direct load may still be writing LDS when the workgroup ends, and no
    // register load may still be in flight when its register is reused: the
    // last K step's fragment reads and the scale loads past the end have no
    // consumer, so they are named after the wait to keep their registers
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    asm volatile("" :: "v"(fr[0].x[0]), "v"(fr[0].x[1]), "v"(fr[0].x[2]), "v"(fr[0].x[3]),
                       "v"(fr[0].y[0]), "v"(fr[0].y[1]), "v"(fr[0].y[2]), "v"(fr[0].y[3]));
    asm volatile("" :: "v"(fr[1].x[0]), "v"(fr[1].x[1]), "v"(fr[1].x[2]), "v"(fr[1].x[3]),
                       "v"(fr[1].y[0]), "v"(fr[1].y[1]), "v"(fr[1].y[2]), "v"(fr[1].y[3]));
    asm volatile("" :: "v"(nsa[0][0]), "v"(nsa[0][1]), "v"(nsa[0][2]), "v"(nsa[0][3]),
                       "v"(nsa[1][0]), "v"(nsa[1][1]), "v"(nsa[1][2]), "v"(nsa[1][3]));
    asm volatile("" :: "v"(nsb[0][0]), "v"(nsb[0][1]), "v"(nsb[0][2]), "v"(nsb[0][3]),
                       "v"(nsb[1][0]), "v"(nsb[1][1]), "v"(nsb[1][2]), "v"(nsb[1][3]));
    // MFMA results must settle before the accumulation registers are read.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                   "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]),
                   "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                   "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));

    NoScale none;
    big_tile::epilogue<OUT, STAGE16>(acc, lds, wave, lane, m0, n0, M, N, D, ldd, ep, vec_ok, none);
}

// Skinny form (up to kSkinnyMaxM rows), as the FP8 one: one workgroup per
// 32 x 32 output tile, the four waves split K into contiguous ranges of
// 8-block chunks, codes are loaded as whole 128-byte row segments and staged
// through LDS into the MFMA layout (lane (r, h) takes the 16 packed bytes and
// the E8M0 byte of block 2 s + h of row r for 64-K step s), and the partial
// sums are added in a fixed order through LDS.  Blocks past K or past the
// wave's range read as zero codes with a zero scale byte (2^-127), which
// contribute nothing.  SUB as for the other kernels: blocks of 16 or 8 take
// one MFMA per block, with the lane's other A values zeroed, and a 2- or
// 4-byte scale load.
constexpr int kSkinnyDepth = 2;              // chunks of 8 blocks in flight per wave
constexpr int kSkinnyWaves = 4;              // waves per workgroup, splitting K
constexpr int64_t kSkinnyMaxM = 64;
constexpr int64_t kSkinnyMaxTiles = 32;      // 128 x 128 tiles below which the skinny form is used too

template <int OUT, int SUB = 1>
__global__ __launch_bounds__(64 * kSkinnyWaves, 8 / kSkinnyWaves) void gemm_mxfp4_skinny_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
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
    const int kbytes = K >> 1, nkb = K >> 5, nsb = nkb * SUB;   // 32-wide blocks, scale bytes per row
    // K is split into chunks of 8 blocks (128 bytes of each row); each wave
    // takes a contiguous range of chunks
    const int nch = (nkb + 7) >> 3;
    const int cper = (nch + kSkinnyWaves - 1) / kSkinnyWaves;
    const int c0 = min(wave * cper, nch), c1 = min(c0 + cper, nch);

    const int rows_a = min(32, M - m0), rows_b = min(32, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A) + static_cast<int64_t>(m0) * kbytes, 0, rows_a * kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B) + static_cast<int64_t>(n0) * kbytes, 0, rows_b * kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sA) + static_cast<int64_t>(m0) * nsb, 0, rows_a * nsb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sB) + static_cast<int64_t>(n0) * nsb, 0, rows_b * nsb, 0x00020000);
    const int r = lane & 31, h = lane >> 5;
    constexpr uint32_t kOut = 0x80000000u;
    // Code loads read whole 128-byte row segments: lane l takes 16-byte piece
    // l & 7 (block 8 c + (l & 7)) of row (l >> 3) + 8 i.  The wave stages the
    // chunk in its own LDS area (piece g of row R at g ^ (R & 7)) and reads the
    // fragments back: for step s of the chunk lane (r, h) takes block
    // 8 c + 2 s + h of row r, with its E8M0 byte.
    const int lr = lane >> 3, lg = lane & 7;
    uint8_t* st_a = stage[wave][0];
    uint8_t* st_b = stage[wave][1];
    uint4 ga[kSkinnyDepth][4], gb[kSkinnyDepth][4];
    uint32_t ea[kSkinnyDepth][4], eb[kSkinnyDepth][4];
    auto fetch = [&](auto SLOT, int c) {
        constexpr int j = SLOT;
        const bool cok = c < c1;
        const bool ok = cok && 8 * c + lg < nkb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = ok ? static_cast<uint32_t>((lr + 8 * i) * kbytes + 128 * c + 16 * lg) : kOut;
            const auto wa = __builtin_amdgcn_raw_buffer_load_b128(rs_a, static_cast<int>(o), 0, 0);
            const auto wb = __builtin_amdgcn_raw_buffer_load_b128(rs_b, static_cast<int>(o), 0, 0);
            ga[j][i] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
            gb[j][i] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int blk = 8 * c + 2 * st + h;
            const uint32_t os = cok && blk < nkb ? static_cast<uint32_t>((r * nkb + blk) * SUB) : kOut;
            if constexpr (SUB == 1) {
                ea[j][st] = __builtin_amdgcn_raw_buffer_load_b8(rs_sa, static_cast<int>(os), 0, 0);
                eb[j][st] = __builtin_amdgcn_raw_buffer_load_b8(rs_sb, static_cast<int>(os), 0, 0);
            } else if constexpr (SUB == 2) {
                ea[j][st] = __builtin_amdgcn_raw_buffer_load_b16(rs_sa, static_cast<int>(os), 0, 0);
                eb[j][st] = __builtin_amdgcn_raw_buffer_load_b16(rs_sb, static_cast<int>(os), 0, 0);
            } else {
                ea[j][st] = __builtin_amdgcn_raw_buffer_load_b32(rs_sa, static_cast<int>(os), 0, 0);
                eb[j][st] = __builtin_amdgcn_raw_buffer_load_b32(rs_sb, static_cast<int>(os), 0, 0);
            }
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
                *reinterpret_cast<uint4*>(st_a + pos) = ga[j][i];
                *reinterpret_cast<uint4*>(st_b + pos) = gb[j][i];
            }
            uint32_t sa4[4], sb4[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                sa4[st] = ea[j][st];
                sb4[st] = eb[j][st];
            }
            fetch(J, c + j + kSkinnyDepth);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int pos = r * 128 + 16 * ((2 * st + h) ^ (r & 7));
                const uint4 xa = *reinterpret_cast<const uint4*>(st_a + pos);
                const uint4 xb = *reinterpret_cast<const uint4*>(st_b + pos);
                // B rows are the row operand
                if constexpr (SUB == 1) {
                    acc = mfma_fp4(xb, xa, sb4[st], sa4[st], acc);
                } else {
                    static_for<SUB>([&](auto Q) {
                        constexpr int q = Q;
                        const uint32_t w[4] = {xa.x, xa.y, xa.z, xa.w};
                        uint32_t z[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) z[i] = (i * SUB / 4 == q) ? w[i] : 0u;
                        acc = mfma_fp4<q>(xb, make_uint4(z[0], z[1], z[2], z[3]), sb4[st], sa4[st], acc);
                    });
                }
            }
        });
    }
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w) {
        const v16f q = part[w][lane];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += q[e];
    }
    // lane (r, h) holds row m0 + r, columns n0 + 8 q + 4 h + e in acc[4 q + e]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float a4[4] = {acc[4 * q + 0], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        finish_row_chunk<OUT, 4>(D, ldd, ep, m0 + r, n0 + 8 * q + 4 * h, M, N, vec_ok, a4);
    }
}

template <int OUT>
hipError_t launch_out(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* a_scales,
                      const uint8_t* b, const uint8_t* b_scales, void* d, int64_t ldd,
                      const Epilogue& ep, hipStream_t stream) {
    const int vec = vec16_ok(OUT, d, ldd, ep);
    if (M <= kSkinnyMaxM || ((M + 127) / 128) * ((N + 127) / 128) < kSkinnyMaxTiles) {
        const int tm = static_cast<int>((M + 31) / 32), tn = static_cast<int>((N + 31) / 32);
        const uint32_t wgs = static_cast<uint32_t>((tn + 7) / 8) * 8u * static_cast<uint32_t>(tm);
        hipLaunchKernelGGL(gemm_mxfp4_skinny_kernel<OUT>, dim3(wgs), dim3(64 * kSkinnyWaves), 0, stream,
                           static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, a_scales, b,
                           b_scales, d, ldd, ep, tm, tn, vec);
        return hipGetLastError();
    }
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    const bool fits32 = M * (K / 2) < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31);
    if (big_tiles >= kBigTileThreshold && fits32) {
        const int tm = static_cast<int>((M + 255) / 256), tn = static_cast<int>((N + 255) / 256);
        const dim3 g(static_cast<uint32_t>(tm) * static_cast<uint32_t>(tn));
        const int Mi = static_cast<int>(M), Ni = static_cast<int>(N), Ki = static_cast<int>(K);
        // K a multiple of 256: the two-buffer kernel; other K: the ring of 128-K buffers
        const bool two = K % 256 == 0;
        if constexpr (OUT != BSFP8_OUT_F32) {
            if (ep.beta == 0.0f) {
                if (two)
                    hipLaunchKernelGGL((gemm_mxfp4_big_kernel<OUT, true, 1>), g, dim3(kThreads), 0, stream,
                                       Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
                else
                    hipLaunchKernelGGL((gemm_mxfp4_ring_kernel<OUT, true>), g, dim3(kThreads), 0, stream,
                                       Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
                return hipGetLastError();
            }
        }
        if (two)
            hipLaunchKernelGGL((gemm_mxfp4_big_kernel<OUT, false, 1>), g, dim3(kThreads), 0, stream,
                               Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
        else
            hipLaunchKernelGGL((gemm_mxfp4_ring_kernel<OUT, false>), g, dim3(kThreads), 0, stream,
                               Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
        return hipGetLastError();
    }
    const int tiles_m = static_cast<int>((M + BM - 1) / BM);
    const int tiles_n = static_cast<int>((N + BN - 1) / BN);
    const dim3 grid(static_cast<uint32_t>(tiles_m) * static_cast<uint32_t>(tiles_n));
    hipLaunchKernelGGL(gemm_mxfp4_kernel<OUT>, grid, dim3(kThreads), 0, stream,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, a_scales,
                       b, b_scales, d, ldd, ep, tiles_m, tiles_n, vec);
    return hipGetLastError();
}

template <int OUT, int SUB>
hipError_t launch_out_sub(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* a_scales,
                          const uint8_t* b, const uint8_t* b_scales, void* d, int64_t ldd,
                          const Epilogue& ep, hipStream_t stream) {
    const int vec = vec16_ok(OUT, d, ldd, ep);
    const int tm = static_cast<int>((M + 255) / 256), tn = static_cast<int>((N + 255) / 256);
    const dim3 g(static_cast<uint32_t>(tm) * static_cast<uint32_t>(tn));
    const int Mi = static_cast<int>(M), Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    if constexpr (OUT != BSFP8_OUT_F32) {
        if (ep.beta == 0.0f) {
            hipLaunchKernelGGL((gemm_mxfp4_big_kernel<OUT, true, SUB>), g, dim3(kThreads), 0, stream,
                               Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_mxfp4_big_kernel<OUT, false, SUB>), g, dim3(kThreads), 0, stream,
                       Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
    return hipGetLastError();
}

template <int OUT, int SUB>
hipError_t launch_tile_sub(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* a_scales,
                           const uint8_t* b, const uint8_t* b_scales, void* d, int64_t ldd,
                           const Epilogue& ep, hipStream_t stream) {
    const int tiles_m = static_cast<int>((M + BM - 1) / BM);
    const int tiles_n = static_cast<int>((N + BN - 1) / BN);
    const dim3 grid(static_cast<uint32_t>(tiles_m) * static_cast<uint32_t>(tiles_n));
    hipLaunchKernelGGL((gemm_mxfp4_kernel<OUT, SUB>), grid, dim3(kThreads), 0, stream,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, a_scales,
                       b, b_scales, d, ldd, ep, tiles_m, tiles_n, vec16_ok(OUT, d, ldd, ep));
    return hipGetLastError();
}

template <int SUB>
hipError_t launch_sub(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* a_scales,
                      const uint8_t* b, const uint8_t* b_scales, int out, void* d, int64_t ldd,
                      const Epilogue& ep, hipStream_t stream) {
    if (M <= kSkinnyMaxM || ((M + 127) / 128) * ((N + 127) / 128) < kSkinnyMaxTiles) {
        const int tm = static_cast<int>((M + 31) / 32), tn = static_cast<int>((N + 31) / 32);
        const uint32_t wgs = static_cast<uint32_t>((tn + 7) / 8) * 8u * static_cast<uint32_t>(tm);
        const int vec = vec16_ok(out, d, ldd, ep);
        const int Mi = static_cast<int>(M), Ni = static_cast<int>(N), Ki = static_cast<int>(K);
        if (out == BSFP8_OUT_F32)
            hipLaunchKernelGGL((gemm_mxfp4_skinny_kernel<BSFP8_OUT_F32, SUB>), dim3(wgs), dim3(64 * kSkinnyWaves),
                               0, stream, Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
        else if (out == BSFP8_OUT_BF16)
            hipLaunchKernelGGL((gemm_mxfp4_skinny_kernel<BSFP8_OUT_BF16, SUB>), dim3(wgs), dim3(64 * kSkinnyWaves),
                               0, stream, Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
        else
            hipLaunchKernelGGL((gemm_mxfp4_skinny_kernel<BSFP8_OUT_F16, SUB>), dim3(wgs), dim3(64 * kSkinnyWaves),
                               0, stream, Mi, Ni, Ki, a, a_scales, b, b_scales, d, ldd, ep, tm, tn, vec);
        return hipGetLastError();
    }
    if (!mx_fp4_big_applies(M, N, K)) {
        if (out == BSFP8_OUT_F32)
            return launch_tile_sub<BSFP8_OUT_F32, SUB>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
        if (out == BSFP8_OUT_BF16)
            return launch_tile_sub<BSFP8_OUT_BF16, SUB>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
        return launch_tile_sub<BSFP8_OUT_F16, SUB>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
    }
    if (out == BSFP8_OUT_F32)
        return launch_out_sub<BSFP8_OUT_F32, SUB>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
    if (out == BSFP8_OUT_BF16)
        return launch_out_sub<BSFP8_OUT_BF16, SUB>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
    return launch_out_sub<BSFP8_OUT_F16, SUB>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
}

}  // namespace

bool mx_fp4_big_applies(int64_t M, int64_t N, int64_t K) {
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    return K % 256 == 0 && M > kSkinnyMaxM && big_tiles >= kBigTileThreshold &&
           M * (K / 2) < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31);
}

hipError_t launch_gemm_mx_fp4(int64_t M, int64_t N, int64_t K, int block, const uint8_t* a,
                                  const uint8_t* a_scales, const uint8_t* b, const uint8_t* b_scales,
                                  int out, void* d, int64_t ldd, const Epilogue& ep, hipStream_t stream) {
    if (block == 16) return launch_sub<2>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, stream);
    return launch_sub<4>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, stream);
}

hipError_t launch_gemm_mxfp4(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                             const uint8_t* a_scales, const uint8_t* b, const uint8_t* b_scales,
                             int out, void* d, int64_t ldd, const Epilogue& ep,
                             hipStream_t stream) {
    if (out == BSFP8_OUT_F32)
        return launch_out<BSFP8_OUT_F32>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
    if (out == BSFP8_OUT_BF16)
        return launch_out<BSFP8_OUT_BF16>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
    return launch_out<BSFP8_OUT_F16>(M, N, K, a, a_scales, b, b_scales, d, ldd, ep, stream);
}

}  // namespace bsfp8
