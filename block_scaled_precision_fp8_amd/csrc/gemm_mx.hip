// gemm_mx.hip -- GEMM of E2M1 operands with blocks of 16 or 8 elements or
// FP16 / BF16 block scales ("Rubin FP4 GEMM deep dive", sections 5.3 and
// 3.2), for gfx950.
//
// D[m][n] = sum_k a[m][k] b[n][k],  a = code * scale(m, k / BLOCK), likewise b.
//
// The block-scaled matrix instructions apply one E8M0 scale per 32 K values
// of a lane, so they cannot take these operands.  Here each operand is
// dequantised exactly while it is staged into LDS, and the product runs on
// v_mfma_f32_32x32x16_bf16 (24 fraction bits kept per group of 8 products):
//  * E8M0 scales: code * 2^e has at most two significant bits, an exact bf16;
//  * FP16 / BF16 scales: code * s has at most 13 significant bits; it is
//    split exactly into hi = bf16(code * s) and lo = code * s - hi (at most 5
//    bits), and D accumulates the products hi*hi, hi*lo, lo*hi and, for FP32
//    output, lo*lo (at most 2^-16 of hi*hi, far inside the 2^-7 tolerance of
//    16-bit outputs, which leave it out).
// No per-block promotion is needed: the scales are inside the operands.
//
// Tiling: 128 x 128 output tile per workgroup, 4 waves of 64 x 64 (2 x 2 MFMA
// tiles of 32 x 32), stages of 64 K, two LDS buffers.  Each thread stages one
// row of A and of B, 32 K values (16 bytes of codes) per stage: it loads
// the codes and their block scales for the next stage while the current one
// is multiplied, then dequantises them into the other buffer.  LDS rows are
// 128 bytes of bf16 (64 K), 16-byte chunk c of row R stored at
// c ^ ((R >> 1) & 7): the 16 rows of a 16-lane read phase then cover all 16
// groups of 4 banks.
#include "big_tile.h"

#include <type_traits>
#include <utility>

namespace bsfp8 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int SK = 64;                         // K per stage
constexpr int kRow = SK * 2;                   // bytes per LDS row (bf16)
constexpr int kPart = 128 * kRow;              // one operand part: 16 KB

template <bool SPLIT>
struct Layout {
    // per buffer: A hi, B hi (, A lo, B lo)
    static constexpr int kParts = SPLIT ? 4 : 2;
    static constexpr int kBuf = kParts * kPart;
    static constexpr int kLds = 2 * kBuf;      // 64 KB, or 128 KB with SPLIT
};

// Block scale of a code as an FP32 factor.
template <int SFMT>
__device__ __forceinline__ float scale_value(uint32_t bits) {
    if constexpr (SFMT == BSFP8_MX_E8M0) {
        // 2^(bits - 127); code 0 is 2^-127, an FP32 subnormal
        return bits == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(bits << 23);
    } else if constexpr (SFMT == BSFP8_MX_F16) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
    } else {
        return __uint_as_float(bits << 16);
    }
}

// The two codes of byte P of w (K 2 P, 2 P + 1), times s, into bf16 slots
// 2 P, 2 P + 1 of hi (and the exact remainders into lo).  With a power-of-two
// s (E8M0 scales) one scaled conversion gives the exact bf16 pair directly.
template <int P, bool SPLIT>
__device__ __forceinline__ void dequant_pair(uint32_t w, float s, v8bf& hi, v8bf& lo) {
    if constexpr (!SPLIT) {
        const v2bf h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, P);
        hi[2 * P] = h[0];
        hi[2 * P + 1] = h[1];
        return;
    }
    const v2f f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, P);
    const v2f v = f * s;                                   // exact
    const v2bf h = __builtin_convertvector(v, v2bf);       // one packed RNE conversion
    const v2f r = v - __builtin_convertvector(h, v2f);     // exact remainders
    const v2bf l = __builtin_convertvector(r, v2bf);       // exact
    hi[2 * P] = h[0];
    hi[2 * P + 1] = h[1];
    lo[2 * P] = l[0];
    lo[2 * P + 1] = l[1];
}

// 32 codes (16 bytes, K order, low nibble first) of one row and their block
// scales -> bf16 hi (and lo) halves, 4 chunks of 8 each.
template <int BLOCK, int SFMT, bool SPLIT>
__device__ __forceinline__ void dequant32(const uint4& codes, const float (&sc)[32 / BLOCK],
                                          v8bf (&hi)[4], v8bf (&lo)[4]) {
    const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {            // chunk j: K 8 j .. 8 j + 7, the nibbles of w[j]
        const float s = sc[(8 * j) / BLOCK];
        dequant_pair<0, SPLIT>(w[j], s, hi[j], lo[j]);
        dequant_pair<1, SPLIT>(w[j], s, hi[j], lo[j]);
        dequant_pair<2, SPLIT>(w[j], s, hi[j], lo[j]);
        dequant_pair<3, SPLIT>(w[j], s, hi[j], lo[j]);
    }
}

template <int BLOCK, int SFMT, int OUT>
__global__ __launch_bounds__(kThreads, SFMT == BSFP8_MX_E8M0 ? 2 : 1) void gemm_mx_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const void* __restrict__ sA,
    const uint8_t* __restrict__ B, const void* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
    constexpr bool SPLIT = SFMT != BSFP8_MX_E8M0;
    constexpr int NB = 32 / BLOCK;            // block scales per 32 K values
    using L = Layout<SPLIT>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[L::kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int nst = (K + SK - 1) / SK;
    const int kh = K >> 1;                    // code bytes per row
    const int nsc = K / BLOCK;                // scales per row

    // staging role: row sr of A and B, K half sh (32 values) of each stage.
    // Lanes 8 i .. 8 i + 7 of a 32-lane group take rows 2 j + (i & 1) (j = 0..7)
    // of its 16 rows and half i >> 1, so the 8 lanes of a write phase store
    // to 8 rows with distinct (R >> 1) & 7, i.e. 8 distinct bank groups.
    const int sr = 16 * (tid >> 5) + 2 * (tid & 7) + ((tid >> 3) & 1);
    const int sh = (tid >> 4) & 1;
    // Range-checked buffer loads, based at the tile's first row: rows past
    // M or N and K past the end read as zero, with no branch, so the compiler
    // waits for them only where they are used (zero scale bits are a finite
    // scale, and they only multiply zero codes).
    constexpr int SB = SFMT == BSFP8_MX_E8M0 ? 1 : 2;    // bytes per scale
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A + static_cast<int64_t>(m0) * kh), 0, rows_a * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B + static_cast<int64_t>(n0) * kh), 0, rows_b * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(sA) + static_cast<int64_t>(m0) * nsc * SB), 0,
        rows_a * nsc * SB, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(sB) + static_cast<int64_t>(n0) * nsc * SB), 0,
        rows_b * nsc * SB, 0x00020000);
    constexpr uint32_t kOut = 0x80000000u;
    const bool a_ok = sr < rows_a;
    const bool b_ok = sr < rows_b;
    // a thread's NB scales of a stage: NB * SB contiguous bytes, aligned to their size
    auto load_scales = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t off) -> uint64_t {
        constexpr int bytes = NB * SB;
        if constexpr (bytes == 1) return __builtin_amdgcn_raw_buffer_load_b8(rs, static_cast<int>(off), 0, 0);
        else if constexpr (bytes == 2) return __builtin_amdgcn_raw_buffer_load_b16(rs, static_cast<int>(off), 0, 0);
        else if constexpr (bytes == 4) return __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(off), 0, 0);
        else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, static_cast<int>(off), 0, 0);
            return static_cast<uint64_t>(v[0]) | (static_cast<uint64_t>(v[1]) << 32);
        }
    };
    // two register slots: the codes and scales of stages s + 1 and s + 2 are
    // in flight while stage s is multiplied
    uint4 ca[2], cbb[2];
    float sca[2][NB], scb[2][NB];
    auto fetch = [&](auto SLOT, int s) {
        constexpr int sl = SLOT;
        const int k0 = s * SK + 32 * sh;      // first K value of this thread
        const bool in_k = k0 < K;             // K is a multiple of 32: all 32 or none
        const uint32_t oa = in_k && a_ok ? static_cast<uint32_t>(sr * kh + k0 / 2) : kOut;
        const uint32_t ob = in_k && b_ok ? static_cast<uint32_t>(sr * kh + k0 / 2) : kOut;
        const auto wa = __builtin_amdgcn_raw_buffer_load_b128(rs_a, static_cast<int>(oa), 0, 0);
        const auto wb = __builtin_amdgcn_raw_buffer_load_b128(rs_b, static_cast<int>(ob), 0, 0);
        ca[sl] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
        cbb[sl] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
        const uint32_t so = static_cast<uint32_t>((k0 / BLOCK) * SB);
        const uint64_t va = load_scales(rs_sa, in_k && a_ok ? static_cast<uint32_t>(sr * nsc * SB) + so : kOut);
        const uint64_t vb = load_scales(rs_sb, in_k && b_ok ? static_cast<uint32_t>(sr * nsc * SB) + so : kOut);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const uint32_t mask = SB == 1 ? 0xFFu : 0xFFFFu;
            sca[sl][j] = scale_value<SFMT>(static_cast<uint32_t>(va >> (8 * SB * j)) & mask);
            scb[sl][j] = scale_value<SFMT>(static_cast<uint32_t>(vb >> (8 * SB * j)) & mask);
        }
    };
    // chunk c (0..7) of LDS row R of part p in buffer buf
    auto chunk_ptr = [&](int buf, int part, int R, int c) {
        return lds + buf * L::kBuf + part * kPart + R * kRow + ((c ^ ((R >> 1) & 7)) << 4);
    };
    auto stage = [&](auto SLOT, int buf) {
        constexpr int sl = SLOT;
        v8bf hi[4], lo[4];
        dequant32<BLOCK, SFMT, SPLIT>(ca[sl], sca[sl], hi, lo);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<v8bf*>(chunk_ptr(buf, 0, sr, 4 * sh + j)) = hi[j];
            if constexpr (SPLIT) *reinterpret_cast<v8bf*>(chunk_ptr(buf, 2, sr, 4 * sh + j)) = lo[j];
        }
        dequant32<BLOCK, SFMT, SPLIT>(cbb[sl], scb[sl], hi, lo);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<v8bf*>(chunk_ptr(buf, 1, sr, 4 * sh + j)) = hi[j];
            if constexpr (SPLIT) *reinterpret_cast<v8bf*>(chunk_ptr(buf, 3, sr, 4 * sh + j)) = lo[j];
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

    // fragment of K step q (16 K): lane half h reads K 16 q + 8 h .. + 7 of
    // row (lane % 32) of its 32-row group = chunk 2 q + h
    const int fr = lane & 31;
    const int fh = lane >> 5;
    auto frag = [&](int buf, int part, int R, int q) {
        return *reinterpret_cast<const v8bf*>(chunk_ptr(buf, part, R, 2 * q + fh));
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    fetch(I0{}, 0);
    fetch(I1{}, 1);
    stage(I0{}, 0);
    __syncthreads();
    fetch(I0{}, 2);
    // the MFMAs of K step q: B rows are the MFMA row operand, A rows the column operand
    auto mul_step = [&](const v8bf (&xa)[2], const v8bf (&xb)[2], int buf, int q) {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int tj = 0; tj < 2; ++tj)
                acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb[ti], xa[tj], acc[ti][tj], 0, 0, 0);
        if constexpr (SPLIT) {
            v8bf ya[2], yb[2];                // lo parts
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                yb[t] = frag(buf, 3, wn * 64 + t * 32 + fr, q);
                ya[t] = frag(buf, 2, wm * 64 + t * 32 + fr, q);
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
                    acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb[ti], ya[tj], acc[ti][tj], 0, 0, 0);
                    acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yb[ti], xa[tj], acc[ti][tj], 0, 0, 0);
                    // lo * lo is below 2^-16 of hi * hi: kept for FP32 output
                    // (tolerance 2^-19), left out for 16-bit output (2^-7)
                    if constexpr (OUT == BSFP8_OUT_F32)
                        acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yb[ti], ya[tj], acc[ti][tj], 0, 0, 0);
                }
        }
    };
    // the NQ K steps of a buffer: all fragments of a step are read before
    // its MFMAs, and the steps are unrolled so the reads of the next overlap them
    auto multiply = [&](auto NQ_, int buf) {
        constexpr int NQ = NQ_;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            v8bf xa[2], xb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                xb[t] = frag(buf, 1, wn * 64 + t * 32 + fr, q);
                xa[t] = frag(buf, 0, wm * 64 + t * 32 + fr, q);
            }
            mul_step(xa, xb, buf, q);
        }
    };
    // stage s: multiply buffer s % 2, dequantise stage s + 1 (slot (s + 1) % 2)
    // into the other buffer, then refill that slot with stage s + 3
    auto step = [&](auto PAR, int s) {
        constexpr int par = PAR;              // s % 2
        const int buf = par;
        multiply(std::integral_constant<int, SK / 16>{}, buf);
        if (s + 1 < nst) stage(std::integral_constant<int, par ^ 1>{}, buf ^ 1);
        __syncthreads();
        if (s + 3 < nst) fetch(std::integral_constant<int, par ^ 1>{}, s + 3);
    };
    // full stages; K % 64 == 32 leaves a last stage of 32 K (two steps)
    const int nfull = K / SK;
    for (int s = 0; s < nfull; s += 2) {
        step(I0{}, s);
        if (s + 1 < nfull) step(I1{}, s + 1);
    }
    if (nfull < nst) {
        multiply(std::integral_constant<int, 2>{}, nfull & 1);
        __syncthreads();                      // its fragment reads end before the epilogue reuses LDS
    }

    // Epilogue: the FP32 tile (128 rows x 512 bytes) through LDS, then whole
    // rows per store; 16-byte chunk c of row R at c ^ (R & 15).  Lane l of
    // wave (wm, wn) holds, for MFMA tile (ti, tj), output row
    // wm 64 + tj 32 + l % 32 and columns wn 64 + ti 32 + 8 q + 4 (l / 32) + e
    // in acc[ti][tj][4 q + e].
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int R = wm * 64 + tj * 32 + fr;
                const int c = wn * 16 + ti * 8 + q * 2 + fh;
                *reinterpret_cast<float4*>(lds + R * 512 + ((c ^ (R & 15)) << 4)) =
                    make_float4(acc[ti][tj][4 * q + 0], acc[ti][tj][4 * q + 1],
                                acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]);
            }
    __syncthreads();
    if constexpr (OUT == BSFP8_OUT_F32) {
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
            const int R = wave * 32 + i * 2 + (lane >> 5);
            const int c = lane & 31;
            const float4 v = *reinterpret_cast<const float4*>(lds + R * 512 + ((c ^ (R & 15)) << 4));
            const float a4[4] = {v.x, v.y, v.z, v.w};
            finish_row_chunk<OUT, 4>(D, ldd, ep, m0 + R, n0 + c * 4, M, N, vec_ok, a4);
        }
    } else {
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

// Large-tile form for E8M0 scales (blocks of 16 or 8): 256 x 256 output tile,
// 4 waves of 128 x 128 (4 x 4 MFMA tiles, accumulators in AGPRs), one
// workgroup per CU.  Per 64-K stage each thread dequantises one row of A and
// one of B (64 K values each) into the bf16 stage buffer (256 + 256 rows of
// 128 bytes, chunk c of row R at c ^ ((R >> 1) & 7)); thread t takes row
// 16 (t / 16) + 2 (t % 8) + (t / 8) % 2 so that the 8 lanes of a write phase
// hit 8 distinct bank groups.  Half the dequantisation and half the fragment
// reads per MFMA of the 128 x 128 form.
constexpr int kBigRows = 256;
constexpr int kBigPart = kBigRows * kRow;       // 32 KB
constexpr int kBigBuf = 2 * kBigPart;           // A, B: 64 KB
constexpr int kBigLds = 2 * kBigBuf;            // 128 KB

template <int BLOCK, int OUT, bool STAGE16>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_big_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
    constexpr int NB = SK / BLOCK;               // scales per row per stage (4 or 8 bytes)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kBigLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, 4, &tm, &tn);
    const int m0 = tm * kBigRows;
    const int n0 = tn * kBigRows;
    const int nfull = K / SK;
    const int nst = (K + SK - 1) / SK;
    const int kh = K >> 1;
    const int nsc = K / BLOCK;

    const int sr = 16 * (tid >> 4) + 2 * (tid & 7) + ((tid >> 3) & 1);
    // Range-checked buffer loads, based at the tile's first row: rows past
    // M or N and K past the end read as zero (an out-of-range offset), with
    // no branch, so the compiler waits for them only where they are used.
    // A zero E8M0 byte is the finite scale 2^-127 and multiplies zero codes.
    const int rows_a = min(kBigRows, M - m0), rows_b = min(kBigRows, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A + static_cast<int64_t>(m0) * kh), 0, rows_a * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B + static_cast<int64_t>(n0) * kh), 0, rows_b * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sA + static_cast<int64_t>(m0) * nsc), 0, rows_a * nsc, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sB + static_cast<int64_t>(n0) * nsc), 0, rows_b * nsc, 0x00020000);
    constexpr uint32_t kOut = 0x80000000u;
    const bool a_ok = sr < rows_a;
    const bool b_ok = sr < rows_b;

    // two register slots of a stage's codes (2 x 16 bytes per row) and scales
    uint4 ca[2][2], cb[2][2];
    uint64_t va[2], vb[2];
    auto fetch = [&](auto SLOT, int s) {
        constexpr int sl = SLOT;
        const int k0 = s * SK;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool in_k = k0 + 32 * h < K;
            const uint32_t oa = in_k && a_ok ? static_cast<uint32_t>(sr * kh + k0 / 2 + 16 * h) : kOut;
            const uint32_t ob = in_k && b_ok ? static_cast<uint32_t>(sr * kh + k0 / 2 + 16 * h) : kOut;
            const auto wa = __builtin_amdgcn_raw_buffer_load_b128(rs_a, static_cast<int>(oa), 0, 0);
            const auto wb = __builtin_amdgcn_raw_buffer_load_b128(rs_b, static_cast<int>(ob), 0, 0);
            ca[sl][h] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
            cb[sl][h] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
        }
        // the scales of each 32-K half (2 bytes for blocks of 16, 4 for 8),
        // loaded apart: a row's scales start at a multiple of that size only
        va[sl] = 0;
        vb[sl] = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool in_k = k0 + 32 * h < K;
            const int so = k0 / BLOCK + h * (NB / 2);
            const uint32_t oa = in_k && a_ok ? static_cast<uint32_t>(sr * nsc + so) : kOut;
            const uint32_t ob = in_k && b_ok ? static_cast<uint32_t>(sr * nsc + so) : kOut;
            uint64_t ha, hb;
            if constexpr (NB == 4) {
                ha = __builtin_amdgcn_raw_buffer_load_b16(rs_sa, static_cast<int>(oa), 0, 0);
                hb = __builtin_amdgcn_raw_buffer_load_b16(rs_sb, static_cast<int>(ob), 0, 0);
            } else {
                ha = __builtin_amdgcn_raw_buffer_load_b32(rs_sa, static_cast<int>(oa), 0, 0);
                hb = __builtin_amdgcn_raw_buffer_load_b32(rs_sb, static_cast<int>(ob), 0, 0);
            }
            va[sl] |= ha << (8 * (NB / 2) * h);
            vb[sl] |= hb << (8 * (NB / 2) * h);
        }
    };
    // Staging, in pieces placed between the MFMAs of a K step: piece p (0..31)
    // converts values 2 p, 2 p + 1 of this thread's row of operand OP (slot
    // SL), 64-K half p / 16, chunk (p / 4) % 4, with its block's E8M0 scale;
    // the fourth piece of a chunk writes it to row sr of part OP of buffer BF
    // (chunk c of row R at c ^ ((R >> 1) & 7)).
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((big_tile::lds_byte*)lds));
    uint32_t wr[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) wr[c] = lds0 + sr * kRow + ((c ^ ((sr >> 1) & 7)) << 4);
    big_tile::u32x4 chunk;
    uint32_t cwd;                                // the chunk's code word and scale,
    float csc;                                   // taken at its first piece
    auto piece = [&](auto OP, auto SL, auto BF, auto Pp) {
        constexpr int op = OP, sl = SL, bf = BF, p = Pp;
        constexpr int h = p >> 4, j = (p >> 2) & 3, c = 4 * h + j;
        if constexpr ((p & 3) == 0) {
            const uint4& w4 = op == 0 ? ca[sl][h] : cb[sl][h];
            cwd = j == 0 ? w4.x : j == 1 ? w4.y : j == 2 ? w4.z : w4.w;
            csc = scale_value<BSFP8_MX_E8M0>(
                static_cast<uint32_t>((op == 0 ? va[sl] : vb[sl]) >> (8 * ((32 * h + 8 * j) / BLOCK))) & 0xFFu);
            // the chunk's work is pinned to this point of the MFMA sequence
            asm volatile("" : "+v"(cwd), "+v"(csc));
        }
        const v2bf pr = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwd, csc, p & 3);
        const uint32_t pb = __builtin_bit_cast(uint32_t, pr);
        asm volatile("" : : "v"(pb));            // and each pair is done here
        chunk[p & 3] = pb;
        if constexpr ((p & 3) == 3) big_tile::lds_write16<op * kBigPart>(wr[c] + bf * kBigBuf, chunk);
    };
    auto stage_row = [&](auto OP, auto SL, auto BF) {
        big_tile::static_for<32>([&](auto Pp) { piece(OP, SL, BF, Pp); });
    };

    // Fragment reads and MFMAs are ordered inline assembly (the scheme of the
    // large MXFP4 kernel): the 8 fragment reads of the next 16-K step are
    // issued between the 16 MFMAs of the current one, and each step starts
    // with an explicit lgkmcnt wait.  Stage s + 1 is dequantised during steps
    // 0..2 of stage s into the other buffer (free since the previous barrier);
    // the barrier before step 3 publishes it, and step 3 reads its first
    // fragments.
    const int fr = lane & 31;
    const int fh = lane >> 5;
    const int sw = (fr >> 1) & 7;
    uint32_t rd_a[2][4], rd_b[2][4];
#pragma unroll
    for (int bf = 0; bf < 2; ++bf)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t pos = static_cast<uint32_t>(((2 * q + fh) ^ sw) << 4);
            rd_a[bf][q] = lds0 + bf * kBigBuf + (wm * 128 + fr) * kRow + pos;
            rd_b[bf][q] = lds0 + bf * kBigBuf + kBigPart + (wn * 128 + fr) * kRow + pos;
        }
    struct Frag { big_tile::u32x4 x[4], y[4]; };    // x: B rows (MFMA row operand), y: A rows
    Frag frg[2];
    auto read_frags = [&](Frag& g, uint32_t ra, uint32_t rb) {
        big_tile::static_for<4>([&](auto t) {
            big_tile::lds_read16<t * 32 * kRow>(g.x[t], rb);
            big_tile::lds_read16<t * 32 * kRow>(g.y[t], ra);
        });
    };
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
    // the 16 MFMAs of one step on f, with the 8 reads of the next step into g
    // and, with DEQ, the 32 staging pieces of operand OP's row of slot SL
    // into buffer BF, two after each MFMA
    auto kstep = [&](auto DEQ, auto OP, auto SL, const Frag& f, Frag& g, uint32_t ra, uint32_t rb) {
        big_tile::static_for<16>([&](auto J) {
            constexpr int j = J;
            constexpr int ti = j >> 2, tj = j & 3;
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+a"(acc[ti][tj]) : "v"(f.x[ti]), "v"(f.y[tj]));
            if constexpr (j < 8) {
                constexpr int t = j >> 1;
                if constexpr (j & 1) big_tile::lds_read16<t * 32 * kRow>(g.y[t], ra);
                else big_tile::lds_read16<t * 32 * kRow>(g.x[t], rb);
            }
            if constexpr (DEQ) {
                piece(OP, SL, SL, std::integral_constant<int, 2 * j>{});
                piece(OP, SL, SL, std::integral_constant<int, 2 * j + 1>{});
            }
        });
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    fetch(I0{}, 0);
    fetch(I1{}, 1);
    stage_row(I0{}, I0{}, I0{});
    stage_row(I1{}, I0{}, I0{});
    big_tile::lds_wait_barrier();
    read_frags(frg[0], rd_a[0][0], rd_b[0][0]);
    fetch(I0{}, 2);
    // Stage s + 1 (slot and buffer s % 2 ^ 1) is dequantised during steps 0
    // and 1 of stage s, also after the last stage, from zeros: that buffer
    // was last read before the previous barrier.
    auto step = [&](auto PAR, int s) {
        constexpr int par = PAR;              // s % 2 = this stage's buffer
        constexpr int nb = par ^ 1;
        using NB_ = std::integral_constant<int, nb>;
        big_tile::lds_wait();
        kstep(std::true_type{}, I0{}, NB_{}, frg[0], frg[1], rd_a[par][1], rd_b[par][1]);
        big_tile::lds_wait();
        kstep(std::true_type{}, I1{}, NB_{}, frg[1], frg[0], rd_a[par][2], rd_b[par][2]);
        big_tile::lds_wait();
        kstep(std::false_type{}, I0{}, NB_{}, frg[0], frg[1], rd_a[par][3], rd_b[par][3]);
        big_tile::lds_wait_barrier();         // stage s + 1 published; buffer par is free after step 3's reads
        kstep(std::false_type{}, I0{}, NB_{}, frg[1], frg[0], rd_a[nb][0], rd_b[nb][0]);
        if (s + 3 < nst) fetch(NB_{}, s + 3);
    };
    // pairs of stages with no branch around either (a conditional second step
    // made the compiler copy all 256 accumulators at the loop's join)
    int s = 0;
    for (; s + 1 < nfull; s += 2) {
        step(I0{}, s);
        step(I1{}, s + 1);
    }
    if (s < nfull) step(I0{}, s);
    if (nfull < nst) {
        // the last 32 K: its first fragments are in frg[0]
        const int pb = nfull & 1;
        big_tile::lds_wait();
        kstep(std::false_type{}, I0{}, I0{}, frg[0], frg[1], rd_a[pb][1], rd_b[pb][1]);
        big_tile::lds_wait();
        kstep(std::false_type{}, I0{}, I0{}, frg[1], frg[0], rd_a[pb][1], rd_b[pb][1]);   // (its reads are not used)
    }
    // the last step's fragment reads have no consumer: naming them after the
    // wait keeps their registers from being reused while they are in flight
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < 2; ++q)
        asm volatile("" :: "v"(frg[q].x[0]), "v"(frg[q].x[1]), "v"(frg[q].x[2]), "v"(frg[q].x[3]),
                           "v"(frg[q].y[0]), "v"(frg[q].y[1]), "v"(frg[q].y[2]), "v"(frg[q].y[3]));
    // MFMA results must settle before the accumulation registers are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                   "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]),
                   "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                   "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));
    // (the epilogue begins with a barrier, after which LDS is reused)
    big_tile::NoScale pre;
    big_tile::epilogue<OUT, STAGE16>(acc, lds, wave, lane, m0, n0, M, N, D, ldd, ep, vec_ok, pre);
}

// Large-tile form for FP16 / BF16 block scales: 256 x 256 output tile, 4 waves
// of 128 x 128 (accumulators in AGPRs), one workgroup per CU, as the E8M0
// form, but with stages of 32 K so that the hi and lo parts of both operands
// (4 parts of 256 rows x 64 bytes) fit twice in LDS.  Row R keeps 16-byte chunk
// c at c ^ ((R >> 2) & 3): the 16 rows of a fragment-read phase and the 8
// consecutive rows of a staging-write phase then hit distinct bank groups.
// Thread t stages row t of A and of B.
//
// Each stage is two K steps of 16, with one barrier between them.  The first
// step multiplies while it reads the second step's fragments and dequantises
// the B rows of the next stage into the other buffer; the barrier publishes
// that stage and frees this one's buffer; the second step multiplies while it
// reads the next stage's first fragments and dequantises the A rows of the
// stage after next into the freed buffer.  A wave issues in order, so the
// conversion overlaps the matrix core only where it sits between MFMAs: one
// pair of values every KINDS MFMAs.  A and B codes are fetched separately,
// each two stages before use.  Stages past the last one are dequantised from
// zeros (range-checked loads past K) and never multiplied.
constexpr int kSRow = 64;                      // bytes per LDS row: 32 bf16
constexpr int kSPart = kBigRows * kSRow;       // 16 KB
constexpr int kSBuf = 4 * kSPart;              // A hi, A lo, B hi, B lo: 64 KB
static_assert(2 * kSBuf == kBigLds, "two stage buffers fill the epilogue's LDS");

template <int BLOCK, int SFMT, int OUT, bool STAGE16>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_split_big_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
    constexpr int NB = 32 / BLOCK;               // scales per row per stage
    constexpr int KINDS = OUT == BSFP8_OUT_F32 ? 4 : 3;   // hi*hi, hi*lo, lo*hi (, lo*lo)
    constexpr int NMF = 16 * KINDS;              // MFMAs per K step
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kBigLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, 4, &tm, &tn);
    const int m0 = tm * kBigRows;
    const int n0 = tn * kBigRows;
    const int nst = K / 32;                      // K is a multiple of 32
    const int kh = K >> 1;
    const int nsc = K / BLOCK;

    // Range-checked buffer loads based at the tile's first row: rows past M
    // or N and K past the end read as zero, with no branch.  Zero scale bits
    // are the scale 0, and they only multiply zero codes.
    const int rows_a = min(kBigRows, M - m0), rows_b = min(kBigRows, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A + static_cast<int64_t>(m0) * kh), 0, rows_a * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B + static_cast<int64_t>(n0) * kh), 0, rows_b * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sA + static_cast<int64_t>(m0) * nsc * 2), 0, rows_a * nsc * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sB + static_cast<int64_t>(n0) * nsc * 2), 0, rows_b * nsc * 2, 0x00020000);
    constexpr uint32_t kOut = 0x80000000u;
    const bool a_ok = tid < rows_a;
    const bool b_ok = tid < rows_b;

    // two register slots per operand of a stage's codes (16 bytes of the row)
    // and scales (2 NB bytes, aligned to their size); stage t uses slot t % 2
    uint4 cw[2][2];                              // [operand][slot]
    uint64_t sv[2][2];
    auto fetch = [&](auto OP, auto SLOT, int s) {
        constexpr int op = OP, sl = SLOT;
        const __amdgpu_buffer_rsrc_t& rs = op == 0 ? rs_a : rs_b;
        const __amdgpu_buffer_rsrc_t& rss = op == 0 ? rs_sa : rs_sb;
        const bool ok = (op == 0 ? a_ok : b_ok) && s * 32 < K;
        const uint32_t oc = ok ? static_cast<uint32_t>(tid * kh + s * 16) : kOut;
        const uint32_t os = ok ? static_cast<uint32_t>(tid * nsc * 2 + (s * 32 / BLOCK) * 2) : kOut;
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(oc), 0, 0);
        cw[op][sl] = make_uint4(w[0], w[1], w[2], w[3]);
        if constexpr (NB == 1) sv[op][sl] = __builtin_amdgcn_raw_buffer_load_b16(rss, static_cast<int>(os), 0, 0);
        else if constexpr (NB == 2) sv[op][sl] = __builtin_amdgcn_raw_buffer_load_b32(rss, static_cast<int>(os), 0, 0);
        else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rss, static_cast<int>(os), 0, 0);
            sv[op][sl] = static_cast<uint64_t>(v[0]) | (static_cast<uint64_t>(v[1]) << 32);
        }
    };

    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((big_tile::lds_byte*)lds));
    // staging writes: chunk c of row tid of buffer 0 (buffer 1 is kSBuf further)
    const int wkey = (tid >> 2) & 3;
    uint32_t wr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) wr[c] = lds0 + tid * kSRow + ((c ^ wkey) << 4);
    // piece p (0..15) of the staging of one row: values 2 p, 2 p + 1 of operand
    // OP from slot SL; the fourth piece of a chunk writes its hi and lo parts
    // to buffer BF
    big_tile::u32x4 chi, clo;                    // a chunk's hi and lo bf16 pairs
    uint32_t cwd;                                // the chunk's code word and scale,
    float csc;                                   // taken at its first piece
    auto piece = [&](auto OP, auto SL, auto BF, auto Pp) {
        constexpr int op = OP, sl = SL, bf = BF, p = Pp;
        constexpr int c = p >> 2;
        if constexpr ((p & 3) == 0) {
            const uint4& w4 = cw[op][sl];
            cwd = c == 0 ? w4.x : c == 1 ? w4.y : c == 2 ? w4.z : w4.w;
            csc = scale_value<SFMT>(static_cast<uint32_t>(sv[op][sl] >> (16 * ((8 * c) / BLOCK))) & 0xFFFFu);
            // the chunk's work is pinned to this point of the MFMA sequence
            // (and each pair's results are required below), so the compiler
            // can neither gather the pieces into one burst nor delay them
            asm volatile("" : "+v"(cwd), "+v"(csc));
        }
        const v2f v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cwd, 1.0f, p & 3) * csc;  // exact
        const v2bf h = __builtin_convertvector(v, v2bf);                          // RNE
        const v2bf l = __builtin_convertvector(v - __builtin_convertvector(h, v2f), v2bf);   // exact
        const uint32_t hb = __builtin_bit_cast(uint32_t, h), lb = __builtin_bit_cast(uint32_t, l);
        asm volatile("" : : "v"(hb), "v"(lb));
        chi[p & 3] = hb;
        clo[p & 3] = lb;
        if constexpr ((p & 3) == 3) {
            const uint32_t addr = wr[c] + bf * kSBuf;
            big_tile::lds_write16<op * 2 * kSPart>(addr, chi);
            big_tile::lds_write16<op * 2 * kSPart + kSPart>(addr, clo);
        }
    };
    auto stage_row = [&](auto OP, auto SL, auto BF) {
        big_tile::static_for<16>([&](auto Pp) { piece(OP, SL, BF, Pp); });
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // fragment reads: lane half h of step q reads chunk 2 q + h of its row
    const int fr = lane & 31;
    const int fh = lane >> 5;
    const int rkey = (fr >> 2) & 3;
    uint32_t rd_a[2][2], rd_b[2][2];
#pragma unroll
    for (int bf = 0; bf < 2; ++bf)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t pos = static_cast<uint32_t>(((2 * q + fh) ^ rkey) << 4);
            rd_a[bf][q] = lds0 + bf * kSBuf + (wm * 128 + fr) * kSRow + pos;
            rd_b[bf][q] = lds0 + bf * kSBuf + 2 * kSPart + (wn * 128 + fr) * kSRow + pos;
        }
    // x: B rows (the MFMA row operand), y: A rows; h / l: hi / lo parts
    struct Frag { big_tile::u32x4 xh[4], yh[4], xl[4], yl[4]; };
    Frag frg[2];
    // read r (0..15) of a step.  The order keeps the first four away from the
    // registers the previous step's last MFMAs read, and puts each fragment
    // well before its first use in the next step.
    auto read = [&](auto Rr, Frag& g, uint32_t ra, uint32_t rb) {
        constexpr int r = Rr;
        constexpr int t = r < 8 ? r & 3 : r < 11 ? r - 8 : r < 15 ? r - 11 : 3;
        constexpr int kLo = kSPart;
        if constexpr (r < 4) big_tile::lds_read16<t * 32 * kSRow>(g.xh[t], rb);
        else if constexpr (r < 8) {
            if constexpr (KINDS == 3) big_tile::lds_read16<kLo + t * 32 * kSRow>(g.yl[t], ra);
            else big_tile::lds_read16<t * 32 * kSRow>(g.yh[t], ra);
        } else if constexpr (r < 11 || r == 15) big_tile::lds_read16<kLo + t * 32 * kSRow>(g.xl[t], rb);
        else {
            if constexpr (KINDS == 3) big_tile::lds_read16<t * 32 * kSRow>(g.yh[t], ra);
            else big_tile::lds_read16<kLo + t * 32 * kSRow>(g.yl[t], ra);
        }
    };
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
    // the NMF MFMAs of one step on f, kind by kind; the 16 reads of the next
    // step into g, one every KINDS MFMAs; the 16 staging pieces of one row of
    // operand OP (slot SL) into buffer BF, one every KINDS MFMAs
    auto kstep = [&](auto OP, auto SL, auto BF, const Frag& f, Frag& g, uint32_t ra, uint32_t rb) {
        big_tile::static_for<NMF>([&](auto J) {
            constexpr int j = J;
            constexpr int kind = j / 16, ti = (j % 16) >> 2, tj = j & 3;
            const big_tile::u32x4& x = kind == 0 || kind == 1 ? f.xh[ti] : f.xl[ti];
            const big_tile::u32x4& y = kind == 0 || kind == 2 ? f.yh[tj] : f.yl[tj];
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[ti][tj]) : "v"(x), "v"(y));
            if constexpr (j % KINDS == 0) read(std::integral_constant<int, j / KINDS>{}, g, ra, rb);
            if constexpr (j % KINDS == 1) piece(OP, SL, BF, std::integral_constant<int, j / KINDS>{});
        });
    };

    // prologue: stage 0 whole and the A rows of stage 1 dequantised, the
    // next codes of each slot in flight
    fetch(I0{}, I0{}, 0);
    fetch(I1{}, I0{}, 0);
    fetch(I0{}, I1{}, 1);
    fetch(I1{}, I1{}, 1);
    stage_row(I0{}, I0{}, I0{});
    stage_row(I1{}, I0{}, I0{});
    stage_row(I0{}, I1{}, I1{});
    fetch(I0{}, I0{}, 2);
    fetch(I1{}, I0{}, 2);
    fetch(I0{}, I1{}, 3);
    big_tile::lds_wait_barrier();
    big_tile::static_for<16>([&](auto Rr) { read(Rr, frg[0], rd_a[0][0], rd_b[0][0]); });
    // stage s: buffer PAR = s % 2 holds it
    auto stage = [&](auto PAR, int s) {
        constexpr int par = PAR;
        using P = std::integral_constant<int, par>;
        using Q = std::integral_constant<int, par ^ 1>;
        big_tile::lds_wait();
        kstep(I1{}, Q{}, Q{}, frg[0], frg[1], rd_a[par][1], rd_b[par][1]);   // B rows of stage s + 1
        fetch(I1{}, Q{}, s + 3);
        big_tile::lds_wait_barrier();         // stage s + 1 published; buffer par is free
        kstep(I0{}, P{}, P{}, frg[1], frg[0], rd_a[par ^ 1][0], rd_b[par ^ 1][0]);   // A rows of stage s + 2
        fetch(I0{}, P{}, s + 4);
    };
    // pairs of stages with no branch around either (see the E8M0 form)
    int s = 0;
    for (; s + 1 < nst; s += 2) {
        stage(I0{}, s);
        stage(I1{}, s + 1);
    }
    if (s < nst) stage(I0{}, s);
    // the last step's fragment reads have no consumer: naming them after the
    // wait keeps their registers from being reused while they are in flight
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        asm volatile("" :: "v"(frg[q].xh[0]), "v"(frg[q].xh[1]), "v"(frg[q].xh[2]), "v"(frg[q].xh[3]),
                           "v"(frg[q].yh[0]), "v"(frg[q].yh[1]), "v"(frg[q].yh[2]), "v"(frg[q].yh[3]));
        asm volatile("" :: "v"(frg[q].xl[0]), "v"(frg[q].xl[1]), "v"(frg[q].xl[2]), "v"(frg[q].xl[3]),
                           "v"(frg[q].yl[0]), "v"(frg[q].yl[1]), "v"(frg[q].yl[2]), "v"(frg[q].yl[3]));
    }
    // MFMA results must settle before the accumulation registers are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                   "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]),
                   "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                   "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));
    // (the epilogue begins with a barrier, after which LDS is reused)
    big_tile::NoScale pre;
    big_tile::epilogue<OUT, STAGE16>(acc, lds, wave, lane, m0, n0, M, N, D, ldd, ep, vec_ok, pre);
}

template <int... I, typename F>
__device__ __forceinline__ void static_for_mx_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for_mx(F&& f) {
    static_for_mx_impl(f, std::make_integer_sequence<int, N>{});
}

// Skinny form (up to 64 rows, or fewer than 32 tiles of 128 x 128): one
// workgroup per 32 x 32 output tile whose four waves split K into contiguous
// ranges of 8-block chunks, as the skinny FP8 and MXFP4 kernels do.  Codes are
// loaded as whole 128-byte row segments and pass through the wave's own LDS
// area; lane (r, h) then takes the 8 packed bytes of K 16 h .. 16 h + 15 of
// block kb of row r (and loads their one or two block scales), dequantises
// them in registers and feeds two bf16 MFMAs (K 16 h .. + 7 in the first, the
// rest in the second).
// Every lane of A and of B uses this same assignment of K to MFMA slots, so
// each dot product is unchanged.  Wide scales use the hi / lo split (three
// products, four for FP32 output).  Blocks past the wave's range read as zero.
constexpr int kMxSkinnyDepth = 2;           // chunks of 8 blocks in flight per wave
constexpr int kMxSkinnyWaves = 4;           // waves per workgroup, splitting K
constexpr int64_t kMxSkinnyMaxM = 64;
constexpr int64_t kMxSkinnyMaxTiles = 32;

template <int BLOCK, int SFMT, int OUT>
__global__ __launch_bounds__(64 * kMxSkinnyWaves, 8 / kMxSkinnyWaves) void gemm_mx_skinny_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, void* __restrict__ D,
    int64_t ldd, Epilogue ep, int tiles_m, int tiles_n, int vec_ok) {
    constexpr bool SPLIT = SFMT != BSFP8_MX_E8M0;
    constexpr int SB = SPLIT ? 2 : 1;                     // bytes per scale
    constexpr int NS = BLOCK == 8 ? 2 : 1;                // scales per lane per block
    __shared__ v16f part[kMxSkinnyWaves - 1][64];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kMxSkinnyWaves][2][32 * 128];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the row tiles of a column tile are launched 8 apart (the same XCD)
    const int grp = static_cast<int>(blockIdx.x) / (8 * tiles_m);
    const int rem = static_cast<int>(blockIdx.x) - grp * 8 * tiles_m;
    const int tm = rem >> 3, tn = grp * 8 + (rem & 7);
    if (tn >= tiles_n) return;
    const int m0 = tm * 32, n0 = tn * 32;
    const int kh = K >> 1, nkb = K >> 5, nsc = K / BLOCK;
    // K is split into chunks of 8 blocks (128 bytes of each row); each wave
    // takes a contiguous range of chunks
    const int nch = (nkb + 7) >> 3;
    const int cper = (nch + kMxSkinnyWaves - 1) / kMxSkinnyWaves;
    const int c0 = min(wave * cper, nch), c1 = min(c0 + cper, nch);

    const int rows_a = min(32, M - m0), rows_b = min(32, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A) + static_cast<int64_t>(m0) * kh, 0, rows_a * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B) + static_cast<int64_t>(n0) * kh, 0, rows_b * kh, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sA) + static_cast<int64_t>(m0) * nsc * SB, 0, rows_a * nsc * SB, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sB) + static_cast<int64_t>(n0) * nsc * SB, 0, rows_b * nsc * SB, 0x00020000);
    const int r = lane & 31, h = lane >> 5;
    constexpr uint32_t kOut = 0x80000000u;
    // Code loads read whole 128-byte row segments: lane l takes 16-byte piece
    // l & 7 (block 8 c + (l & 7)) of row (l >> 3) + 8 i.  The wave stages the
    // chunk in its own LDS area (piece g of row R at g ^ (R & 7)); for block b
    // of the chunk lane (r, h) reads back the 8 bytes of K 16 h .. 16 h + 15
    // of row r and loads their scale(s) itself.
    const int lr = lane >> 3, lg = lane & 7;
    uint8_t* st_a = stage[wave][0];
    uint8_t* st_b = stage[wave][1];
    // the scale index of this lane's first value of block kb
    auto sidx = [&](int kb) { return (32 * kb + 16 * h) / BLOCK; };
    uint4 ga[kMxSkinnyDepth][4], gb[kMxSkinnyDepth][4];
    uint32_t va[kMxSkinnyDepth][8], vb[kMxSkinnyDepth][8];   // NS scales of SB bytes per block
    auto fetch = [&](auto SLOT, int c) {
        constexpr int j = SLOT;
        const bool cok = c < c1;
        const bool ok = cok && 8 * c + lg < nkb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = ok ? static_cast<uint32_t>((lr + 8 * i) * kh + 128 * c + 16 * lg) : kOut;
            const auto wa = __builtin_amdgcn_raw_buffer_load_b128(rs_a, static_cast<int>(o), 0, 0);
            const auto wb = __builtin_amdgcn_raw_buffer_load_b128(rs_b, static_cast<int>(o), 0, 0);
            ga[j][i] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
            gb[j][i] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int kb = 8 * c + b;
            const uint32_t os = cok && kb < nkb ? static_cast<uint32_t>((r * nsc + sidx(kb)) * SB) : kOut;
            if constexpr (NS * SB == 1) {
                va[j][b] = __builtin_amdgcn_raw_buffer_load_b8(rs_sa, static_cast<int>(os), 0, 0);
                vb[j][b] = __builtin_amdgcn_raw_buffer_load_b8(rs_sb, static_cast<int>(os), 0, 0);
            } else if constexpr (NS * SB == 2) {
                va[j][b] = __builtin_amdgcn_raw_buffer_load_b16(rs_sa, static_cast<int>(os), 0, 0);
                vb[j][b] = __builtin_amdgcn_raw_buffer_load_b16(rs_sb, static_cast<int>(os), 0, 0);
            } else {
                va[j][b] = __builtin_amdgcn_raw_buffer_load_b32(rs_sa, static_cast<int>(os), 0, 0);
                vb[j][b] = __builtin_amdgcn_raw_buffer_load_b32(rs_sb, static_cast<int>(os), 0, 0);
            }
        }
    };
    // 16 codes (two words, K order) with their scale(s) -> bf16 hi (and lo),
    // 8 values per MFMA step
    auto dequant = [&](const uint2& w, uint32_t v, v8bf (&hi)[2], v8bf (&lo)[2]) {
        constexpr uint32_t mask = SB == 1 ? 0xFFu : 0xFFFFu;
        const float s0 = scale_value<SFMT>(v & mask);
        const float s1 = NS == 2 ? scale_value<SFMT>((v >> (8 * SB)) & mask) : s0;
        dequant_pair<0, SPLIT>(w.x, s0, hi[0], lo[0]);
        dequant_pair<1, SPLIT>(w.x, s0, hi[0], lo[0]);
        dequant_pair<2, SPLIT>(w.x, s0, hi[0], lo[0]);
        dequant_pair<3, SPLIT>(w.x, s0, hi[0], lo[0]);
        dequant_pair<0, SPLIT>(w.y, s1, hi[1], lo[1]);
        dequant_pair<1, SPLIT>(w.y, s1, hi[1], lo[1]);
        dequant_pair<2, SPLIT>(w.y, s1, hi[1], lo[1]);
        dequant_pair<3, SPLIT>(w.y, s1, hi[1], lo[1]);
    };
    v16f acc = v16f{};
    static_for_mx<kMxSkinnyDepth>([&](auto J) { fetch(J, c0 + J); });
    for (int c = c0; c < c1; c += kMxSkinnyDepth) {
        static_for_mx<kMxSkinnyDepth>([&](auto J) {
            constexpr int j = J;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = lr + 8 * i;
                const int pos = row * 128 + 16 * (lg ^ (row & 7));
                *reinterpret_cast<uint4*>(st_a + pos) = ga[j][i];
                *reinterpret_cast<uint4*>(st_b + pos) = gb[j][i];
            }
            uint32_t sa8[8], sb8[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                sa8[b] = va[j][b];
                sb8[b] = vb[j][b];
            }
            fetch(J, c + j + kMxSkinnyDepth);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int pos = r * 128 + 16 * (b ^ (r & 7)) + 8 * h;
                const uint2 wa = *reinterpret_cast<const uint2*>(st_a + pos);
                const uint2 wb = *reinterpret_cast<const uint2*>(st_b + pos);
                v8bf ah[2], al[2], bh[2], bl[2];
                dequant(wa, sa8[b], ah, al);
                dequant(wb, sb8[b], bh, bl);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    // B rows are the MFMA row operand, A rows the column operand
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[q], ah[q], acc, 0, 0, 0);
                    if constexpr (SPLIT) {
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[q], al[q], acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[q], ah[q], acc, 0, 0, 0);
                        if constexpr (OUT == BSFP8_OUT_F32)
                            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[q], al[q], acc, 0, 0, 0);
                    }
                }
            }
        });
    }
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kMxSkinnyWaves - 1; ++w) {
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

template <int BLOCK, int SFMT, int OUT>
hipError_t launch_out(int64_t M, int64_t N, int64_t K, const uint8_t* a, const void* sa,
                      const uint8_t* b, const void* sb, void* d, int64_t ldd, const Epilogue& ep,
                      hipStream_t stream) {
    if constexpr (SFMT == BSFP8_MX_E8M0 && BLOCK != 32) {
        // the block-scaled FP4 instruction, 32 / BLOCK per 64 K (blocks of 16
        // at half the FP4 rate, twice the bf16 one; blocks of 8 at the bf16
        // rate without the dequantisation): on the MXFP4 kernels' skinny,
        // large or 128 x 128 form.  Blocks of 8 on large shapes that the large
        // form does not take (at least 128 tiles of 256 x 256, K not a
        // multiple of 256) stay on the large dequantising kernel, which the
        // 128 x 128 form did not beat there; blocks of 16 did (by 29-32%).
        const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
        const bool skinny = M <= kMxSkinnyMaxM || ((M + 127) / 128) * ((N + 127) / 128) < kMxSkinnyMaxTiles;
        if (BLOCK == 16 || skinny || mx_fp4_big_applies(M, N, K) || big < 128)
            return launch_gemm_mx_fp4(M, N, K, BLOCK, a, static_cast<const uint8_t*>(sa), b,
                                      static_cast<const uint8_t*>(sb), OUT, d, ldd, ep, stream);
    }
    if (M <= kMxSkinnyMaxM || ((M + 127) / 128) * ((N + 127) / 128) < kMxSkinnyMaxTiles) {
        const int tm = static_cast<int>((M + 31) / 32), tn = static_cast<int>((N + 31) / 32);
        const uint32_t wgs = static_cast<uint32_t>((tn + 7) / 8) * 8u * static_cast<uint32_t>(tm);
        hipLaunchKernelGGL((gemm_mx_skinny_kernel<BLOCK, SFMT, OUT>), dim3(wgs), dim3(64 * kMxSkinnyWaves), 0, stream,
                           static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a,
                           static_cast<const uint8_t*>(sa), b, static_cast<const uint8_t*>(sb), d, ldd, ep,
                           tm, tn, vec16_ok(OUT, d, ldd, ep));
        return hipGetLastError();
    }
    if constexpr (SFMT != BSFP8_MX_E8M0) {
        // the large tile wherever it still gives the chip enough workgroups
        const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
        if (big >= 128) {
            const int tm = static_cast<int>((M + 255) / 256), tn = static_cast<int>((N + 255) / 256);
            const dim3 g(static_cast<uint32_t>(tm) * static_cast<uint32_t>(tn));
            const int vec = vec16_ok(OUT, d, ldd, ep);
            const uint8_t* sa8 = static_cast<const uint8_t*>(sa);
            const uint8_t* sb8 = static_cast<const uint8_t*>(sb);
            if (OUT != BSFP8_OUT_F32 && ep.beta == 0.0f)
                hipLaunchKernelGGL((gemm_mx_split_big_kernel<BLOCK, SFMT, OUT, OUT != BSFP8_OUT_F32>), g,
                                   dim3(kThreads), 0, stream, static_cast<int>(M), static_cast<int>(N),
                                   static_cast<int>(K), a, sa8, b, sb8, d, ldd, ep, tm, tn, vec);
            else
                hipLaunchKernelGGL((gemm_mx_split_big_kernel<BLOCK, SFMT, OUT, false>), g, dim3(kThreads), 0,
                                   stream, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a,
                                   sa8, b, sb8, d, ldd, ep, tm, tn, vec);
            return hipGetLastError();
        }
    }
    if constexpr (SFMT == BSFP8_MX_E8M0 && BLOCK != 32) {
        // the large tile wherever it still gives the chip enough workgroups
        const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
        if (big >= 128) {
            const int tm = static_cast<int>((M + 255) / 256), tn = static_cast<int>((N + 255) / 256);
            const dim3 g(static_cast<uint32_t>(tm) * static_cast<uint32_t>(tn));
            const int vec = vec16_ok(OUT, d, ldd, ep);
            const uint8_t* sa8 = static_cast<const uint8_t*>(sa);
            const uint8_t* sb8 = static_cast<const uint8_t*>(sb);
            if (OUT != BSFP8_OUT_F32 && ep.beta == 0.0f)
                hipLaunchKernelGGL((gemm_mx_big_kernel<BLOCK, OUT, OUT != BSFP8_OUT_F32>), g, dim3(kThreads), 0,
                                   stream, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a,
                                   sa8, b, sb8, d, ldd, ep, tm, tn, vec);
            else
                hipLaunchKernelGGL((gemm_mx_big_kernel<BLOCK, OUT, false>), g, dim3(kThreads), 0, stream,
                                   static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, sa8, b,
                                   sb8, d, ldd, ep, tm, tn, vec);
            return hipGetLastError();
        }
    }
    const int tiles_m = static_cast<int>((M + BM - 1) / BM);
    const int tiles_n = static_cast<int>((N + BN - 1) / BN);
    const dim3 grid(static_cast<uint32_t>(tiles_m) * static_cast<uint32_t>(tiles_n));
    hipLaunchKernelGGL((gemm_mx_kernel<BLOCK, SFMT, OUT>), grid, dim3(kThreads), 0, stream,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, sa, b, sb,
                       d, ldd, ep, tiles_m, tiles_n, vec16_ok(OUT, d, ldd, ep));
    return hipGetLastError();
}

template <int BLOCK, int SFMT>
hipError_t launch_scale(int64_t M, int64_t N, int64_t K, const uint8_t* a, const void* sa,
                        const uint8_t* b, const void* sb, int out, void* d, int64_t ldd,
                        const Epilogue& ep, hipStream_t stream) {
    if (out == BSFP8_OUT_F32) return launch_out<BLOCK, SFMT, BSFP8_OUT_F32>(M, N, K, a, sa, b, sb, d, ldd, ep, stream);
    if (out == BSFP8_OUT_BF16) return launch_out<BLOCK, SFMT, BSFP8_OUT_BF16>(M, N, K, a, sa, b, sb, d, ldd, ep, stream);
    return launch_out<BLOCK, SFMT, BSFP8_OUT_F16>(M, N, K, a, sa, b, sb, d, ldd, ep, stream);
}

template <int BLOCK>
hipError_t launch_block(int64_t M, int64_t N, int64_t K, int sfmt, const uint8_t* a, const void* sa,
                        const uint8_t* b, const void* sb, int out, void* d, int64_t ldd,
                        const Epilogue& ep, hipStream_t stream) {
    if (sfmt == BSFP8_MX_E8M0) return launch_scale<BLOCK, BSFP8_MX_E8M0>(M, N, K, a, sa, b, sb, out, d, ldd, ep, stream);
    if (sfmt == BSFP8_MX_F16) return launch_scale<BLOCK, BSFP8_MX_F16>(M, N, K, a, sa, b, sb, out, d, ldd, ep, stream);
    return launch_scale<BLOCK, BSFP8_MX_BF16>(M, N, K, a, sa, b, sb, out, d, ldd, ep, stream);
}

}  // namespace

hipError_t launch_gemm_mx(int64_t M, int64_t N, int64_t K, int block, int sfmt, const uint8_t* a,
                          const void* a_scales, const uint8_t* b, const void* b_scales, int out,
                          void* d, int64_t ldd, const Epilogue& ep, hipStream_t stream) {
    if (block == 32) return launch_block<32>(M, N, K, sfmt, a, a_scales, b, b_scales, out, d, ldd, ep, stream);
    if (block == 16) return launch_block<16>(M, N, K, sfmt, a, a_scales, b, b_scales, out, d, ldd, ep, stream);
    return launch_block<8>(M, N, K, sfmt, a, a_scales, b, b_scales, out, d, ldd, ep, stream);
}

}  // namespace bsfp8
