// gemm_fp8_big.hip -- per-tile-scaled FP8 GEMM with 256 x 256 output tiles.
//
// The same arithmetic as gemm_fp8_kernel (gemm_fp8.hip): every 32-wide K
// block's partial product P_kb of a 32 x 32 MFMA tile is computed in a fresh
// accumulator by two K = 16 FP8 instructions and promoted into the FP32
// result with acc = fma(sa * sb, P_kb, acc) ("Why grind FP8 GEMM on CDNA4",
// sections 3.2 and 3.3; "Rubin FP4 GEMM deep dive", section 2.2 scales each K
// block's partial sum before accumulating it).  Only the tiling differs.
//
// That kernel is bound by the chip's power: with the exact promotion the FP8
// instructions cannot run at the rate the clock allows, and every byte moved
// costs clock.  This kernel moves fewer bytes per FLOP:
//  * a 256 x 256 workgroup tile (one per CU, 8 waves, two per SIMD) loads each
//    A and B byte from L2 into LDS once per 256 outputs instead of 128: half
//    the L2-to-LDS traffic per FLOP, and fewer L2 misses per FLOP;
//  * each wave owns 64 rows x 128 columns (2 x 4 MFMA tiles), so a 32-wide K
//    block reads 6 fragments of 16 bytes per lane for 16 MFMAs instead of 4
//    for 8: a quarter fewer LDS reads per MFMA.
// The per-tile scales are per 128 rows of A and 128 columns of B, so each
// wave's 64 x 128 tile lies inside one (A tile, B tile) pair and its sigma is
// uniform, as in the 128 x 128 kernel.
//
// Data movement (as gemm_fp8_kernel): direct global-to-LDS loads one stage
// (128 K) ahead into unpadded 128-byte rows, chunk g of row R stored at
// g ^ ((R >> 1) & 7); fragment reads of the next block issued before the
// current block's MFMAs; the promotion software-pipelined (each tile's
// product promoted while the next tile's MFMAs run); the output tile leaves
// through LDS so that every store writes whole rows.
#include "big_tile.h"

#include <type_traits>

namespace bsfp8 {

namespace {

using big_tile::lds_read16;
using big_tile::lds_wait;
using big_tile::static_for;
using big_tile::u32x4;
using big_tile::v16f;

typedef __attribute__((address_space(3))) uint8_t lds_byte;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 512;
constexpr int kTile = 256;
constexpr int kRow = 128;                  // LDS bytes per row and stage (128 K)
constexpr int kOperand = kTile * kRow;     // 32 KB: one operand, one stage
// LDS: A stage buffers at 0 and 32 KB, B's at 64 KB and 96 KB, so that the
// second buffer of an operand is an immediate offset (< 64 KB) from the first
constexpr int kBOffset = 2 * kOperand;
constexpr int kLds = 4 * kOperand;         // 128 KB: one workgroup per CU
// tiles of 256 x 256 below which the 128 x 128 kernel is used (it gives a
// smaller problem four times the workgroups)
constexpr int64_t kBigMinTiles = 192;

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

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Eight FP8 codes -> eight bf16, exactly (unit scale); A and B go through the
// same mapping, so their K indices still pair up.
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

// One 32 x 32 tile's product over one 32-wide K block: lane half h holds K
// 16h .. 16h+15 of its row in x (B) and y (A).  16-bit outputs multiply the
// codes with the FP8 instructions; FP32 output widens them exactly to bf16
// and uses the bf16 instruction (24 fraction bits instead of 13).
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

__device__ __forceinline__ void promote(v16f& a, float sg, const v16f& p) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = fmaf(sg, p[r], a[r]);
}
template <int H>
__device__ __forceinline__ void promote_half(v16f& a, float sg, const v16f& p) {
#pragma unroll
    for (int r = 8 * H; r < 8 * H + 8; ++r) a[r] = fmaf(sg, p[r], a[r]);
}
// Half H of tile_product: the instruction over K 16 H .. 16 H + 15 of the block.
template <int AF, int BF, int OUT, int H>
__device__ __forceinline__ v16f product_half(const u32x4& x, const u32x4& y, v16f p) {
    static_assert(OUT != BSFP8_OUT_F32, "the FP8 instructions are for 16-bit outputs");
    const uint64_t xv = static_cast<uint64_t>(x[2 * H]) | (static_cast<uint64_t>(x[2 * H + 1]) << 32);
    const uint64_t yv = static_cast<uint64_t>(y[2 * H]) | (static_cast<uint64_t>(y[2 * H + 1]) << 32);
    return mfma_codes<AF, BF>(xv, yv, p);
}

// Map a workgroup to its 256 x 256 tile.  Workgroups are dealt to the 8 XCDs
// round-robin; each XCD is given a contiguous range of tiles, walked in groups
// of 4 tile rows, so that the 32 tiles an XCD runs at once (one per CU) form a
// 4 x 8 block that reads 4 A strips and 8 B strips through that XCD's L2.
__device__ __forceinline__ void map_big_tile(int pid, int tiles_m, int tiles_n, int* tm, int* tn) {
    map_tile(pid, tiles_m, tiles_n, 4, tm, tn);
}

// TILE_ONLY: both operands have per-tile scales (tensor_mask == 0), so the
// per-tensor selects drop out of the scale products at compile time (two
// VALU instructions per K block; the common case gets its own instantiation).
template <int AF, int BF, int OUT, bool TILE_ONLY>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_big_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sA,
    const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ D, int64_t ldd,
    Epilogue ep, int tiles_m, int tiles_n, int vec_ok, int tensor_mask) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3;        // rows wm * 64 .. + 63 of the tile
    const int wn = wave >> 2;       // columns wn * 128 .. + 127
    int tm, tn;
    map_big_tile(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
    const int m0 = tm * kTile;
    const int n0 = tn * kTile;
    const int nkb = K >> 5;
    const int nst = (nkb + 3) >> 2;          // 128 K per stage
    const int last = nst - 1;
    const int nfull = nkb >> 2;

    // Direct loads: load i (0..3) of wave w fills LDS rows 64 i + 8 w .. + 7
    // of an operand (1 KB, lane l: row 8 w + l / 8 (+ 64 i), the global chunk
    // that belongs at position l % 8).  The resources start at the tile's
    // first row and cover its rows, so offsets stay below 256 K < 2^31
    // (K < 2^23) and rows past M or N read as zero.  The stage's K offset
    // rides in the scalar offset, which the range check does not cover: in a
    // partial last stage the chunks at or past K get an out-of-range VGPR
    // offset (CHECKED loads) and read as zero without touching memory.
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(A) + static_cast<int64_t>(m0) * K, 0, min(kTile, M - m0) * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(B) + static_cast<int64_t>(n0) * K, 0, min(kTile, N - n0) * K, 0x00020000);
    const int drow = 8 * wave + (lane >> 3);
    const int dchunk = (lane & 7) ^ ((drow >> 1) & 7);
    const uint32_t dma = static_cast<uint32_t>(drow) * K + dchunk * 16;
    const uint32_t row_step = 64u * static_cast<uint32_t>(K);
    const int kend = K - dchunk * 16;
    // Load J (0..7) of a stage: A for even J, B for odd, rows 64 (J / 2) + ...
    // checked: the stage may be the partial last one; the select costs a few
    // VALU instructions but keeps the stage one basic block.  MC (compile
    // time) false drops the select from the stages that never need it.
    auto dma_one = [&](auto J, int stage, int buf, auto MC, bool checked) {
        constexpr int j = J;
        constexpr int i = j >> 1;
        const int so = min(stage, last) * 128;
        uint32_t vo = dma + i * row_step;
        if constexpr (MC) {
            // bit 31 set puts every chunk at or past K out of range; the empty
            // asm keeps the compiler from turning the select into a branch per load
            uint32_t oob = (!checked || so < kend) ? 0u : 0x80000000u;
            asm volatile("" : "+v"(oob));
            vo |= oob;
        }
        lds_void* dst = (lds_void*)(lds + (j & 1) * kBOffset + buf * kOperand + (64 * i + 8 * wave) * kRow);
        __builtin_amdgcn_raw_ptr_buffer_load_lds((j & 1) ? rs_b : rs_a, dst, 16, vo, so, 0, 0);
    };

    // Fragment reads: lane (frag_row r, half h) reads 16-byte chunk 2 kb + h
    // of rows wm 64 + 32 t + r (A, t = 0, 1) and wn 128 + 32 t + r (B,
    // t = 0..3); t and the stage buffer are immediate offsets.
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte*)lds));
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    const int sw = (frag_row >> 1) & 7;
    uint32_t rd_a[4], rd_b[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const uint32_t pos = static_cast<uint32_t>(((2 * kb + half) ^ sw) * 16);
        rd_a[kb] = lds0 + (wm * 64 + frag_row) * kRow + pos;
        rd_b[kb] = lds0 + kBOffset + (wn * 128 + frag_row) * kRow + pos;
    }
    // fragment reads of block kb in stage buffer BUF: A tile t (0, 1), B tile t (0..3)
    auto read_a = [&](u32x4& v, int kb, auto BUF, auto T) {
        lds_read16<BUF * kOperand + T * 32 * kRow>(v, rd_a[kb]);
    };
    auto read_b = [&](u32x4& v, int kb, auto BUF, auto T) {
        lds_read16<BUF * kOperand + T * 32 * kRow>(v, rd_b[kb]);
    };

    // Scales: this wave's A tile row and B tile column (128-row scale tiles).
    // A per-tensor side (bit 0 of tensor_mask: A, bit 1: B) has a one-float
    // array: its offset stays zero and the dwords past it read as zero (the
    // range check of a dwordx4 load is per dword); sa0 / sb0 stand in.
    const bool a_tensor = !TILE_ONLY && (tensor_mask & 1) != 0;
    const bool b_tensor = !TILE_ONLY && (tensor_mask & 2) != 0;
    const int st_m = (M + 127) >> 7, st_n = (N + 127) >> 7;
    const __amdgpu_buffer_rsrc_t rs_sa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(sA), 0, a_tensor ? 4 : st_m * nkb * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(sB), 0, b_tensor ? 4 : st_n * nkb * 4, 0x00020000);
    const uint32_t so_a = a_tensor ? 0u : static_cast<uint32_t>(2 * tm + (wm >> 1)) * nkb * 4;
    const uint32_t so_b = b_tensor ? 0u : static_cast<uint32_t>(2 * tn + wn) * nkb * 4;
    // bit 2 (bit 3): that side's scales are per row, applied at write-back
    const float sa0 = TILE_ONLY ? 0.0f : (tensor_mask & 4) ? 1.0f : sA[0];
    const float sb0 = TILE_ONLY ? 0.0f : (tensor_mask & 8) ? 1.0f : sB[0];
    u32x4 nsa, nsb;
    // A full stage's four scales lie inside the tile row (stage offset in the
    // scalar offset); a partial last stage's would reach past it, so CHECKED
    // loads put the stage offset in the range-checked VGPR offset.
    auto load_scales = [&](u32x4& ra, u32x4& rb, int stage, bool chk) {
        const int so = min(stage, last) * 16;
        const int so_sa = a_tensor ? 0 : so;
        const int so_sb = b_tensor ? 0 : so;
        const uint32_t va = so_a + (chk ? so_sa : 0), vb = so_b + (chk ? so_sb : 0);
        const int sa_s = chk ? 0 : so_sa, sb_s = chk ? 0 : so_sb;
        asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(ra) : "v"(va), "s"(rs_sa), "s"(sa_s) : "memory");
        asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(rb) : "v"(vb), "s"(rs_sb), "s"(sb_s) : "memory");
    };

    v16f acc[4][2];    // [B tile ti][A tile tj]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
    // the last tile's product of the previous block, promoted during the next
    // block (a zero product with a zero scale before the first)
    v16f pend = v16f{};
    float pend_sig = 0.0f;

    // Fragments in registers: the current block's two A fragments, the next
    // block's (read during the current block's last group), and two slots for
    // the B fragments, each read one group (two 32 x 32 tiles) ahead.
    u32x4 fa[2][2], fb[2];      // fa[set][t]
    // FP32 output: this block's A fragments widened to bf16 once, [t][half]
    // (widening them for every group cost 3 VALU instructions per MFMA)
    v8bf wa[2][2];
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // stage 0 and its scales; stage s + 1 is loaded during stage s
    using MayCheck = std::true_type;
    using NoCheck = std::false_type;
    static_for<8>([&](auto J) { dma_one(J, 0, 0, MayCheck{}, true); });
    load_scales(nsa, nsb, 0, true);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    read_a(fa[0][0], 0, I0{}, I0{});
    read_a(fa[0][1], 0, I0{}, I1{});
    read_b(fb[0], 0, I0{}, I0{});

    // One stage (4 blocks of 4 groups) in LDS buffer CB (compile time); it
    // loads the next stage's scales at its top and the next stage's codes into
    // the other buffer, one direct load in each group of blocks 0 and 1 (a
    // burst of loads between MFMAs holds a wave's MFMAs back; the other
    // buffer is free since the last stage's barrier), checked in the last full
    // stage (the only one that can load a partial stage).  Group g multiplies
    // B tile g with both A tiles, the tiles (g, 0) and (g, 1), while the VALU
    // promotes the tile before each.
    auto run_stage = [&](int s, auto CB, auto MC, bool checked) {
        constexpr int cb = CB;
        // this stage's scales were loaded during the last stage, whose barrier
        // waited for every load

        u32x4 ca = nsa, cbv = nsb;
        asm volatile("" : "+v"(ca), "+v"(cbv));
        float sig[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            sig[k] = (a_tensor ? sa0 : __uint_as_float(ca[k])) * (b_tensor ? sb0 : __uint_as_float(cbv[k]));
        load_scales(nsa, nsb, s + 1, MC && checked);
        static_for<4>([&](auto KB) {
            constexpr int kb = KB;
            constexpr int as = kb & 1;          // this block's A set
            const float sg = sig[kb];
            static_for<4>([&](auto G) {
                constexpr int g = G;
                u32x4& bcur = fb[g & 1];
                if constexpr (kb == 3 && g == 3) {
                    // the next stage's codes and scales are in; after the
                    // barrier every wave is done with this stage's buffer
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                } else {
                    lds_wait();
                }
                asm volatile("" : "+v"(bcur), "+v"(fa[as][0]), "+v"(fa[as][1]));
                // the reads one group ahead
                if constexpr (g < 3) {
                    read_b(fb[(g + 1) & 1], kb, CB, std::integral_constant<int, g + 1>{});
                } else if constexpr (kb < 3) {
                    read_a(fa[as ^ 1][0], kb + 1, CB, I0{});
                    read_a(fa[as ^ 1][1], kb + 1, CB, I1{});
                    read_b(fb[0], kb + 1, CB, I0{});
                } else {
                    read_a(fa[as ^ 1][0], 0, std::integral_constant<int, cb ^ 1>{}, I0{});
                    read_a(fa[as ^ 1][1], 0, std::integral_constant<int, cb ^ 1>{}, I1{});
                    read_b(fb[0], 0, std::integral_constant<int, cb ^ 1>{}, I0{});
                }
                if constexpr (kb < 2) dma_one(std::integral_constant<int, 4 * kb + g>{}, s + 1, cb ^ 1, MC, checked);
                // tile (g, 0) while the previous tile is promoted, then tile
                // (g, 1) while (g, 0) is: one MFMA, then 8 FMAs on a product
                // that an earlier MFMA finished, four times.  The scheduling
                // barriers fix that order: left free, the compiler placed
                // FMAs right behind the MFMA whose result they read, so the
                // wave waited there with its next MFMA held back (7-11%
                // slower; 2.5% on FP32 output).
                v16f& prev = acc[g == 0 ? 3 : g - 1][1];
                const float psg = g == 0 ? pend_sig : sg;
                v8bf xb[2];
                if constexpr (OUT == BSFP8_OUT_F32) {
                    if constexpr (g == 0) {
                        wa[0][0] = widen8<AF>(fa[as][0][0], fa[as][0][1]);
                        wa[0][1] = widen8<AF>(fa[as][0][2], fa[as][0][3]);
                        wa[1][0] = widen8<AF>(fa[as][1][0], fa[as][1][1]);
                        wa[1][1] = widen8<AF>(fa[as][1][2], fa[as][1][3]);
                    }
                    xb[0] = widen8<BF>(bcur[0], bcur[1]);
                    xb[1] = widen8<BF>(bcur[2], bcur[3]);
                }
                // half H of the product of B tile g and A tile T
                auto mf = [&](auto T, auto H, const v16f& c) -> v16f {
                    if constexpr (OUT == BSFP8_OUT_F32)
                        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb[H], wa[T][H], c, 0, 0, 0);
                    else
                        return product_half<AF, BF, OUT, H>(bcur, fa[as][T], c);
                };
                {
                    __builtin_amdgcn_sched_barrier(0);
                    v16f p0 = mf(I0{}, I0{}, v16f{});
                    __builtin_amdgcn_sched_barrier(0);
                    promote_half<0>(prev, psg, pend);
                    __builtin_amdgcn_sched_barrier(0);
                    p0 = mf(I0{}, I1{}, p0);
                    __builtin_amdgcn_sched_barrier(0);
                    promote_half<1>(prev, psg, pend);
                    __builtin_amdgcn_sched_barrier(0);
                    v16f pn = mf(I1{}, I0{}, v16f{});
                    __builtin_amdgcn_sched_barrier(0);
                    promote_half<0>(acc[g][0], sg, p0);
                    __builtin_amdgcn_sched_barrier(0);
                    pn = mf(I1{}, I1{}, pn);
                    __builtin_amdgcn_sched_barrier(0);
                    promote_half<1>(acc[g][0], sg, p0);
                    __builtin_amdgcn_sched_barrier(0);
                    pend = pn;
                }
                // the group's promotions finish before the next group starts,
                // so that at most two products are live (the MFMA builtins
                // are pure: only data dependencies order them)
                asm volatile("" : "+v"(prev), "+v"(acc[g][0]));
            });
            pend_sig = sg;
        });
    };
    // stages before nfast load a full next stage: their loads need no check
    const int nfast = nfull < nst ? nfull - 1 : nfull;
    int s0 = 0;
    for (; s0 + 1 < nfast; s0 += 2) {
        run_stage(s0, I0{}, NoCheck{}, false);
        run_stage(s0 + 1, I1{}, NoCheck{}, false);
    }
    // the one or two full stages left, the last of which may load a partial one
    if (s0 < nfull) {
        run_stage(s0, I0{}, MayCheck{}, s0 >= nfast);
        ++s0;
    }
    if (s0 < nfull) run_stage(s0, I1{}, MayCheck{}, s0 >= nfast);
    promote(acc[3][1], pend_sig, pend);

    if (nfull < nst) {
        // partial stage (1 to 3 blocks) in buffer nfull % 2: its scales and
        // block 0's A and first B fragments are already loaded (set 0)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        u32x4 ca = nsa, cbv = nsb;
        asm volatile("" : "+v"(ca), "+v"(cbv));
        const int nk = nkb - 4 * nfull;
        const uint32_t bo = (nfull & 1) ? kOperand : 0;
        for (int kb = 0; kb < nk; ++kb) {
            u32x4 xa[2], xb;
            if (kb == 0) {
                lds_wait();
                xa[0] = fa[0][0]; xa[1] = fa[0][1];
            } else {
                // block kb of the stage: chunk 2 kb + h of the same rows
                const uint32_t dpos = ((((2 * kb + half) ^ sw) - (half ^ sw)) * 16);
                lds_read16<0>(xa[0], rd_a[0] + bo + dpos);
                lds_read16<32 * kRow>(xa[1], rd_a[0] + bo + dpos);
                lds_wait();
            }
            asm volatile("" : "+v"(xa[0]), "+v"(xa[1]));
            const float sg = (a_tensor ? sa0 : __uint_as_float(ca[kb])) * (b_tensor ? sb0 : __uint_as_float(cbv[kb]));
            static_for<4>([&](auto TI) {
                constexpr int ti = TI;
                const uint32_t dpos = ((((2 * kb + half) ^ sw) - (half ^ sw)) * 16);
                lds_read16<ti * 32 * kRow>(xb, rd_b[0] + bo + dpos);
                lds_wait();
                asm volatile("" : "+v"(xb));
                promote(acc[ti][0], sg, tile_product<AF, BF, OUT>(xb, xa[0]));
                promote(acc[ti][1], sg, tile_product<AF, BF, OUT>(xb, xa[1]));
            });
        }
    }
    // the last stage's scale loads and fragment reads may have no consumer:
    // naming them after the wait keeps their registers from being reused
    // while they are in flight
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    asm volatile("" :: "v"(nsa), "v"(nsb), "v"(fa[0][0]), "v"(fa[0][1]), "v"(fa[1][0]), "v"(fa[1][1]),
                       "v"(fb[0]), "v"(fb[1]));

    // Epilogue through LDS (free now): acc[ti][tj][4 q + e] is tile element
    // (wm 64 + 32 tj + lane % 32, wn 128 + 32 ti + 8 q + 4 (lane / 32) + e).
    // 16-byte chunk c of LDS row R sits at c ^ (R & 15), which keeps the
    // scattered writes and the row reads free of bank conflicts.
    __syncthreads();
    if constexpr (OUT != BSFP8_OUT_F32) {
        if (ep.beta == 0.0f && !ep.row_scale && !ep.col_scale) {
            // 16-bit output without C: alpha * acc converted while staged,
            // 256 rows x 512 bytes = the whole 128 KB in one pass
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int R = wm * 64 + tj * 32 + frag_row;
                        const int c = wn * 16 + ti * 4 + q;
                        const uint32_t h0 = to_half_bits<OUT>(ep.alpha * acc[ti][tj][4 * q + 0]);
                        const uint32_t h1 = to_half_bits<OUT>(ep.alpha * acc[ti][tj][4 * q + 1]);
                        const uint32_t h2 = to_half_bits<OUT>(ep.alpha * acc[ti][tj][4 * q + 2]);
                        const uint32_t h3 = to_half_bits<OUT>(ep.alpha * acc[ti][tj][4 * q + 3]);
                        *reinterpret_cast<uint2*>(lds + R * 512 + ((c ^ (R & 15)) << 4) + 8 * half) =
                            make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
                    }
            __syncthreads();
#pragma unroll 4
            for (int i = 0; i < 16; ++i) {
                const int R = wave * 32 + 2 * i + half;
                const int c = lane & 31;
                const uint4 w = *reinterpret_cast<const uint4*>(lds + R * 512 + ((c ^ (R & 15)) << 4));
                store_half8(D, ldd, m0 + R, n0 + c * 8, M, N, vec_ok, w);
            }
            return;
        }
    }
    // General case: the FP32 tile in two passes of 128 rows x 1 KB (waves
    // wm = 0, 1 hold rows 0-127, waves wm = 2, 3 rows 128-255); alpha,
    // beta * C and the output conversion are applied in the row phase.
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if ((wm >> 1) == p) {
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int R = (wm & 1) * 64 + tj * 32 + frag_row;
                        const int c = wn * 32 + ti * 8 + q * 2 + half;
                        *reinterpret_cast<float4*>(lds + R * 1024 + ((c ^ (R & 15)) << 4)) =
                            make_float4(acc[ti][tj][4 * q + 0], acc[ti][tj][4 * q + 1],
                                        acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]);
                    }
        }
        __syncthreads();
        if constexpr (OUT == BSFP8_OUT_F32) {
#pragma unroll 4
            for (int i = 0; i < 16; ++i) {
                const int R = wave * 16 + i;
                const int c = lane;
                const float4 v = *reinterpret_cast<const float4*>(lds + R * 1024 + ((c ^ (R & 15)) << 4));
                const float a4[4] = {v.x, v.y, v.z, v.w};
                finish_row_chunk<OUT, 4>(D, ldd, ep, m0 + p * 128 + R, n0 + c * 4, M, N, vec_ok, a4);
            }
        } else {
#pragma unroll 4
            for (int i = 0; i < 8; ++i) {
                const int R = wave * 16 + i * 2 + half;
                const int c = (lane & 31) * 2;
                const float4 v0 = *reinterpret_cast<const float4*>(lds + R * 1024 + ((c ^ (R & 15)) << 4));
                const float4 v1 = *reinterpret_cast<const float4*>(lds + R * 1024 + (((c + 1) ^ (R & 15)) << 4));
                const float a8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                finish_row_chunk<OUT, 8>(D, ldd, ep, m0 + p * 128 + R, n0 + c * 4, M, N, vec_ok, a8);
            }
        }
        __syncthreads();
    }
}

template <int AF, int BF, int OUT>
hipError_t launch_out(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                      const uint8_t* b, const float* sb, void* d, int64_t ldd, const Epilogue& ep,
                      int tensor_mask, hipStream_t stream) {
    const int tiles_m = static_cast<int>((M + kTile - 1) / kTile);
    const int tiles_n = static_cast<int>((N + kTile - 1) / kTile);
    const dim3 grid(static_cast<uint32_t>(tiles_m) * static_cast<uint32_t>(tiles_n));
    if (tensor_mask == 0)
        hipLaunchKernelGGL((gemm_fp8_big_kernel<AF, BF, OUT, true>), grid, dim3(kThreads), 0, stream,
                           static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, sa, b, sb, d, ldd,
                           ep, tiles_m, tiles_n, vec16_ok(OUT, d, ldd, ep), tensor_mask);
    else
        hipLaunchKernelGGL((gemm_fp8_big_kernel<AF, BF, OUT, false>), grid, dim3(kThreads), 0, stream,
                           static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), a, sa, b, sb, d, ldd,
                           ep, tiles_m, tiles_n, vec16_ok(OUT, d, ldd, ep), tensor_mask);
    return hipGetLastError();
}

template <int AF, int BF>
hipError_t launch_typed(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                        const uint8_t* b, const float* sb, int out, void* d, int64_t ldd,
                        const Epilogue& ep, int tensor_mask, hipStream_t stream) {
    if (out == BSFP8_OUT_F32)
        return launch_out<AF, BF, BSFP8_OUT_F32>(M, N, K, a, sa, b, sb, d, ldd, ep, tensor_mask, stream);
    if (out == BSFP8_OUT_BF16)
        return launch_out<AF, BF, BSFP8_OUT_BF16>(M, N, K, a, sa, b, sb, d, ldd, ep, tensor_mask, stream);
    return launch_out<AF, BF, BSFP8_OUT_F16>(M, N, K, a, sa, b, sb, d, ldd, ep, tensor_mask, stream);
}

}  // namespace

bool gemm_fp8_big_fits(int64_t M, int64_t N, int64_t K) {
    // a 256-row band of an operand is addressed with 32-bit offsets
    if (K >= (int64_t(1) << 23)) return false;
    return ((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile) >= kBigMinTiles;
}

hipError_t launch_gemm_fp8_big(int64_t M, int64_t N, int64_t K, int a_fmt, const uint8_t* a,
                               const float* a_scales, int b_fmt, const uint8_t* b,
                               const float* b_scales, int out, void* d, int64_t ldd,
                               const Epilogue& ep, int tensor_mask, hipStream_t stream) {
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E4M3)
        return launch_typed<BSFP8_E4M3, BSFP8_E4M3>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, tensor_mask, stream);
    if (a_fmt == BSFP8_E4M3 && b_fmt == BSFP8_E5M2)
        return launch_typed<BSFP8_E4M3, BSFP8_E5M2>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, tensor_mask, stream);
    if (a_fmt == BSFP8_E5M2 && b_fmt == BSFP8_E4M3)
        return launch_typed<BSFP8_E5M2, BSFP8_E4M3>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, tensor_mask, stream);
    return launch_typed<BSFP8_E5M2, BSFP8_E5M2>(M, N, K, a, a_scales, b, b_scales, out, d, ldd, ep, tensor_mask, stream);
}

}  // namespace bsfp8
