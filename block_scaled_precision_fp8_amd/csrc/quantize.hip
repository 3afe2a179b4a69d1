// quantize.hip -- FP8 per-tile and MXFP4 per-block quantisation kernels for gfx950.
//
// Both kernels are HBM-bound streaming passes: each FP32 element is read once
// with 16-byte loads, its tile or block maximum is reduced across the lanes
// holding that tile (cross-lane shuffles, then LDS for FP8 tiles), and the
// codes are written once.
//
// FP8 ("Why grind FP8 GEMM on CDNA4", sections 3.3 and 4.2): per 128 x 32
// tile, s = fl32(amax / F) (1 for an all-zero tile), code = satRNE(fl32(x / s)).
// The quotient, its clamp and the code conversion are in fp8_codec.h.
//
// MXFP4 ("Rubin FP4 GEMM deep dive", sections 2.1, 2.2, 3.1 and 4.2): per 32
// consecutive K elements, e = smallest integer with 6 * 2^e >= amax, read off
// the FP32 exponent and mantissa bits of amax; elements are scaled by the exact
// power of two 2^-e and converted with v_cvt_scalef32_pk_fp4_f32 (unit scale),
// which rounds to nearest even; two codes per byte, low nibble first.
#include "fp8_codec.h"

namespace bsfp8 {

namespace {

constexpr int kThreads = 256;

// The FP32 input is read exactly once: non-temporal loads keep it from
// displacing cached data (about 14% more bandwidth on large inputs).
__device__ __forceinline__ float4 load_once(const float* p) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}

// One workgroup quantises a 128-row x 128-column block = four 128 x 32 tiles.
// Thread t holds 16-byte chunk (t % 32) of rows (t / 32) + 8 i, i = 0..15, so a
// wave reads two full 512-byte row segments per load instruction and every
// thread's 64 values belong to a single tile (chunk / 8).
template <int FMT>
__device__ __forceinline__ void quantize_block(const float* __restrict__ x, int64_t rows, int64_t k,
                                               int64_t ld, uint8_t* __restrict__ codes,
                                               float* __restrict__ scales, int64_t ncol_blocks,
                                               int64_t bid, float (*red)[4]) {
    constexpr float F = FMT == BSFP8_E4M3 ? 448.0f : 57344.0f;
    const int64_t rt = bid / ncol_blocks;
    const int64_t cb = bid - rt * ncol_blocks;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int chunk = tid & 31;
    const int ro = tid >> 5;
    const int64_t col = cb * 128 + chunk * 4;
    const bool col_ok = col < k;  // k is a multiple of 32: whole tiles are in or out
    const int64_t r0 = rt * 128;
    const int64_t nkb = k >> 5;

    float4 v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t r = r0 + ro + 8 * i;
        if (col_ok && r < rows)
            v[i] = load_once(x + r * ld + col);
        else
            v[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        amax = fmaxf(amax, abs_max4(v[i]));
    }
    // The 16 lanes of a wave that hold one tile differ in lane bits 0, 1, 2 and 5.
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if ((lane & 0x27) == 0) red[wave][(lane >> 3) & 3] = amax;
    __syncthreads();

    const int t = chunk >> 3;
    amax = fmaxf(fmaxf(red[0][t], red[1][t]), fmaxf(red[2][t], red[3][t]));
    float s = amax / F;
    if (s == 0.0f) s = 1.0f;

    if (tid < 4 && cb * 128 + tid * 32 < k) {
        const float a = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
        float st = a / F;
        if (st == 0.0f) st = 1.0f;
        scales[rt * nkb + cb * 4 + tid] = st;
    }

    const Fp8Quotient qt(s);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t r = r0 + ro + 8 * i;
        if (!(col_ok && r < rows)) continue;
        *reinterpret_cast<uint32_t*>(codes + r * k + col) = fp8_codes4<FMT>(qt, v[i]);
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void fp8_quantize_kernel(
    const float* __restrict__ x, int64_t rows, int64_t k, int64_t ld,
    uint8_t* __restrict__ codes, float* __restrict__ scales, int64_t ncol_blocks) {
    __shared__ float red[4][4];
    quantize_block<FMT>(x, rows, k, ld, codes, scales, ncol_blocks, blockIdx.x, red);
}

// Two operands with the same K in one launch (the A and B of one GEMM): the
// first blocks_a workgroups take A's 128 x 128 blocks, the rest B's.  Each
// workgroup does exactly what fp8_quantize_kernel does for its block.
template <int FA, int FB>
__global__ __launch_bounds__(kThreads) void fp8_quantize_pair_kernel(
    const float* __restrict__ xa, int64_t rows_a, int64_t lda, uint8_t* __restrict__ codes_a,
    float* __restrict__ scales_a, int64_t blocks_a, const float* __restrict__ xb, int64_t rows_b,
    int64_t ldb, uint8_t* __restrict__ codes_b, float* __restrict__ scales_b, int64_t k,
    int64_t ncol_blocks) {
    __shared__ float red[4][4];
    const int64_t bid = blockIdx.x;
    if (bid < blocks_a)
        quantize_block<FA>(xa, rows_a, k, lda, codes_a, scales_a, ncol_blocks, bid, red);
    else
        quantize_block<FB>(xb, rows_b, k, ldb, codes_b, scales_b, ncol_blocks, bid - blocks_a, red);
}

// Transposing variant: x is k x rows row-major (for example a gradient or an
// activation stored token-major) and the result is the quantisation of x^T,
// i.e. rows x k codes with K contiguous, exactly as fp8_quantize would produce
// from an explicitly transposed copy.  One workgroup takes a 128 (k) x 128
// (rows) input block = four 32 x 128 tiles of x (128 x 32 tiles of x^T).
// Thread (chunk = t % 32, g = t / 32) loads 16-byte chunk `chunk` of input rows
// 4 g + 32 q + j (q, j = 0..3): each load instruction reads two whole
// 512-byte row segments, and each thread's 4 x 4 values per tile give, per
// column, 4 consecutive K codes that go to LDS as one 32-bit word.  The block
// is written back row by row of x^T with 16-byte stores.
constexpr int kTPitch = 132;    // LDS bytes per x^T row (128 codes + 4)

template <int FMT>
__global__ __launch_bounds__(kThreads) void fp8_quantize_t_kernel(
    const float* __restrict__ x, int64_t k, int64_t rows, int64_t ld,
    uint8_t* __restrict__ codes, float* __restrict__ scales, int64_t nrb) {
    constexpr float F = FMT == BSFP8_E4M3 ? 448.0f : 57344.0f;
    __shared__ float red[4][4];
    __shared__ __attribute__((aligned(16))) uint8_t tl[128 * kTPitch];

    const int64_t bid = blockIdx.x;
    const int64_t kt = bid / nrb;            // 128-wide K block
    const int64_t rb = bid - kt * nrb;       // 128-wide block of x^T rows (columns of x)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int chunk = tid & 31;
    const int g = tid >> 5;
    const int64_t k0 = kt * 128;
    const int64_t c0 = rb * 128 + chunk * 4;   // first x column of this thread
    const int64_t nkb = k >> 5;

    float4 v[4][4];
    float tmax[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        tmax[q] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t kr = k0 + 4 * g + 32 * q + j;
            float4 t = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (kr < k) {
                const float* p = x + kr * ld + c0;
                if (c0 + 3 < rows) {
                    t = load_once(p);
                } else {
                    if (c0 + 0 < rows) t.x = p[0];
                    if (c0 + 1 < rows) t.y = p[1];
                    if (c0 + 2 < rows) t.z = p[2];
                }
            }
            v[q][j] = t;
            tmax[q] = fmaxf(tmax[q], abs_max4(t));
        }
    }
    // every lane of a wave holds part of all four tiles: full-wave reductions
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) tmax[q] = fmaxf(tmax[q], __shfl_xor(tmax[q], m));
    }
    if (lane == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wave][q] = tmax[q];
    }
    __syncthreads();

    float sc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float a = fmaxf(fmaxf(red[0][q], red[1][q]), fmaxf(red[2][q], red[3][q]));
        float st = a / F;
        if (st == 0.0f) st = 1.0f;
        sc[q] = st;
    }
    if (tid < 4 && k0 + 32 * tid < k) scales[rb * nkb + kt * 4 + tid] = sc[tid];

#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const Fp8Quotient qt(sc[q]);
        // column jj of this thread: its K codes j = 0..3 packed into one word
        uint32_t wcol[4];
        wcol[0] = fp8_pack4<FMT>(qt(v[q][0].x, F), qt(v[q][1].x, F), qt(v[q][2].x, F), qt(v[q][3].x, F));
        wcol[1] = fp8_pack4<FMT>(qt(v[q][0].y, F), qt(v[q][1].y, F), qt(v[q][2].y, F), qt(v[q][3].y, F));
        wcol[2] = fp8_pack4<FMT>(qt(v[q][0].z, F), qt(v[q][1].z, F), qt(v[q][2].z, F), qt(v[q][3].z, F));
        wcol[3] = fp8_pack4<FMT>(qt(v[q][0].w, F), qt(v[q][1].w, F), qt(v[q][2].w, F), qt(v[q][3].w, F));
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            *reinterpret_cast<uint32_t*>(tl + (chunk * 4 + jj) * kTPitch + 4 * g + 32 * q) = wcol[jj];
    }
    __syncthreads();

    // write back: x^T row r (128 codes) as 8 x 16 bytes
    const int part = tid & 7;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int r = pass * 32 + (tid >> 3);
        const int64_t orow = rb * 128 + r;
        const int64_t ocol = k0 + 16 * part;
        if (orow >= rows || ocol >= k) continue;
        const uint8_t* src = tl + r * kTPitch + 16 * part;
        const uint4 w = make_uint4(*reinterpret_cast<const uint32_t*>(src),
                                   *reinterpret_cast<const uint32_t*>(src + 4),
                                   *reinterpret_cast<const uint32_t*>(src + 8),
                                   *reinterpret_cast<const uint32_t*>(src + 12));
        *reinterpret_cast<uint4*>(codes + orow * k + ocol) = w;
    }
}

// Rows in chunks of up to 4096 values, 16 per lane of a wave: lane l holds
// values 256 i + 4 l .. 256 i + 4 l + 3 (i = 0..15) of the chunk, so each load
// instruction reads 1 KB in lane order.  The loads are range-checked buffer
// loads over the chunk: values at or past the row's end read as zero with no
// branch, so all 16 are in flight together (a conditional load compiles to a
// branch that waits for the loads before it).  Stores past the end are dropped
// the same way.
constexpr int kChunk = 4096;
constexpr int kCachePolicyNT = 2;             // non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

// values [c0, min(c0 + 4096, n)) of row xr
template <bool NT>
__device__ __forceinline__ void load_chunk(const float* xr, int64_t c0, int64_t n, int lane, float4 (&v)[16]) {
    const __amdgpu_buffer_rsrc_t rs = span_rsrc(xr + c0, 4 * min(n - c0, static_cast<int64_t>(kChunk)));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, (i * 64 + lane) * 16, 0, NT ? kCachePolicyNT : 0);
        v[i] = make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                           __uint_as_float(w[3]));
    }
}

template <int FMT>
__device__ __forceinline__ void store_chunk(uint8_t* cr, int64_t c0, int64_t n, int lane, const Fp8Quotient& qt,
                                            const float4 (&v)[16]) {
    const __amdgpu_buffer_rsrc_t rs = span_rsrc(cr + c0, min(n - c0, static_cast<int64_t>(kChunk)));
#pragma unroll
    for (int i = 0; i < 16; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(fp8_codes4<FMT>(qt, v[i]), rs, (i * 64 + lane) * 4, 0, 0);
}

__device__ __forceinline__ float wave_max(float a) {
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    a = fmaxf(a, __shfl_xor(a, 8));
    a = fmaxf(a, __shfl_xor(a, 16));
    return fmaxf(a, __shfl_xor(a, 32));
}

__device__ __forceinline__ float chunk_max(const float4 (&v)[16]) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, abs_max4(v[i]));
    return a;
}

// Per-row scales ("Why grind FP8 GEMM on CDNA4", section 3.3 weighs per-row,
// per-column and per-tensor scales against per-tile ones): one wave per row,
// amax reduced across the wave, s = fl32(amax / F), then the codes.  A row of
// up to 4096 values stays in registers between the two steps; longer rows are
// read twice (the second time mostly from cache).  The per-row scales of a B
// operand stored N x K are its per-column scales.
template <int FMT, bool LONG>
__global__ __launch_bounds__(kThreads) void fp8_quantize_rows_kernel(
    const float* __restrict__ x, int64_t rows, int64_t k, int64_t ld,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
    constexpr float F = FMT == BSFP8_E4M3 ? 448.0f : 57344.0f;
    const int lane = threadIdx.x & 63;
    // wave-uniform, so the buffer resources built from it stay in scalar registers
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows) return;                    // the whole wave leaves together
    const float* xr = x + row * ld;
    uint8_t* cr = codes + row * k;
    float4 v[16];
    float amax = 0.0f;
    if constexpr (!LONG) {
        load_chunk<true>(xr, 0, k, lane, v);
        amax = chunk_max(v);
    } else {
        for (int64_t c0 = 0; c0 < k; c0 += kChunk) {
            load_chunk<false>(xr, c0, k, lane, v);
            amax = fmaxf(amax, chunk_max(v));
        }
    }
    amax = wave_max(amax);
    float s = amax / F;
    if (s == 0.0f) s = 1.0f;
    if (lane == 0) scales[row] = s;
    const Fp8Quotient qt(s);
    if constexpr (!LONG) {
        store_chunk<FMT>(cr, 0, k, lane, qt, v);
    } else {
        for (int64_t c0 = 0; c0 < k; c0 += kChunk) {
            load_chunk<false>(xr, c0, k, lane, v);
            store_chunk<FMT>(cr, c0, k, lane, qt, v);
        }
    }
}

// Per-tensor scale, in three launches on one stream: every workgroup of the
// first reduces the maximum |x| of its rows into one partial maximum; one
// workgroup then reduces the partials and stores s = fl32(amax / F); the last
// launch writes the codes.  The partials are kept in the code buffer, which
// the last launch overwrites in full (it holds at least 32 bytes per row, and
// there is one 4-byte partial per workgroup of at least 4 rows), so no
// workspace is needed and nothing has to be cleared first.
constexpr int kMaxPartials = 2048;

// One wave per row, as in the per-row kernel, striding over the rows.  These
// loads are ordinary ones, so the second pass over x finds much of it in cache.
__global__ __launch_bounds__(kThreads) void amax_kernel(const float* __restrict__ x, int64_t rows,
                                                        int64_t k, int64_t ld, float* partial) {
    __shared__ float red[4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    float amax = 0.0f;
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave; row < rows;
         row += static_cast<int64_t>(gridDim.x) * 4) {
        const float* xr = x + row * ld;
        float4 v[16];
        for (int64_t c0 = 0; c0 < k; c0 += kChunk) {
            load_chunk<false>(xr, c0, k, lane, v);
            amax = fmaxf(amax, chunk_max(v));
        }
    }
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void tensor_scale_kernel(const float* partial, int n, float* scale) {
    constexpr float F = FMT == BSFP8_E4M3 ? 448.0f : 57344.0f;
    __shared__ float red[4];
    float amax = 0.0f;
    for (int i = threadIdx.x; i < n; i += kThreads) amax = fmaxf(amax, partial[i]);
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / F;
        if (s == 0.0f) s = 1.0f;
        *scale = s;
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void fp8_quantize_tensor_kernel(
    const float* __restrict__ x, int64_t rows, int64_t k, int64_t ld, const float* scale,
    uint8_t* __restrict__ codes) {
    const int lane = threadIdx.x & 63;
    // wave-uniform, so the buffer resources built from it stay in scalar registers
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows) return;                    // the whole wave leaves together
    const Fp8Quotient qt(*scale);
    const float* xr = x + row * ld;
    uint8_t* cr = codes + row * k;
    float4 v[16];
    for (int64_t c0 = 0; c0 < k; c0 += kChunk) {
        load_chunk<true>(xr, c0, k, lane, v);
        store_chunk<FMT>(cr, c0, k, lane, qt, v);
    }
}

// One thread per 16-byte chunk (4 elements) of kMxRows rows (its loads all in
// flight before the first block is reduced: one 16-byte load per thread left
// too few bytes in flight to keep HBM busy); the 8 consecutive lanes of a
// 32-element block reduce their maximum with three shuffles.
constexpr int kMxRows = 4;

__global__ __launch_bounds__(kThreads) void mxfp4_quantize_kernel(
    const float* __restrict__ x, int64_t rows, int64_t k, int64_t ld, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales, int64_t chunks_per_row, int64_t total) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const bool in = g < total;                       // total = row groups x chunks per row
    const int64_t rg = in ? g / chunks_per_row : 0;
    const int64_t c = in ? g - rg * chunks_per_row : 0;

    float4 v[kMxRows];
#pragma unroll
    for (int j = 0; j < kMxRows; ++j) {
        const int64_t r = rg * kMxRows + j;
        v[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (in && r < rows) v[j] = load_once(x + r * ld + 4 * c);
    }
#pragma unroll
    for (int j = 0; j < kMxRows; ++j) {
        const int64_t r = rg * kMxRows + j;
        float amax = abs_max4(v[j]);
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));

        // e = ceil(log2(amax / 6)) from the bits of amax = f * 2^E, f in [1, 2):
        // e = E - 2 when f <= 1.5, else E - 1; subnormal amax clamps to -127.
        const uint32_t u = __float_as_uint(amax);
        int e;
        if (amax == 0.0f) {
            e = 0;
        } else if (u < 0x00800000u) {
            e = -127;
        } else {
            e = static_cast<int>(u >> 23) - 127 - 2 + ((u & 0x007FFFFFu) > 0x00400000u ? 1 : 0);
            if (e < -127) e = -127;
        }
        // 2^-e as an FP32 bit pattern; finite amax gives e <= 126, so the exponent field is >= 1.
        const float y = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);

        if (in && r < rows) {
            int w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0, v[j].x * y, v[j].y * y, 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[j].z * y, v[j].w * y, 1.0f, 1);
            *reinterpret_cast<uint16_t*>(packed + r * (k >> 1) + 2 * c) = static_cast<uint16_t>(w & 0xFFFF);
            if ((c & 7) == 0) scales[r * (k >> 5) + (c >> 3)] = static_cast<uint8_t>(e + 127);
        }
    }
}

// MX variants ("Rubin FP4 GEMM deep dive", section 5.3: blocks of 16 or 8
// elements; section 3.2: FP16 or BF16 block scales).  One thread per 16-byte
// chunk as above; the BLOCK / 4 lanes of a block reduce their maximum with
// shuffles.  E8M0 scales follow the MXFP4 rule.  A wide scale is the FP16 or
// BF16 value nearest to amax / 6: the quotient is formed in FP64 (no FP64
// rounding can land on a midpoint of the narrow format unless the quotient
// itself is one, since amax / 6 has a repeating binary expansion) and rounded
// to P significand bits with an integer round-half-even on its significand;
// it saturates at the format's largest value and is 1 when it is zero.  The
// codes are then satRNE_E2M1(fl32(x / s)), the per-tile FP8 rule with F = 6.
template <int P, int EMIN>
__device__ __forceinline__ float nearest_scale(float amax, float vmax) {
    if (amax == 0.0f) return 1.0f;
    const double q = static_cast<double>(amax) / 6.0;            // normal in FP64
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(q));
    const int e = static_cast<int>((u >> 52) & 0x7FF) - 1023;     // q in [2^e, 2^(e+1))
    const uint64_t m = (u & ((uint64_t(1) << 52) - 1)) | (uint64_t(1) << 52);
    const int lsb = (e > EMIN ? e : EMIN) - (P - 1);              // exponent of the last kept bit
    const int sh = lsb - (e - 52);                                // >= 53 - P
    uint64_t n;
    if (sh >= 54) {
        n = 0;                                                    // below half the smallest subnormal
    } else {
        n = m >> sh;
        const uint64_t rem = m & ((uint64_t(1) << sh) - 1);
        const uint64_t half = uint64_t(1) << (sh - 1);
        if (rem > half || (rem == half && (n & 1))) ++n;
    }
    float s = __builtin_ldexpf(static_cast<float>(n), lsb);       // exact: n has at most P + 1 bits
    if (s > vmax) s = vmax;
    return s == 0.0f ? 1.0f : s;
}

template <int BLOCK, int SFMT>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(
    const float* __restrict__ x, int64_t rows, int64_t k, int64_t ld, uint8_t* __restrict__ packed,
    void* __restrict__ scales, int64_t chunks_per_row, int64_t total) {
    constexpr int kChunks = BLOCK / 4;
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const bool in = g < total;                       // total = row groups x chunks per row
    const int64_t rg = in ? g / chunks_per_row : 0;
    const int64_t c = in ? g - rg * chunks_per_row : 0;

    float4 v[kMxRows];
#pragma unroll
    for (int j = 0; j < kMxRows; ++j) {
        const int64_t r = rg * kMxRows + j;
        v[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (in && r < rows) v[j] = load_once(x + r * ld + 4 * c);
    }
#pragma unroll
    for (int j = 0; j < kMxRows; ++j) {
        const int64_t r = rg * kMxRows + j;
        const bool ok = in && r < rows;
        float amax = abs_max4(v[j]);
#pragma unroll
        for (int o = 1; o < kChunks; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));

        int w = 0;
        if constexpr (SFMT == BSFP8_MX_E8M0) {
            const uint32_t u = __float_as_uint(amax);
            int e;
            if (amax == 0.0f) {
                e = 0;
            } else if (u < 0x00800000u) {
                e = -127;
            } else {
                e = static_cast<int>(u >> 23) - 127 - 2 + ((u & 0x007FFFFFu) > 0x00400000u ? 1 : 0);
                if (e < -127) e = -127;
            }
            const float y = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
            if (ok) {
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0, v[j].x * y, v[j].y * y, 1.0f, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[j].z * y, v[j].w * y, 1.0f, 1);
                if ((c % kChunks) == 0)
                    static_cast<uint8_t*>(scales)[r * (k / BLOCK) + c / kChunks] = static_cast<uint8_t>(e + 127);
            }
        } else {
            const float sc = SFMT == BSFP8_MX_F16 ? nearest_scale<11, -14>(amax, 65504.0f)
                                                  : nearest_scale<8, -126>(amax, __uint_as_float(0x7F7F0000u));
            if (ok) {
                const Fp8Quotient qt(sc);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0, qt(v[j].x, 6.0f), qt(v[j].y, 6.0f), 1.0f, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, qt(v[j].z, 6.0f), qt(v[j].w, 6.0f), 1.0f, 1);
                if ((c % kChunks) == 0) {
                    const uint16_t bits = SFMT == BSFP8_MX_F16 ? __builtin_bit_cast(uint16_t, static_cast<_Float16>(sc))
                                                               : static_cast<uint16_t>(__float_as_uint(sc) >> 16);
                    static_cast<uint16_t*>(scales)[r * (k / BLOCK) + c / kChunks] = bits;
                }
            }
        }
        if (ok) *reinterpret_cast<uint16_t*>(packed + r * (k >> 1) + 2 * c) = static_cast<uint16_t>(w & 0xFFFF);
    }
}

// K = 0: D = beta * C, or zeros.
template <int OUT>
__global__ __launch_bounds__(kThreads) void fill_kernel(int64_t M, int64_t N, void* d, int64_t ldd,
                                                         Epilogue ep) {
    const int64_t total = M * N;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int64_t r = i / N, c = i - r * N;
        float v = 0.0f;
        if (ep.beta != 0.0f) {
            if constexpr (OUT == BSFP8_OUT_F32)
                v = ep.beta * static_cast<const float*>(ep.c)[r * ep.ldc + c];
            else
                v = ep.beta * from_half_bits<OUT>(static_cast<const uint16_t*>(ep.c)[r * ep.ldc + c]);
        }
        if constexpr (OUT == BSFP8_OUT_F32)
            static_cast<float*>(d)[r * ldd + c] = v;
        else
            static_cast<uint16_t*>(d)[r * ldd + c] = to_half_bits<OUT>(v);
    }
}

}  // namespace

hipError_t launch_fp8_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int fmt,
                               uint8_t* codes, float* scales, hipStream_t stream) {
    const int64_t nrt = (rows + 127) / 128;
    const int64_t ncb = (k + 127) / 128;
    const int64_t blocks = nrt * ncb;
    if (blocks == 0) return hipSuccess;
    if (fmt == BSFP8_E4M3)
        hipLaunchKernelGGL(fp8_quantize_kernel<BSFP8_E4M3>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(kThreads), 0, stream, x, rows, k, ld, codes, scales, ncb);
    else
        hipLaunchKernelGGL(fp8_quantize_kernel<BSFP8_E5M2>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(kThreads), 0, stream, x, rows, k, ld, codes, scales, ncb);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize_pair(const float* a, int64_t rows_a, int64_t lda, int fmt_a,
                                    uint8_t* codes_a, float* scales_a, const float* b, int64_t rows_b,
                                    int64_t ldb, int fmt_b, uint8_t* codes_b, float* scales_b, int64_t k,
                                    hipStream_t stream) {
    const int64_t ncb = (k + 127) / 128;
    const int64_t blocks_a = (rows_a + 127) / 128 * ncb;
    const int64_t blocks = blocks_a + (rows_b + 127) / 128 * ncb;
    if (blocks == 0) return hipSuccess;
    const dim3 g(static_cast<uint32_t>(blocks));
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, g, dim3(kThreads), 0, stream, a, rows_a, lda, codes_a, scales_a,
                           blocks_a, b, rows_b, ldb, codes_b, scales_b, k, ncb);
    };
    if (fmt_a == BSFP8_E4M3 && fmt_b == BSFP8_E4M3)
        go(fp8_quantize_pair_kernel<BSFP8_E4M3, BSFP8_E4M3>);
    else if (fmt_a == BSFP8_E4M3)
        go(fp8_quantize_pair_kernel<BSFP8_E4M3, BSFP8_E5M2>);
    else if (fmt_b == BSFP8_E4M3)
        go(fp8_quantize_pair_kernel<BSFP8_E5M2, BSFP8_E4M3>);
    else
        go(fp8_quantize_pair_kernel<BSFP8_E5M2, BSFP8_E5M2>);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize_t(const float* x, int64_t k, int64_t rows, int64_t ld, int fmt,
                                 uint8_t* codes, float* scales, hipStream_t stream) {
    const int64_t nkt = (k + 127) / 128;
    const int64_t nrb = (rows + 127) / 128;
    const int64_t blocks = nkt * nrb;
    if (blocks == 0) return hipSuccess;
    if (fmt == BSFP8_E4M3)
        hipLaunchKernelGGL(fp8_quantize_t_kernel<BSFP8_E4M3>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(kThreads), 0, stream, x, k, rows, ld, codes, scales, nrb);
    else
        hipLaunchKernelGGL(fp8_quantize_t_kernel<BSFP8_E5M2>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(kThreads), 0, stream, x, k, rows, ld, codes, scales, nrb);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize_rows(const float* x, int64_t rows, int64_t k, int64_t ld, int fmt,
                                    uint8_t* codes, float* scales, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>((rows + 3) / 4));
    // separate kernels: the loop over long rows would raise the register use
    // (and lower the occupancy) of the common one
    const bool long_rows = k > kChunk;
    if (fmt == BSFP8_E4M3) {
        if (long_rows) hipLaunchKernelGGL((fp8_quantize_rows_kernel<BSFP8_E4M3, true>), grid, dim3(kThreads), 0, stream, x, rows, k, ld, codes, scales);
        else hipLaunchKernelGGL((fp8_quantize_rows_kernel<BSFP8_E4M3, false>), grid, dim3(kThreads), 0, stream, x, rows, k, ld, codes, scales);
    } else {
        if (long_rows) hipLaunchKernelGGL((fp8_quantize_rows_kernel<BSFP8_E5M2, true>), grid, dim3(kThreads), 0, stream, x, rows, k, ld, codes, scales);
        else hipLaunchKernelGGL((fp8_quantize_rows_kernel<BSFP8_E5M2, false>), grid, dim3(kThreads), 0, stream, x, rows, k, ld, codes, scales);
    }
    return hipGetLastError();
}

hipError_t launch_fp8_quantize_tensor(const float* x, int64_t rows, int64_t k, int64_t ld, int fmt,
                                      uint8_t* codes, float* scales, hipStream_t stream) {
    const int64_t wgs = (rows + 3) / 4;
    const int parts = static_cast<int>(min(wgs, static_cast<int64_t>(kMaxPartials)));
    float* partial = reinterpret_cast<float*>(codes);     // rows * k >= 32 * rows bytes
    hipLaunchKernelGGL(amax_kernel, dim3(parts), dim3(kThreads), 0, stream, x, rows, k, ld, partial);
    const dim3 grid(static_cast<uint32_t>(wgs));
    if (fmt == BSFP8_E4M3) {
        hipLaunchKernelGGL(tensor_scale_kernel<BSFP8_E4M3>, dim3(1), dim3(kThreads), 0, stream, partial, parts, scales);
        hipLaunchKernelGGL(fp8_quantize_tensor_kernel<BSFP8_E4M3>, grid, dim3(kThreads), 0, stream, x, rows, k, ld, scales, codes);
    } else {
        hipLaunchKernelGGL(tensor_scale_kernel<BSFP8_E5M2>, dim3(1), dim3(kThreads), 0, stream, partial, parts, scales);
        hipLaunchKernelGGL(fp8_quantize_tensor_kernel<BSFP8_E5M2>, grid, dim3(kThreads), 0, stream, x, rows, k, ld, scales, codes);
    }
    return hipGetLastError();
}

template <int BLOCK, int SFMT>
hipError_t launch_mx_typed(const float* x, int64_t rows, int64_t k, int64_t ld, uint8_t* packed,
                           void* scales, hipStream_t stream) {
    const int64_t cpr = k / 4;
    const int64_t total = ((rows + kMxRows - 1) / kMxRows) * cpr;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((mx_quantize_kernel<BLOCK, SFMT>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kThreads), 0, stream, x, rows, k, ld, packed, scales, cpr, total);
    return hipGetLastError();
}

template <int BLOCK>
hipError_t launch_mx_block(const float* x, int64_t rows, int64_t k, int64_t ld, int sfmt,
                           uint8_t* packed, void* scales, hipStream_t stream) {
    if (sfmt == BSFP8_MX_E8M0) return launch_mx_typed<BLOCK, BSFP8_MX_E8M0>(x, rows, k, ld, packed, scales, stream);
    if (sfmt == BSFP8_MX_F16) return launch_mx_typed<BLOCK, BSFP8_MX_F16>(x, rows, k, ld, packed, scales, stream);
    return launch_mx_typed<BLOCK, BSFP8_MX_BF16>(x, rows, k, ld, packed, scales, stream);
}

hipError_t launch_mx_quantize(const float* x, int64_t rows, int64_t k, int64_t ld, int block,
                              int sfmt, uint8_t* packed, void* scales, hipStream_t stream) {
    if (block == 32) return launch_mx_block<32>(x, rows, k, ld, sfmt, packed, scales, stream);
    if (block == 16) return launch_mx_block<16>(x, rows, k, ld, sfmt, packed, scales, stream);
    return launch_mx_block<8>(x, rows, k, ld, sfmt, packed, scales, stream);
}

hipError_t launch_mxfp4_quantize(const float* x, int64_t rows, int64_t k, int64_t ld,
                                 uint8_t* packed, uint8_t* scales, hipStream_t stream) {
    const int64_t cpr = k / 4;
    const int64_t total = ((rows + kMxRows - 1) / kMxRows) * cpr;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(mxfp4_quantize_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads),
                       0, stream, x, rows, k, ld, packed, scales, cpr, total);
    return hipGetLastError();
}

hipError_t launch_fill(int64_t M, int64_t N, int out, void* d, int64_t ldd, const Epilogue& ep,
                       hipStream_t stream) {
    const int64_t total = M * N;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    const dim3 g(static_cast<uint32_t>(blocks));
    if (out == BSFP8_OUT_F32)
        hipLaunchKernelGGL(fill_kernel<BSFP8_OUT_F32>, g, dim3(kThreads), 0, stream, M, N, d, ldd, ep);
    else if (out == BSFP8_OUT_BF16)
        hipLaunchKernelGGL(fill_kernel<BSFP8_OUT_BF16>, g, dim3(kThreads), 0, stream, M, N, d, ldd, ep);
    else
        hipLaunchKernelGGL(fill_kernel<BSFP8_OUT_F16>, g, dim3(kThreads), 0, stream, M, N, d, ldd, ep);
    return hipGetLastError();
}

}  // namespace bsfp8
