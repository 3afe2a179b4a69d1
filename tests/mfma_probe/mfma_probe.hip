// mfma_probe.hip -- test instrument: single matrix-core instructions of gfx950
// evaluated on caller-chosen dot products.
//
// Part of the test suite, not of the library: it runs one MFMA per 32 dot
// products so that the tests can observe the instruction's numerics (alignment
// bits, grouping of products, treatment of the accumulator input, final
// rounding), the feature-vector method of "Exact models of AMD matrix cores"
// (sections 2 and 3) applied to CDNA4.
//
// Case i of a batch is the dot product  d_i = sum_k a_i[k] b_i[k] + c_i  of one
// row of A with one column of B.  A wave puts 32 cases on the diagonal of one
// 32 x 32 output tile: row r of the instruction's A operand holds a_{base+r},
// column r of its B operand holds b_{base+r}, the accumulator input is c_i on
// the diagonal and +0 elsewhere, and only the diagonal of the result is written
// back.  Off-diagonal outputs mix different cases and are discarded.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Instruction selector (the values of the `instr` argument).
enum Instr {
    kFp8Fp8 = 0,    // v_mfma_f32_32x32x16_fp8_fp8   K = 16, A E4M3, B E4M3
    kFp8Bf8 = 1,    // v_mfma_f32_32x32x16_fp8_bf8   K = 16, A E4M3, B E5M2
    kBf8Fp8 = 2,    // v_mfma_f32_32x32x16_bf8_fp8   K = 16, A E5M2, B E4M3
    kBf8Bf8 = 3,    // v_mfma_f32_32x32x16_bf8_bf8   K = 16, A E5M2, B E5M2
    kBf16 = 4,      // v_mfma_f32_32x32x16_bf16      K = 16, bf16 bit patterns
    kScaleFp4 = 5,  // v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 x E2M1, E8M0 scales, K = 64
    kScaleE4m3 = 6, // the same instruction, E4M3 x E4M3, E8M0 scales, K = 64
    kScaleE5m2 = 7, // the same instruction, E5M2 x E5M2, E8M0 scales, K = 64
    kK64E4m3 = 8,   // v_mfma_f32_32x32x64_f8f6f4 (no scales), E4M3 x E4M3, K = 64
    kK64E5m2 = 9,   // the same, E5M2 x E5M2
    kNumInstr = 10
};

__device__ __forceinline__ int out_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int N>
__device__ __forceinline__ void load_bytes(uint8_t (&dst)[N], const uint8_t* src, bool ok) {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = ok ? src[i] : 0;
}

// One wave (64 lanes) per 32 cases.
__global__ __launch_bounds__(64) void probe_kernel(int instr, int64_t ncases, const uint8_t* __restrict__ A,
                                                   const uint8_t* __restrict__ B, const uint8_t* __restrict__ sA,
                                                   const uint8_t* __restrict__ sB, const float* __restrict__ C,
                                                   float* __restrict__ D) {
    const int lane = threadIdx.x;
    const int row = lane & 31;
    const int half = lane >> 5;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * 32;
    const int64_t mycase = base + row;      // the case this lane feeds as operand row/column
    const bool ok = mycase < ncases;

    v16f c;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = out_row(r, lane);
        c[r] = (i == row && ok) ? C[mycase] : 0.0f;
    }

    v16f d;
    if (instr <= kBf8Bf8) {
        uint8_t xa[8], xb[8];
        load_bytes(xa, A + mycase * 16 + 8 * half, ok);
        load_bytes(xb, B + mycase * 16 + 8 * half, ok);
        long a, b;
        __builtin_memcpy(&a, xa, 8);
        __builtin_memcpy(&b, xb, 8);
        if (instr == kFp8Fp8) d = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
        else if (instr == kFp8Bf8) d = __builtin_amdgcn_mfma_f32_32x32x16_fp8_bf8(a, b, c, 0, 0, 0);
        else if (instr == kBf8Fp8) d = __builtin_amdgcn_mfma_f32_32x32x16_bf8_fp8(a, b, c, 0, 0, 0);
        else d = __builtin_amdgcn_mfma_f32_32x32x16_bf8_bf8(a, b, c, 0, 0, 0);
    } else if (instr == kBf16) {
        uint8_t xa[16], xb[16];
        load_bytes(xa, A + (mycase * 16 + 8 * half) * 2, ok);
        load_bytes(xb, B + (mycase * 16 + 8 * half) * 2, ok);
        v8bf a, b;
        __builtin_memcpy(&a, xa, 16);
        __builtin_memcpy(&b, xb, 16);
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    } else if (instr >= kK64E4m3) {
        // same operand layout as the scaled instruction with 8-bit elements
        uint8_t lo_a[16], hi_a[16], lo_b[16], hi_b[16];
        load_bytes(lo_a, A + mycase * 64 + 16 * half, ok);
        load_bytes(hi_a, A + mycase * 64 + 32 + 16 * half, ok);
        load_bytes(lo_b, B + mycase * 64 + 16 * half, ok);
        load_bytes(hi_b, B + mycase * 64 + 32 + 16 * half, ok);
        uint8_t xa[32], xb[32];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            xa[i] = lo_a[i]; xa[16 + i] = hi_a[i];
            xb[i] = lo_b[i]; xb[16 + i] = hi_b[i];
        }
        v8i a, b;
        __builtin_memcpy(&a, xa, 32);
        __builtin_memcpy(&b, xb, 32);
        d = c;
        if (instr == kK64E4m3)
            asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0 cbsz:0 blgp:0" : "+v"(d) : "v"(a), "v"(b));
        else
            asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+v"(d) : "v"(a), "v"(b));
        // the result must settle before it is read
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d));
    } else {
        // Lane (row, half) supplies the E8M0 scale of K block `half` (K values
        // 32 half .. 32 half + 31) in byte 0 of its scale register.  E2M1
        // elements: registers 0-3 carry K values 32 half .. 32 half + 31.
        uint8_t xa[32] = {}, xb[32] = {};
        const uint32_t sa = ok ? sA[mycase * 2 + half] : 127u;
        const uint32_t sb = ok ? sB[mycase * 2 + half] : 127u;
        v8i a, b;
        if (instr == kScaleFp4) {
            uint8_t ta[16], tb[16];
            load_bytes(ta, A + mycase * 32 + 16 * half, ok);
            load_bytes(tb, B + mycase * 32 + 16 * half, ok);
#pragma unroll
            for (int i = 0; i < 16; ++i) { xa[i] = ta[i]; xb[i] = tb[i]; }
            __builtin_memcpy(&a, xa, 32);
            __builtin_memcpy(&b, xb, 32);
            d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, static_cast<int>(sa), 0,
                                                                static_cast<int>(sb));
        } else {
            // 8-bit elements: registers 0-3 carry K values 16 half .. 16 half + 15
            // and registers 4-7 carry K values 32 + 16 half .. 32 + 16 half + 15.
            uint8_t lo_a[16], hi_a[16], lo_b[16], hi_b[16];
            load_bytes(lo_a, A + mycase * 64 + 16 * half, ok);
            load_bytes(hi_a, A + mycase * 64 + 32 + 16 * half, ok);
            load_bytes(lo_b, B + mycase * 64 + 16 * half, ok);
            load_bytes(hi_b, B + mycase * 64 + 32 + 16 * half, ok);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                xa[i] = lo_a[i]; xa[16 + i] = hi_a[i];
                xb[i] = lo_b[i]; xb[16 + i] = hi_b[i];
            }
            __builtin_memcpy(&a, xa, 32);
            __builtin_memcpy(&b, xb, 32);
            if (instr == kScaleE4m3)
                d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, static_cast<int>(sa), 0,
                                                                    static_cast<int>(sb));
            else
                d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 1, 1, 0, static_cast<int>(sa), 0,
                                                                    static_cast<int>(sb));
        }
    }

#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = out_row(r, lane);
        if (i == row && ok) D[mycase] = d[r];
    }
}

}  // namespace

extern "C" {

// K of one instruction (products per dot product), or 0 for an unknown selector.
int mfma_probe_k(int instr) {
    if (instr < 0 || instr >= kNumInstr) return 0;
    return instr <= kBf16 ? 16 : 64;   // 5..9: K = 64
}

// Evaluate `ncases` dot products with instruction `instr` (see Instr above).
// All pointers are device pointers.  Operand storage per case:
//   instr 0-3: a, b: 16 FP8 codes each (a in the A format, b in the B format)
//   instr 4:   a, b: 16 bf16 bit patterns each (little-endian uint16)
//   instr 5:   a, b: 64 E2M1 values in 32 bytes, element 2i in the low nibble of byte i
//   instr 6-9: a, b: 64 FP8 codes each
//   instr 5-7: sa, sb: 2 E8M0 bytes per case (K values 0-31, then 32-63); unused otherwise
//   c: ncases FP32 accumulator inputs; d: ncases FP32 results.
// Returns 0 on success, 1 for a bad argument, 2 for a launch error.
int mfma_probe_dot(int instr, int64_t ncases, const void* a, const void* b, const void* sa, const void* sb,
                   const float* c, float* d, hipStream_t stream) {
    if (instr < 0 || instr >= kNumInstr || ncases < 0) return 1;
    if (ncases == 0) return 0;
    if (!a || !b || !c || !d) return 1;
    if (instr >= kScaleFp4 && instr <= kScaleE5m2 && (!sa || !sb)) return 1;
    const int64_t waves = (ncases + 31) / 32;
    if (waves > 0x7fffffff) return 1;
    hipLaunchKernelGGL(probe_kernel, dim3(static_cast<unsigned>(waves)), dim3(64), 0, stream, instr, ncases,
                       static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b),
                       static_cast<const uint8_t*>(sa), static_cast<const uint8_t*>(sb), c, d);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
