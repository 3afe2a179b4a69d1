// big_tile.h -- pieces shared by the 256 x 256-tile GEMM kernels (gfx950):
// ordered LDS access as inline assembly, compile-time loops, and the epilogue
// that writes a 256 x 256 tile of 4 x 4 MFMA 32 x 32 accumulators per wave.
#pragma once

#include "internal.h"

#include <utility>

namespace bsfp8 {
namespace big_tile {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_byte;

// The main loop of the large-tile kernel issues its LDS traffic and MFMAs as
// volatile inline assembly: volatile statements keep their program order, so
// the fragment reads for the next K step, the staging writes and the MFMAs of
// the current step interleave exactly as written (the compiler would otherwise
// sink every read next to its first use and stall each MFMA on LDS latency).
// The compiler does not track LDS completions of these statements, so each
// consumer is preceded by an explicit lgkmcnt wait.
template <int OFF>
__device__ __forceinline__ void lds_read16(u32x4& v, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_write16(uint32_t addr, const u32x4& v) {
    asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_wait_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The epilogue's per-element hook when nothing scales the accumulators.
struct NoScale {
    __device__ void load(int) {}
    __device__ float operator()(int, int, int, float v) const { return v; }
};

// Epilogue of a 256 x 256 tile.  Wave w = (wm, wn) = (w & 1, w >> 1) holds
// acc[ti][tj][4 q + e] = tile element (wm 128 + 32 tj + lane % 32,
// wn 128 + 32 ti + 8 q + 4 (lane / 32) + e), i.e. B is the MFMA row operand.
// pre(ti, tj, r, v) returns the value stored for accumulator element r of MFMA
// tile (ti, tj) (a per-element scale, or v itself); pre.load(ti) is called
// before the elements of row-operand tile ti are used.  alpha, beta * C and
// the output conversion follow.  STAGE16 selects the one-pass converted staging
// for 16-bit output with beta == 0.  Uses 128 KB of LDS from lds; all of the
// workgroup's threads must call it.
template <int OUT, bool STAGE16, class Pre>
__device__ __forceinline__ void epilogue(v16f (&acc)[4][4], uint8_t* lds, int wave, int lane, int m0,
                                         int n0, int M, int N, void* D, int64_t ldd,
                                         const Epilogue& ep, int vec_ok, Pre& pre) {
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    // Epilogue: the tile goes out through LDS (free now) so that every store
    // instruction writes whole rows (the MFMA layout would give 32 rows x 16
    // bytes).  16-byte chunk c of LDS row R sits at c ^ (R & 15), which keeps
    // both the scattered writes and the row reads free of bank conflicts.
    __syncthreads();
    if constexpr (STAGE16) {
        static_assert(OUT != BSFP8_OUT_F32, "converted staging is for 16-bit outputs");
        {
            // 16-bit output without C: alpha * acc converted while staged,
            // 256 rows x 512 bytes = the whole 128 KB in one pass
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                pre.load(ti);
#pragma unroll
                for (int tj = 0; tj < 4; ++tj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int R = wm * 128 + tj * 32 + frag_row;
                        const int c = wn * 16 + ti * 4 + q;
                        const uint32_t h0 = to_half_bits<OUT>(ep.alpha * pre(ti, tj, 4 * q + 0, acc[ti][tj][4 * q + 0]));
                        const uint32_t h1 = to_half_bits<OUT>(ep.alpha * pre(ti, tj, 4 * q + 1, acc[ti][tj][4 * q + 1]));
                        const uint32_t h2 = to_half_bits<OUT>(ep.alpha * pre(ti, tj, 4 * q + 2, acc[ti][tj][4 * q + 2]));
                        const uint32_t h3 = to_half_bits<OUT>(ep.alpha * pre(ti, tj, 4 * q + 3, acc[ti][tj][4 * q + 3]));
                        *reinterpret_cast<uint2*>(lds + R * 512 + ((c ^ (R & 15)) << 4) + 8 * half) =
                            make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
                    }
            }
            __syncthreads();
#pragma unroll 4
            for (int i = 0; i < 32; ++i) {
                const int R = wave * 64 + 2 * i + half;
                const int c = lane & 31;
                const uint4 w = *reinterpret_cast<const uint4*>(lds + R * 512 + ((c ^ (R & 15)) << 4));
                store_half8(D, ldd, m0 + R, n0 + c * 8, M, N, vec_ok, w);
            }
            return;
        }
    }
    // General case: the FP32 tile in two passes of 128 rows x 1 KB; alpha,
    // beta * C and the output conversion are applied in the row phase.
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (wm == p) {
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                pre.load(ti);
#pragma unroll
                for (int tj = 0; tj < 4; ++tj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int R = tj * 32 + frag_row;
                        const int c = wn * 32 + ti * 8 + q * 2 + half;
                        *reinterpret_cast<float4*>(lds + R * 1024 + ((c ^ (R & 15)) << 4)) =
                            make_float4(pre(ti, tj, 4 * q + 0, acc[ti][tj][4 * q + 0]),
                                        pre(ti, tj, 4 * q + 1, acc[ti][tj][4 * q + 1]),
                                        pre(ti, tj, 4 * q + 2, acc[ti][tj][4 * q + 2]),
                                        pre(ti, tj, 4 * q + 3, acc[ti][tj][4 * q + 3]));
                    }
            }
        }
        __syncthreads();
        if constexpr (OUT == BSFP8_OUT_F32) {
#pragma unroll 4
            for (int i = 0; i < 32; ++i) {
                const int R = wave * 32 + i;
                const int c = lane;
                const float4 v = *reinterpret_cast<const float4*>(lds + R * 1024 + ((c ^ (R & 15)) << 4));
                const float a4[4] = {v.x, v.y, v.z, v.w};
                finish_row_chunk<OUT, 4>(D, ldd, ep, m0 + p * 128 + R, n0 + c * 4, M, N, vec_ok, a4);
            }
        } else {
#pragma unroll 4
            for (int i = 0; i < 16; ++i) {
                const int R = wave * 32 + i * 2 + half;
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

}  // namespace big_tile
}  // namespace bsfp8
