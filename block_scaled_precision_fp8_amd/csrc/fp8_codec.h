// fp8_codec.h -- FP32 -> FP8 encoding pieces shared by the quantisers and the
// GEMM that quantises its A operand while loading it.
//
// Per 128 x 32 tile ("Why grind FP8 GEMM on CDNA4", sections 3.3 and 4.2):
// s = fl32(amax / F) (1 for an all-zero tile), code = satRNE(fl32(x / s)).
// The quotient fl32(x / s) is obtained without a per-element division, by
// Markstein's correction step: with r the correctly rounded reciprocal of s
// and q0 = fl32(x r), RN(q0 + r (x - s q0)) is the correctly rounded x / s,
// provided the residual x - s q0 (one FMA) is exact, i.e. does not underflow.
// Saturation is an explicit clamp to +-F, after which the hardware
// v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 conversion is exact round-to-nearest-even.
#pragma once

#include "internal.h"

namespace bsfp8 {

template <int FMT>
__device__ __forceinline__ constexpr float fp8_max() {
    return FMT == BSFP8_E4M3 ? 448.0f : 57344.0f;
}

__device__ __forceinline__ float abs_max4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// fl32(x / s) clamped to +-F, for any scale.  Both x and s are first scaled by
// the same power of two (exact, quotient unchanged) so that the scaled s lies
// in [1/2, 1); the residual can then underflow only when |x / s| < 2^-99,
// where every FP8 code is a signed zero and the sign is restored from x.
// (Checked against IEEE division on 1.7e10 in-range pairs per format, zero
// code mismatches.)
struct Fp8Quotient {
    int se;
    float ss, rs;
    __device__ explicit Fp8Quotient(float s) {
        (void)__builtin_frexpf(s, &se);
        ss = __builtin_ldexpf(s, -se);     // s 2^k in [1/2, 1)
        rs = 1.0f / ss;                    // correctly rounded
    }
    __device__ float operator()(float x, float F) const {
        const float xs = __builtin_ldexpf(x, -se);
        const float q0 = xs * rs;
        const float e = __builtin_fmaf(-q0, ss, xs);
        const float q = __builtin_copysignf(__builtin_fmaf(e, rs, q0), x);
        return fminf(fmaxf(q, -F), F);
    }
};

// The same quotient without the power-of-two scaling, for s >= 2^-82 (four
// operations per element instead of six).  The residual is exact for
// |x| >= 2^-100; a smaller |x| has |x / s| < 2^-18, below half the smallest
// subnormal of either format, so its code is a zero whatever the last bits of
// the quotient.  The residual is formed as s q0 - x and subtracted, so that a
// zero x (q0 = x r, a zero of x's sign) yields a zero of x's sign.  (Checked
// against IEEE division on 5.1e8 pairs over both formats, including scales
// near 2^-82 and tiny x: no quotient of magnitude 2^-18 or more differs, and
// no sign differs.)
constexpr float kNearScaleMin = 0x1p-82f;
struct Fp8QuotientNear {
    float s, r;
    __device__ explicit Fp8QuotientNear(float s_) : s(s_), r(1.0f / s_) {}
    __device__ float operator()(float x, float F) const {
        const float q0 = x * r;
        const float e = __builtin_fmaf(q0, s, -x);
        return __builtin_amdgcn_fmed3f(__builtin_fmaf(-e, r, q0), -F, F);
    }
};

// Four clamped quotients -> four FP8 codes (round to nearest even), byte i = qi.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_pack4(float q0, float q1, float q2, float q3) {
    int w;
    if constexpr (FMT == BSFP8_E4M3) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(q0, q1, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(q2, q3, w, true);
    }
    return static_cast<uint32_t>(w);
}

template <int FMT, class Q>
__device__ __forceinline__ uint32_t fp8_codes4(const Q& qt, float4 v) {
    constexpr float F = fp8_max<FMT>();
    return fp8_pack4<FMT>(qt(v.x, F), qt(v.y, F), qt(v.z, F), qt(v.w, F));
}

}  // namespace bsfp8
