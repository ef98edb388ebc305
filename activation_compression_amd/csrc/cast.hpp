// cast.hpp -- shared device code of the activation kernels: 16-value BF16
// loads, |x| maxima on BF16 bit patterns, and the correctly rounded E4M3 cast
// y = RN32(448 x / a) (power-of-two prescale of a into [1, 2), RN reciprocal,
// one Markstein correction), round to nearest even, clamped to +-448.
#pragma once

#include "device.hpp"

namespace coat {

// Abs-max bits (low 16 = BF16 pattern) of 16 BF16 values held in 8 dwords.
__device__ __forceinline__ uint32_t absmax16(const uint32_t w[8]) {
    uint32_t acc = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = pk_absmax_u16(acc, w[i]);
    return max(acc & 0xFFFFu, acc >> 16);
}

__device__ __forceinline__ void load16(const uint16_t *p, uint32_t w[8]) {
    const uint4 a = reinterpret_cast<const uint4 *>(p)[0];
    const uint4 b = reinterpret_cast<const uint4 *>(p)[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Scaling constants for a (non-negative) absmax a: a = a_s 2^-sh, a_s in [1, 2).
struct CastQ {
    int sh;       // x 2^sh lies in [-2, 2] (exact: a power-of-two scale)
    float a_s;    // prescaled absmax
    float inv_s;  // RN(1 / a_s)
    float m448;   // 448, or 0 for an all-zero tensor / slice (every code 0)
};

__device__ __forceinline__ CastQ cast_q(float a) {
    CastQ q;
    if (!(a > 0.0f)) {
        q.sh = 0; q.a_s = 1.0f; q.inv_s = 1.0f; q.m448 = 0.0f;
        return q;
    }
    int e;
    const float ma = frexpf(a, &e);
    q.a_s = 2.0f * ma;
    q.sh = 1 - e;
    q.inv_s = 1.0f / q.a_s;
    q.m448 = 448.0f;
    return q;
}

// E4M3 codes of 16 BF16 values.  448 (x 2^sh) is exact -- a BF16 value in
// [-2, 2] times 7 * 2^6 has at most 11 significant bits -- and neither factor
// leaves the FP32 range for any finite BF16 slice, however large or small.
// kAnyScale: a may be below max |x| (a scale the caller supplies); x 2^sh is
// then clamped to +-2^100 first, which saturates all the same, so that the
// product cannot overflow to infinity and the quotient's correction cannot
// turn it into NaN.
template <bool kAnyScale = false>
__device__ __forceinline__ uint4 cast16(const uint32_t w[8], const CastQ &q) {
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float x = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
        float xs = __builtin_amdgcn_ldexpf(x, q.sh);
        if constexpr (kAnyScale) xs = __builtin_amdgcn_fmed3f(xs, -0x1p100f, 0x1p100f);
        const float t = div_rn_from_rcp(xs * q.m448, q.a_s, q.inv_s);
        y[i] = __builtin_amdgcn_fmed3f(t, -448.0f, 448.0f);
    }
    return make_uint4(cvt4<kE4M3>(y[0], y[1], y[2], y[3]), cvt4<kE4M3>(y[4], y[5], y[6], y[7]),
                      cvt4<kE4M3>(y[8], y[9], y[10], y[11]), cvt4<kE4M3>(y[12], y[13], y[14], y[15]));
}

}  // namespace coat
