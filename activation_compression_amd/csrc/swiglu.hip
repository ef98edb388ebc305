// swiglu.hip -- SwiGLU with Group Scaling stage 1 fused into its epilogue,
// for gfx950.
//
// "COAT: compressing optimizer states and activations for memory-efficient
// FP8 training" explainer (blog.daoxuan.cc/posts/57954): GLU-type activations
// produce the outlier-heavy tensors of section "why activations are hard";
// section "mixed granularity" gives the tensor SwiGLU produces (the input of
// the down projection, a linear layer) one per-tensor E4M3 scale, whose
// absmax is found in two stages, the first fused into the producing op --
// here -- so that it costs 4/G extra bytes per element instead of a second
// read of the tensor.  The same pass can also save SwiGLU's own inputs (gate,
// up: a nonlinear layer's input) in 1xG E4M3 for the backward pass.
//
// Per element h = silu(g) * u in FP32 (silu(g) = g / (1 + 2^(-g log2 e)),
// native exp2 and reciprocal), stored as BF16 (round to nearest even); the
// slice maxima are taken over |h| as stored.  Each lane owns 16 consecutive
// elements; a 1xG slice is G/16 adjacent lanes; one 1024-element chunk per
// wave.  Gates below -80 take a second, exponent-split form (see swiglu_far),
// run only by lanes that hold one.
#include "cast.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace coat {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// Gates below this take swiglu_far: there e^-g > 2^115 nears the top of FP32
// and silu(g) itself reaches FP32's denormals from g < -87.3, while the
// product with u can still be a normal number.
constexpr float kFarGate = -80.0f;

// silu(g) u for g >= kFarGate.
__device__ __forceinline__ float swiglu_near(float g, float u) {
    return (g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * kLog2e))) * u;
}

// silu(g) u for g < kFarGate.  silu(g) = g e^g / (1 + e^g) is g e^g to within
// e^g < 2^-115 relative, and |g e^g u| = (mg mu 2^f) 2^(eg + eu + n) with
// |g| = mg 2^eg and |u| = mu 2^eu split exactly (frexp) and g log2 e = n + f
// (n = rint, f exact): every factor stays normal and the power of two is
// applied last, so h is rounded at its own magnitude.  The sign is that of
// -u (g < 0).  A gate so negative that g log2 e overflows gives n = -1024
// (clamped, to keep the exponent an int), f = -inf and h = 0.
__device__ __forceinline__ float swiglu_far(float g, float u) {
    const float t = g * kLog2e;
    const float n = __builtin_fmaxf(__builtin_rintf(t), -1024.0f);
    const float ag = __builtin_fabsf(g), au = __builtin_fabsf(u);
    const float m = (__builtin_amdgcn_frexp_mantf(ag) * __builtin_amdgcn_frexp_mantf(au)) *
                    __builtin_amdgcn_exp2f(t - n);
    const float mag = __builtin_amdgcn_ldexpf(
        m, __builtin_amdgcn_frexp_expf(ag) + __builtin_amdgcn_frexp_expf(au) + (int)n);
    return with_sign_of(mag, -u);
}

template <int G, bool kSaveInputs>
__global__ __launch_bounds__(kBlock) void swiglu_fused_kernel(const uint16_t *__restrict__ gate,
                                                              const uint16_t *__restrict__ up, int64_t n,
                                                              int64_t n_chunks, uint16_t *__restrict__ h_out,
                                                              float *__restrict__ h_partial,
                                                              uint8_t *__restrict__ gate_codes,
                                                              float *__restrict__ gate_scales,
                                                              uint8_t *__restrict__ up_codes,
                                                              float *__restrict__ up_scales) {
    constexpr int LPG = G / 16;
    const int lane = threadIdx.x & 63;
    const int64_t chunk = xcd_block(blockIdx.x, gridDim.x) * (kBlock / 64) + (threadIdx.x >> 6);
    if (chunk >= n_chunks) return;
    const int64_t e0 = chunk * kWaveElems + lane * 16;
    const bool act = e0 < n;  // n % G == 0, G >= 32: a lane is all in or all out
    uint32_t gw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u}, uw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (act) {
        load16(gate + e0, gw);
        load16(up + e0, uw);
    }
    uint32_t hw[8];
    bool far = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float g0 = bf16_lo(gw[i]), g1 = bf16_hi(gw[i]);
        far |= (g0 < kFarGate) | (g1 < kFarGate);
        hw[i] = bf16x2(swiglu_near(g0, bf16_lo(uw[i])), swiglu_near(g1, bf16_hi(uw[i])));
    }
    if (far) {  // a gate below kFarGate in this lane's 16 elements
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float g0 = bf16_lo(gw[i]), g1 = bf16_hi(gw[i]);
            const float u0 = bf16_lo(uw[i]), u1 = bf16_hi(uw[i]);
            hw[i] = bf16x2(g0 < kFarGate ? swiglu_far(g0, u0) : swiglu_near(g0, u0),
                           g1 < kFarGate ? swiglu_far(g1, u1) : swiglu_near(g1, u1));
        }
    }
    const uint32_t hm = run_max<LPG>(absmax16(hw));
    const int64_t grp = e0 / G;
    const bool leader = (lane % LPG) == 0;
    if (act) {
        uint4 *hp = reinterpret_cast<uint4 *>(h_out + e0);
        hp[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        hp[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        if (leader) h_partial[grp] = __uint_as_float(hm << 16);
    }
    if constexpr (kSaveInputs) {
        const float ga = __uint_as_float(run_max<LPG>(absmax16(gw)) << 16);
        const float ua = __uint_as_float(run_max<LPG>(absmax16(uw)) << 16);
        const uint4 gc = cast16(gw, cast_q(ga));
        const uint4 uc = cast16(uw, cast_q(ua));
        if (act) {
            *reinterpret_cast<uint4 *>(gate_codes + e0) = gc;
            *reinterpret_cast<uint4 *>(up_codes + e0) = uc;
            if (leader) {
                gate_scales[grp] = ga > 0.0f ? ga / 448.0f : 1.0f;
                up_scales[grp] = ua > 0.0f ? ua / 448.0f : 1.0f;
            }
        }
    }
}

template <int G, bool kSave>
hipError_t launch_g(const uint16_t *gate, const uint16_t *up, int64_t n, uint16_t *h, float *hp, uint8_t *gc,
                    float *gs, uint8_t *uc, float *us, hipStream_t s) {
    const int64_t nc = ceil_div(n, kWaveElems);
    void *args[] = {&gate, &up, &n, const_cast<int64_t *>(&nc), &h, &hp, &gc, &gs, &uc, &us};
    return hipLaunchKernel(reinterpret_cast<const void *>(&swiglu_fused_kernel<G, kSave>),
                           dim3((unsigned)ceil_div(nc, kBlock / 64)), dim3(kBlock), args, stream_lds_bytes(0), s);
}

template <bool kSave>
hipError_t launch_s(const uint16_t *gate, const uint16_t *up, int64_t n, int G, uint16_t *h, float *hp,
                    uint8_t *gc, float *gs, uint8_t *uc, float *us, hipStream_t s) {
    switch (G) {
    case 32: return launch_g<32, kSave>(gate, up, n, h, hp, gc, gs, uc, us, s);
    case 64: return launch_g<64, kSave>(gate, up, n, h, hp, gc, gs, uc, us, s);
    case 128: return launch_g<128, kSave>(gate, up, n, h, hp, gc, gs, uc, us, s);
    case 256: return launch_g<256, kSave>(gate, up, n, h, hp, gc, gs, uc, us, s);
    case 512: return launch_g<512, kSave>(gate, up, n, h, hp, gc, gs, uc, us, s);
    case 1024: return launch_g<1024, kSave>(gate, up, n, h, hp, gc, gs, uc, us, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_swiglu_fused(const uint16_t *gate, const uint16_t *up, int64_t n, int G, uint16_t *h,
                               float *h_partial, uint8_t *gate_codes, float *gate_scales, uint8_t *up_codes,
                               float *up_scales, hipStream_t s) {
    if (gate_codes)
        return launch_s<true>(gate, up, n, G, h, h_partial, gate_codes, gate_scales, up_codes, up_scales, s);
    return launch_s<false>(gate, up, n, G, h, h_partial, nullptr, nullptr, nullptr, nullptr, s);
}

}  // namespace coat
