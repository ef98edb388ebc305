// rmsnorm.hip -- RMSNorm with Group Scaling stage 1 fused into its epilogue,
// for gfx950.
//
// "COAT: compressing optimizer states and activations for memory-efficient
// FP8 training" explainer (blog.daoxuan.cc/posts/57954): the normalization
// layers are among the nonlinear layers that hold most of the activation
// memory (section "why activations are hard"), and their inputs are the
// example the section "mixed granularity" gives for 1xG groups along the
// channel axis.  Their output feeds a linear layer whose per-tensor E4M3 scale
// needs the tensor absmax; its stage 1 is taken here, where the tensor is
// produced.
//
// One wave per row: the row (cols <= 8192) stays in registers between the
// sum of squares and the normalization, so x is read from HBM once.  The sum
// of squares is taken in FP32 on the row scaled by a power of two (its max
// |x| in [0.5, 1)), and mean + eps and its inverse square root in binary64,
// so every finite BF16 row is in range.  Lane l
// owns the 16-element pieces l, l + 64, l + 128, ... of its row; a 1xG slice
// is G/16 adjacent lanes of one of those 64-piece sweeps.
#include "cast.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace coat {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

template <int PPL, int G, bool kSave>
__global__ __launch_bounds__(kBlock) void rmsnorm_fused_kernel(const uint16_t *__restrict__ x,
                                                               const uint16_t *__restrict__ weight, int64_t rows,
                                                               int cols, float eps, uint16_t *__restrict__ y,
                                                               float *__restrict__ y_partial,
                                                               float *__restrict__ rstd,
                                                               uint8_t *__restrict__ x_codes,
                                                               float *__restrict__ x_scales) {
    constexpr int LPG = G / 16;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int pieces = cols >> 4;
    const int64_t base = row * (int64_t)cols;
    uint32_t xw[PPL][8];
    uint32_t am = 0u;
#pragma unroll
    for (int c = 0; c < PPL; ++c) {
        const int p = c * 64 + lane;
        if (p < pieces) {
            load16(x + base + p * 16, xw[c]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xw[c][i] = 0u;
        }
        am = max(am, absmax16(xw[c]));
    }
    // The squares are summed after an exact power-of-two scale that brings the
    // row's max |x| into [0.5, 1), so no finite BF16 row over- or underflows
    // FP32; the per-row remainder runs in binary64.
    const float amf = __uint_as_float(run_max<64>(am) << 16);
    const int e = amf > 0.0f ? __builtin_amdgcn_frexp_expf(amf) : 0;
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < PPL; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float a = __builtin_amdgcn_ldexpf(bf16_lo(xw[c][i]), -e);
            const float b = __builtin_amdgcn_ldexpf(bf16_hi(xw[c][i]), -e);
            ss = __builtin_fmaf(a, a, ss);
            ss = __builtin_fmaf(b, b, ss);
        }
    }
    ss = wave_sum(ss);
    const double mean = ldexp((double)ss / (double)cols, 2 * e);
    const float r = (float)(1.0 / sqrt(mean + (double)eps));
    if (rstd && lane == 0) rstd[row] = r;
    const int64_t gbase = row * (int64_t)(cols / G);
#pragma unroll
    for (int c = 0; c < PPL; ++c) {
        if (c * 64 >= pieces) break;  // uniform over the wave
        const int p = c * 64 + lane;
        const bool act = p < pieces;  // pieces % (G/16) == 0: a slice is all in or all out
        uint32_t ww[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        if (weight && act) load16(weight + p * 16, ww);
        uint32_t yw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float y0 = bf16_lo(xw[c][i]) * r, y1 = bf16_hi(xw[c][i]) * r;
            if (weight) {
                y0 *= bf16_lo(ww[i]);
                y1 *= bf16_hi(ww[i]);
            }
            yw[i] = bf16x2(y0, y1);
        }
        const uint32_t ym = run_max<LPG>(absmax16(yw));
        const bool leader = (lane % LPG) == 0;
        const int64_t grp = gbase + p / LPG;
        if (act) {
            uint4 *yp = reinterpret_cast<uint4 *>(y + base + p * 16);
            yp[0] = make_uint4(yw[0], yw[1], yw[2], yw[3]);
            yp[1] = make_uint4(yw[4], yw[5], yw[6], yw[7]);
            if (leader) y_partial[grp] = __uint_as_float(ym << 16);
        }
        if constexpr (kSave) {
            const float xa = __uint_as_float(run_max<LPG>(absmax16(xw[c])) << 16);
            const uint4 xc = cast16(xw[c], cast_q(xa));
            if (act) {
                *reinterpret_cast<uint4 *>(x_codes + base + p * 16) = xc;
                if (leader) x_scales[grp] = xa > 0.0f ? xa / 448.0f : 1.0f;
            }
        }
    }
}

template <int PPL, int G, bool kSave>
hipError_t launch_p(const uint16_t *x, const uint16_t *w, int64_t rows, int cols, float eps, uint16_t *y,
                    float *yp, float *rstd, uint8_t *xc, float *xs, hipStream_t s) {
    void *args[] = {&x, &w, &rows, &cols, &eps, &y, &yp, &rstd, &xc, &xs};
    return hipLaunchKernel(reinterpret_cast<const void *>(&rmsnorm_fused_kernel<PPL, G, kSave>),
                           dim3((unsigned)ceil_div(rows, kBlock / 64)), dim3(kBlock), args, 0, s);
}

template <int G, bool kSave>
hipError_t launch_g(const uint16_t *x, const uint16_t *w, int64_t rows, int cols, float eps, uint16_t *y,
                    float *yp, float *rstd, uint8_t *xc, float *xs, hipStream_t s) {
    if (cols <= 1024) return launch_p<1, G, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    if (cols <= 2048) return launch_p<2, G, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    if (cols <= 4096) return launch_p<4, G, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    if (cols <= kRmsNormMaxCols) return launch_p<8, G, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    return hipErrorInvalidValue;
}

template <bool kSave>
hipError_t launch_s(const uint16_t *x, const uint16_t *w, int64_t rows, int cols, int G, float eps, uint16_t *y,
                    float *yp, float *rstd, uint8_t *xc, float *xs, hipStream_t s) {
    switch (G) {
    case 32: return launch_g<32, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    case 64: return launch_g<64, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    case 128: return launch_g<128, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    case 256: return launch_g<256, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    case 512: return launch_g<512, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    case 1024: return launch_g<1024, kSave>(x, w, rows, cols, eps, y, yp, rstd, xc, xs, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_rmsnorm_fused(const uint16_t *x, const uint16_t *weight, int64_t rows, int cols, int G, float eps,
                                uint16_t *y, float *y_partial, float *rstd, uint8_t *x_codes, float *x_scales,
                                hipStream_t s) {
    if (x_codes) return launch_s<true>(x, weight, rows, cols, G, eps, y, y_partial, rstd, x_codes, x_scales, s);
    return launch_s<false>(x, weight, rows, cols, G, eps, y, y_partial, rstd, nullptr, nullptr, s);
}

}  // namespace coat
