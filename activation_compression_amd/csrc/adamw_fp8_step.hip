// adamw_fp8_step.hip -- fused AdamW update with FP8 moments and per-group
// dynamic-range expansion, for gfx950.
//
// Method: "COAT: compressing optimizer states and activations for
// memory-efficient FP8 training" explainer (blog.daoxuan.cc/posts/57954),
// sections on why the second moment is the sensitive one, on its smaller
// dynamic range, and "expansion function"; the update rule of "LLM atlas --
// systems / numerics", section "08 Adam -> AdamW".
//
// One pass over HBM per step.  Every lane owns 16 consecutive parameters, so
// a 1xG group is G/16 adjacent lanes of one wave (2 .. 64 lanes) and its
// statistics are a DPP reduction -- no LDS round trip, no second kernel.  The
// per-lane stream is 64 B of FP32 master weights, 32 B of BF16 gradient and
// 16 B of each FP8 moment in, the same minus the gradient out.
//
// Dequantization  x = sign(c) amax (|dec c| / MAX)^(1/k)  is evaluated as
// amax * 2^(L(c) / k), with L(c) = log2(|dec c| / MAX) read from a 256-entry
// LDS table (hi + lo FP32 pair per code, built per workgroup in binary64 from
// the hardware FP8 decode) and the product L(c) / k carried in two floats, so
// the only rounding of consequence is that of the final exp2.  A zero code's
// table entry is -2^100: 2^(-2^100 / k) is exactly 0 for every k the format
// range can produce, so zero needs no branch.
//
// Requantization  c = RNE_sat(sign(x) MAX (|x| / amax)^k)  forms the ratio
// |x| / amax correctly rounded (power-of-two prescale, RN reciprocal and one
// Markstein correction), then exp2(k log2 r) with the native transcendental
// instructions, and converts with v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32.  The
// group maximum gives r = 1 exactly and lands on MAX exactly.
#include "device.hpp"
#include "kernels.hpp"

namespace coat {
namespace {

constexpr float kLn2 = 0.693147180559945309417f;

// log2(|decode(c)| / MAX) for code magnitude c, split into hi + lo FP32.
template <int F>
__device__ float2 log_table_entry(uint32_t c) {
    const float d = decode1<F>(c);
    if (c == 0 || !(d > 0.0f) || !__builtin_isfinite(d))
        return make_float2(-0x1p100f, 0.0f);
    const double L = log2((double)d) - log2((double)Fp8<F>::kMax);
    const float hi = (float)L;
    return make_float2(hi, (float)(L - (double)hi));
}

// 1/k as hi + lo: hi = RN(1/k), lo = hi * (1 - k hi) (the FMA residual is exact).
__device__ __forceinline__ void recip2(float k, float &hi, float &lo) {
    hi = 1.0f / k;
    lo = __builtin_fmaf(-k, hi, 1.0f) * hi;
}

// Inverse expansion of one code with its group's (amax, 1/k = ih + il).
__device__ __forceinline__ float dequant(uint32_t code, const float2 *tab, float amax,
                                         float ih, float il) {
    const float2 L = tab[code & 0x7Fu];
    const float ph = L.x * ih;
    float pl = __builtin_fmaf(L.x, ih, -ph);  // exact rounding error of ph
    pl = __builtin_fmaf(L.x, il, pl);
    pl = __builtin_fmaf(L.y, ih, pl);
    const float ea = __builtin_amdgcn_exp2f(ph) * amax;
    const float mag = __builtin_fmaf(ea, pl * kLn2, ea);  // 2^pl ~ 1 + pl ln 2
    return __uint_as_float(__float_as_uint(mag) | ((code & 0x80u) << 24));
}

// Per-group quantization parameters of a new moment.
struct GroupQ {
    float amax;    // stored scale: the group's max |x|
    float k;       // stored expansion exponent
    float amax_s;  // amax * 2^sh, in [1, 2)
    float inv_s;   // RN(1 / amax_s)
    int sh;
};

// mx: bits of max |x|; mn: bits of min nonzero |x| (0 when none).
__device__ __forceinline__ GroupQ group_q(uint32_t mx, uint32_t mn, float log2_range) {
    GroupQ q;
    q.amax = __uint_as_float(mx);
    if (mx == 0u) {
        q.k = 1.0f; q.amax_s = 1.0f; q.inv_s = 1.0f; q.sh = 0;
        return q;
    }
    int ea;
    const float ma = frexpf(q.amax, &ea);  // amax = ma 2^ea, ma in [0.5, 1)
    q.sh = 1 - ea;
    q.amax_s = 2.0f * ma;
    q.inv_s = 1.0f / q.amax_s;
    if (mn == mx) {
        q.k = 1.0f;  // all nonzero magnitudes equal: ln R = 0
    } else {
        int eb;
        const float mb = frexpf(__uint_as_float(mn), &eb);
        // log2(amax / amin) without overflow for any FP32 pair
        const float lg = (float)(ea - eb) + log2f(ma / mb);
        q.k = log2_range / lg;  // (amax/amin)^k spans MAX / min_subnormal
    }
    return q;
}

// sign(x) * min(MAX (|x| / amax)^k, MAX), ready for the FP8 convert.
template <int F>
__device__ __forceinline__ float expand(float x, const GroupQ &q) {
    const float xs = __builtin_amdgcn_ldexpf(__builtin_fabsf(x), q.sh);
    const float r = div_rn_from_rcp(xs, q.amax_s, q.inv_s);
    float y = __builtin_amdgcn_exp2f(__builtin_amdgcn_logf(r) * q.k) * Fp8<F>::kMax;
    y = __builtin_fminf(y, Fp8<F>::kMax);
    return with_sign_of(y, x);
}

template <int G, int VF>
__global__ __launch_bounds__(kBlock) void adamw_fp8_step_kernel(const StepArgs a) {
    __shared__ float2 tab[256];  // [0, 128): m codes (E4M3); [128, 256): v codes
    {
        const uint32_t t = threadIdx.x;
        tab[t] = t < 128 ? log_table_entry<kE4M3>(t) : log_table_entry<VF>(t - 128);
    }
    __syncthreads();

    constexpr int LPG = G / 16;  // lanes per group
    const int lane = threadIdx.x & 63;
    const bool leader = (lane % LPG) == 0;
    const int64_t wave0 = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    const int64_t wstride = (int64_t)gridDim.x * (kBlock / 64);

    for (int64_t chunk = wave0; chunk < a.n_chunks; chunk += wstride) {
        const int64_t e0 = chunk * kWaveElems + lane * 16;
        const bool act = e0 < a.n;  // n % 32 == 0: a lane is all in or all out
        const int64_t grp = e0 / G;

        float th[16];
        uint32_t gw[8], mw[4], vw[4];
        float am_m = 0.0f, k_m = 1.0f, am_v = 0.0f, k_v = 1.0f;
        if (act) {
            const float4 *pp = reinterpret_cast<const float4 *>(a.param + e0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 t = pp[i];
                th[4 * i] = t.x; th[4 * i + 1] = t.y; th[4 * i + 2] = t.z; th[4 * i + 3] = t.w;
            }
            const uint4 *gp = reinterpret_cast<const uint4 *>(a.grad + e0);
            const uint4 g0 = gp[0], g1 = gp[1];
            gw[0] = g0.x; gw[1] = g0.y; gw[2] = g0.z; gw[3] = g0.w;
            gw[4] = g1.x; gw[5] = g1.y; gw[6] = g1.z; gw[7] = g1.w;
            const uint4 mc = *reinterpret_cast<const uint4 *>(a.m_codes + e0);
            const uint4 vc = *reinterpret_cast<const uint4 *>(a.v_codes + e0);
            mw[0] = mc.x; mw[1] = mc.y; mw[2] = mc.z; mw[3] = mc.w;
            vw[0] = vc.x; vw[1] = vc.y; vw[2] = vc.z; vw[3] = vc.w;
            am_m = a.m_amax[grp]; k_m = a.m_k[grp];
            am_v = a.v_amax[grp]; k_v = a.v_k[grp];
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) th[i] = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) gw[i] = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) { mw[i] = 0u; vw[i] = 0u; }
        }

        float ihm, ilm, ihv, ilv;
        recip2(k_m, ihm, ilm);
        recip2(k_v, ihv, ilv);

        // dequantize, AdamW in FP32, group statistics of the new moments
        float m1[16], v1[16];
        uint32_t mx_m = 0u, mn_m = ~0u, mx_v = 0u, mn_v = ~0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t cm = (mw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
            const uint32_t cv = (vw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
            const float m0 = dequant(cm, tab, am_m, ihm, ilm);
            const float v0 = dequant(cv, tab + 128, am_v, ihv, ilv);
            const float g = (i & 1) ? bf16_hi(gw[i >> 1]) : bf16_lo(gw[i >> 1]);

            const float m = __builtin_fmaf(a.beta1, m0, a.omb1 * g);
            const float v = __builtin_fmaf(a.beta2, v0, a.omb2 * (g * g));
            const float den = __builtin_fmaf(__builtin_amdgcn_sqrtf(v), a.inv_sqrt_bc2, a.eps);
            const float u = m * __builtin_amdgcn_rcpf(den);
            th[i] = __builtin_fmaf(th[i], a.decay, -a.step_size * u);
            m1[i] = m;
            v1[i] = v;

            const uint32_t bm = __float_as_uint(m) & 0x7FFFFFFFu;
            const uint32_t bv = __float_as_uint(v) & 0x7FFFFFFFu;
            mx_m = max(mx_m, bm); mn_m = min(mn_m, bm - 1u);  // zero wraps to ~0
            mx_v = max(mx_v, bv); mn_v = min(mn_v, bv - 1u);
        }
        if (act) {
            float4 *pp = reinterpret_cast<float4 *>(a.param + e0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pp[i] = make_float4(th[4 * i], th[4 * i + 1], th[4 * i + 2], th[4 * i + 3]);
        }

        mx_m = run_max<LPG>(mx_m); mn_m = run_min<LPG>(mn_m);
        mx_v = run_max<LPG>(mx_v); mn_v = run_min<LPG>(mn_v);
        const GroupQ qm = group_q(mx_m, mn_m + 1u, a.m_log2_range);
        const GroupQ qv = group_q(mx_v, mn_v + 1u, a.v_log2_range);

        uint32_t om[4], ov[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            om[j] = cvt4<kE4M3>(expand<kE4M3>(m1[4 * j], qm), expand<kE4M3>(m1[4 * j + 1], qm),
                                expand<kE4M3>(m1[4 * j + 2], qm), expand<kE4M3>(m1[4 * j + 3], qm));
            ov[j] = cvt4<VF>(expand<VF>(v1[4 * j], qv), expand<VF>(v1[4 * j + 1], qv),
                             expand<VF>(v1[4 * j + 2], qv), expand<VF>(v1[4 * j + 3], qv));
        }
        if (act) {
            *reinterpret_cast<uint4 *>(a.m_codes + e0) = make_uint4(om[0], om[1], om[2], om[3]);
            *reinterpret_cast<uint4 *>(a.v_codes + e0) = make_uint4(ov[0], ov[1], ov[2], ov[3]);
            if (leader) {
                a.m_amax[grp] = qm.amax; a.m_k[grp] = qm.k;
                a.v_amax[grp] = qv.amax; a.v_k[grp] = qv.k;
            }
        }
    }
}

template <int G, int VF>
hipError_t launch(const StepArgs &a, hipStream_t stream, int grid_cap) {
    const int64_t blocks = ceil_div(a.n_chunks, kBlock / 64);
    const dim3 grid((unsigned)(blocks < grid_cap ? blocks : grid_cap)), block(kBlock);
    void *args[] = {const_cast<StepArgs *>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&adamw_fp8_step_kernel<G, VF>),
                           grid, block, args, 0, stream);
}

template <int VF>
hipError_t launch_g(const StepArgs &a, int G, hipStream_t s, int cap) {
    switch (G) {
    case 32: return launch<32, VF>(a, s, cap);
    case 64: return launch<64, VF>(a, s, cap);
    case 128: return launch<128, VF>(a, s, cap);
    case 256: return launch<256, VF>(a, s, cap);
    case 512: return launch<512, VF>(a, s, cap);
    case 1024: return launch<1024, VF>(a, s, cap);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_adamw_fp8_step(const StepArgs &a, int group_size, int v_format,
                                 hipStream_t stream, int grid_cap) {
    return v_format == kE5M2 ? launch_g<kE5M2>(a, group_size, stream, grid_cap)
                             : launch_g<kE4M3>(a, group_size, stream, grid_cap);
}

}  // namespace coat
