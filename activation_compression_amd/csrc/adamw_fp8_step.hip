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
// LDS table (hi + lo FP32 pair per code, computed once on the host in binary64
// from the format's field definitions, passed in the kernel arguments and
// copied into LDS by every workgroup) and the product L(c) / k carried in two
// floats, so the only rounding of consequence is that of the final exp2.  A
// zero code's table entry is Z = -2^40, so zero needs no branch: 2^(Z / k) is
// exactly 0 for every k the step stores (k < 2^29), and the correction term
// Z (1/k)_lo stays below 2^21 in magnitude (|(1/k)_lo| <= 2^-23 / k, k >=
// 0.13 on this form), so the factor amax (1 + ln2 pl) it multiplies is finite
// for amax <= 2^100 and the product is 0, as the expansion maps zero to zero
// (sign(0) = 0).  Groups with a larger amax take the wide form below, whose
// factor has amax's mantissa in place of amax.
//
// Requantization  c = RNE_sat(sign(x) MAX (|x| / amax)^k)  forms the ratio
// |x| / amax correctly rounded (RN reciprocal and one Markstein correction),
// then exp2(k log2 r) with the native transcendental instructions, and
// converts with v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32.  The group maximum gives
// r = 1 exactly and lands on MAX; r <= 1 keeps every value within a few ulps
// of MAX or below, so the conversion itself saturates.
//
// Wide groups.  FP32 spans 2^277 from the smallest denormal to the largest
// value, so a group's max / min can exceed what the ratio |x| / amax (and the
// factor 2^(L/k) of dequantization) can hold: |x| / amax below 2^-126 loses
// bits or flushes to zero, and the native log2 flushes denormal inputs.  A
// group whose range passes 2^120 (k < log2 R_fmt / 120), or whose amax lies
// outside [2^-120, 2^120], takes the log domain instead: |x| = mx 2^ex and
// amax = ma 2^ea split exactly (frexp), log2(|x| / amax) = (ex - ea) +
// log2(mx / ma) with the mantissa quotient correctly rounded in (1/2, 2); and
// dequantization splits 2^(L/k) = 2^f 2^n (n = rint(L/k), exact) and applies
// 2^(n + ea) last with ldexp; dequantization also takes this form for a
// group stored with amax above 2^100.  Such groups are rare (gradients
// spanning dozens of decades within G values, or moments beyond 1e30), so the
// branch is taken by whole lanes and costs the common path a compare.
#include "device.hpp"
#include "kernels.hpp"

namespace coat {
namespace {

constexpr float kLn2 = 0.693147180559945309417f;

// log2(MAX) rounded to FP32 (folded into the exp2 argument of requantization).
template <int F> struct Log2Max;
template <> struct Log2Max<kE4M3> { static constexpr float v = 8.80735492205760410744f; };
template <> struct Log2Max<kE5M2> { static constexpr float v = 15.80735492205760410744f; };

// 1/k as hi + lo: hi ~ 1/k (native reciprocal), lo = hi (1 - k hi) (the FMA
// residual is exact), so hi + lo = 1/k to second order in the residual.
__device__ __forceinline__ void recip2(float k, float &hi, float &lo) {
    hi = __builtin_amdgcn_rcpf(k);
    lo = __builtin_fmaf(-k, hi, 1.0f) * hi;
}

// RN(1/b) for a normal b with a normal reciprocal: native reciprocal plus one
// Newton step.
__device__ __forceinline__ float rcp_rn(float b) {
    const float y = __builtin_amdgcn_rcpf(b);
    return __builtin_fmaf(__builtin_fmaf(-b, y, 1.0f), y, y);
}

// Inverse expansion of one code with its group's amax and 1/k = ih + il:
// amax 2^(L/k) = amax 2^ph 2^pl ~ 2^ph (amax + amax ln2 pl).
template <bool kSigned>
__device__ __forceinline__ float dequant(uint32_t byte, const float2 *tab, float amax, float amax_ln2,
                                         float ih, float il) {
    const float2 L = tab[byte];
    const float ph = L.x * ih;
    float pl = __builtin_fmaf(L.x, ih, -ph);  // exact rounding error of ph
    pl = __builtin_fmaf(L.x, il, pl);
    pl = __builtin_fmaf(L.y, ih, pl);
    const float mag = __builtin_amdgcn_exp2f(ph) * __builtin_fmaf(amax_ln2, pl, amax);
    if constexpr (kSigned)
        return __uint_as_float(__float_as_uint(mag) | ((byte & 0x80u) << 24));
    return mag;
}

// The same inverse expansion for a wide group (amax = ma 2^ea, ma_ln2 = ma
// ln2): 2^(L/k) = 2^f 2^n with n = rint(ph) and f = ph - n exact, the power
// 2^(n + ea) applied last.  A zero code's ph is -2^40 / k, below -2^11 for
// every k a group can store (k < 2^29); n is clamped at -1024 so the exponent
// stays an int, and 2^f with f = ph + 1024 is then 0.  The factor beside it
// stays finite: ma < 1 and |pl| < 2^22 (1/k <= 16 here).
template <bool kSigned>
__device__ __forceinline__ float dequant_wide(uint32_t byte, const float2 *tab, float ma, float ma_ln2, int ea,
                                              float ih, float il) {
    const float2 L = tab[byte];
    const float ph = L.x * ih;
    float pl = __builtin_fmaf(L.x, ih, -ph);
    pl = __builtin_fmaf(L.x, il, pl);
    pl = __builtin_fmaf(L.y, ih, pl);
    const float n = __builtin_fmaxf(__builtin_rintf(ph), -1024.0f);
    const float mag = __builtin_amdgcn_ldexpf(
        __builtin_amdgcn_exp2f(ph - n) * __builtin_fmaf(ma_ln2, pl, ma), ea + (int)n);
    if constexpr (kSigned)
        return __uint_as_float(__float_as_uint(mag) | ((byte & 0x80u) << 24));
    return mag;
}

// A stored group the fast dequantization cannot take: 2^(L/k) for the
// smallest nonzero code, 2^(-log2 R_fmt / k), would pass 2^-120, or amax is
// above 2^100 (a zero code's correction term could then overflow the factor
// amax (1 + ln2 pl)).
__device__ __forceinline__ bool wide_group(float k, float amax, float log2_range) {
    return k * 120.0f < log2_range || amax > 0x1p100f;
}

// Per-group quantization parameters of one new moment.
struct GroupQ {
    float amax;   // stored scale: the group's max |x|
    float k;      // stored expansion exponent
    float amq;    // amax; for a wide group its mantissa ma in [1/2, 1)
    float invq;   // RN(1 / amq)
    int ea;       // wide group: amax = ma 2^ea
    int wide;     // nonzero: the log-domain requantization
};

// mx: bits of max |x|; mn: bits of min nonzero |x| (0 when none).
//
// k = log2(R_fmt) / log2(amax / amin) takes its denominator from the very
// expression requantization evaluates for amin (-log2 of RN(amin / amax), or
// its exponent-split form in a wide group), so that amin lands on the
// smallest subnormal whatever the ratio's rounding.  A group only a few ulps
// wide would otherwise meet two roundings of one ratio that differ by tens of
// percent -- enough to push its smallest element below half the smallest
// subnormal, to code 0.
__device__ __forceinline__ GroupQ group_q(uint32_t mx, uint32_t mn, float log2_range) {
    GroupQ q;
    q.amax = __uint_as_float(mx);
    q.k = 1.0f; q.amq = 1.0f; q.invq = 1.0f; q.ea = 0; q.wide = 0;
    if (mx == 0u) return q;  // all-zero group: every code is 0
    const float amin = __uint_as_float(mn);
    const float ma = __builtin_amdgcn_frexp_mantf(q.amax);  // [0.5, 1)
    const int ea = __builtin_amdgcn_frexp_expf(q.amax);
    const float mb = __builtin_amdgcn_frexp_mantf(amin);
    const int eb = __builtin_amdgcn_frexp_expf(amin);
    const float inv_ma = rcp_rn(ma);
    // log2(amin / amax) as expand_wide evaluates it for amin
    const float lw = (float)(eb - ea) + __builtin_amdgcn_logf(div_rn_from_rcp(mb, ma, inv_ma));
    const bool wide = mx < 0x03800000u || mx > 0x7B800000u || lw < -120.0f;  // amax outside [2^-120, 2^120]
    q.amq = wide ? ma : q.amax;
    q.invq = wide ? inv_ma : rcp_rn(q.amax);
    if (mn != mx) {
        // log2(amax / amin) as expand evaluates -log2(amin / amax)
        float lg = -(wide ? lw : __builtin_amdgcn_logf(div_rn_from_rcp(amin, q.amq, q.invq)));
        // Two distinct floats differ by at least 2^-24 relative: the true value is at least
        // log2(1 + 2^-24) ~ 8.6e-8, and the clamp keeps k finite and positive whatever the log returns.
        lg = __builtin_fmaxf(lg, 8.5e-8f);
        // k = log2(R_fmt) / log2(amax / amin): (amax/amin)^k spans MAX / min_subnormal
        q.k = div_rn_from_rcp(log2_range, lg, rcp_rn(lg));
    }
    q.ea = ea;
    q.wide = wide;
    return q;
}

// Broadcast lane J of every aligned run of W lanes to the whole run.
template <int W, int J>
__device__ __forceinline__ float run_bcast(float v) {
    const int x = __float_as_int(v);
    int r;
    if constexpr (W == 2)
        r = __builtin_amdgcn_mov_dpp(x, J == 0 ? 0xA0 : 0xF5, 0xF, 0xF, true);  // quad_perm [J,J,J+2,J+2]
    else if constexpr (W == 4)
        r = __builtin_amdgcn_mov_dpp(x, J == 0 ? 0x00 : 0x55, 0xF, 0xF, true);  // quad_perm [J,J,J,J]
    else if constexpr (W <= 32)
        r = __builtin_amdgcn_ds_swizzle(x, ((J & 0x1F) << 5) | (0x1F & ~(W - 1)));  // (lane & ~(W-1)) | J
    else
        r = __shfl(x, J);
    return __int_as_float(r);
}

// MAX (|x| / amax)^k for xs = |x| with the group's (amq = amax, invq, k); the
// caller restores the sign.  The correctly rounded ratio is at most 1, so the
// exponent is at most log2(MAX) rounded to FP32 (within 2^-21 of it) and the
// result exceeds MAX by a relative 2^-20 at most: the round-to-nearest-even
// conversion takes such a value to MAX (the midpoint to the next magnitude
// lies 1/28 above it in E4M3, 1/14 in E5M2), so no clamp is needed.
template <int F>
__device__ __forceinline__ float expand(float xs, float amq, float invq, float k) {
    const float r = div_rn_from_rcp(xs, amq, invq);  // RN(|x| / amax) <= 1
    return __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_amdgcn_logf(r), k, Log2Max<F>::v));
}

// The same for a wide group (amax = ma 2^ea, inv_ma = RN(1 / ma)): the
// exponent difference enters through the FMA exactly, the mantissa quotient
// lies in (1/2, 2), and no intermediate leaves the normal range.  |x| = 0
// gives log2(0) = -inf and code 0.
template <int F>
__device__ __forceinline__ float expand_wide(float ax, float ma, float inv_ma, int ea, float k) {
    const float mx = __builtin_amdgcn_frexp_mantf(ax);
    const int ex = __builtin_amdgcn_frexp_expf(ax);
    const float q = div_rn_from_rcp(mx, ma, inv_ma);
    const float t = __builtin_fmaf(__builtin_amdgcn_logf(q), k, Log2Max<F>::v);
    const float y = __builtin_amdgcn_exp2f(__builtin_fmaf((float)(ex - ea), k, t));
    return __builtin_fminf(y, Fp8<F>::kMax);
}

// What one lane reads for its 16 parameters: master weights, gradient, both
// moments' codes and its group's (amax, k) of each moment.
struct ChunkIn {
    float th[16];
    uint32_t gw[8], mw[4], vw[4];
    float am_m, k_m, am_v, k_v;
};

// The loads of one wave's chunk (base wave-uniform), issued without a branch
// so that the table fill behind them waits for its own loads only.  A lane
// with act false (past n, or in a wave with no chunk: base is then 0) reads
// the chunk's first 16 parameters and group instead; whole groups of such
// lanes are past n, so what they compute from it is never stored.  base + 16
// <= n holds for every live chunk (base < n, n a multiple of 16).
template <int G>
__device__ __forceinline__ void load_chunk(const StepBufs &b, int64_t base, int lane, bool act, ChunkIn &in) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int LPG = G / 16;
    const int l = act ? lane : 0;
    const int64_t grp = base / G + l / LPG;
    const gmem<const f32x4> *pp = reinterpret_cast<const gmem<const f32x4> *>(as_global(b.param + base)) + l * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 t = pp[i];
        in.th[4 * i] = t.x; in.th[4 * i + 1] = t.y; in.th[4 * i + 2] = t.z; in.th[4 * i + 3] = t.w;
    }
    const gmem<const u32x4> *gp = reinterpret_cast<const gmem<const u32x4> *>(as_global(b.grad + base)) + l * 2;
    const u32x4 g0 = gp[0], g1 = gp[1];
    in.gw[0] = g0.x; in.gw[1] = g0.y; in.gw[2] = g0.z; in.gw[3] = g0.w;
    in.gw[4] = g1.x; in.gw[5] = g1.y; in.gw[6] = g1.z; in.gw[7] = g1.w;
    const u32x4 mc = reinterpret_cast<const gmem<const u32x4> *>(as_global(b.m_codes + base))[l];
    const u32x4 vc = reinterpret_cast<const gmem<const u32x4> *>(as_global(b.v_codes + base))[l];
    in.mw[0] = mc.x; in.mw[1] = mc.y; in.mw[2] = mc.z; in.mw[3] = mc.w;
    in.vw[0] = vc.x; in.vw[1] = vc.y; in.vw[2] = vc.z; in.vw[3] = vc.w;
    in.am_m = as_global(b.m_amax)[grp]; in.k_m = as_global(b.m_k)[grp];
    in.am_v = as_global(b.v_amax)[grp]; in.k_v = as_global(b.v_k)[grp];
}

// One wave's pass over the 1024 consecutive parameters starting at `base`
// (wave-uniform) whose loads load_chunk issued.  Lanes past n (act false, in
// the last, partial chunk) store nothing; their whole groups are past n as
// well, since n % G == 0.
template <int G, int VF, bool kBf16>
__device__ __forceinline__ void step_chunk(const StepParams &p, const StepBufs &b, const float2 *tab, int64_t base,
                                           int lane, bool act, ChunkIn &in) {
    constexpr int LPG = G / 16;  // lanes per group (2 .. 64)
    const int j = lane & (LPG - 1);
    const bool v_lane = j == 1;  // lane 0 of a group computes m's parameters, lane 1 v's
    const int64_t gbase = base / G;  // first group of the chunk
    const int lgrp = lane / LPG;     // this lane's group within the chunk
    float *th = in.th;
    const uint32_t *gw = in.gw, *mw = in.mw, *vw = in.vw;
    const float am_m = in.am_m, k_m = in.k_m, am_v = in.am_v, k_v = in.k_v;

    float ihm, ilm, ihv, ilv;
    recip2(k_m, ihm, ilm);
    recip2(k_v, ihv, ilv);

    // dequantize the old moments into m1 / v1 (a lane's groups decide its path)
    float m1[16], v1[16];
    if (!(wide_group(k_m, am_m, p.m_log2_range) || wide_group(k_v, am_v, p.v_log2_range))) {
        const float am_m_ln2 = am_m * kLn2, am_v_ln2 = am_v * kLn2;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            m1[i] = dequant<true>((mw[i >> 2] >> (8 * (i & 3))) & 0xFFu, tab, am_m, am_m_ln2, ihm, ilm);
            v1[i] = dequant<false>((vw[i >> 2] >> (8 * (i & 3))) & 0xFFu, tab + 256, am_v, am_v_ln2, ihv, ilv);
        }
    } else {
        const float ma_m = __builtin_amdgcn_frexp_mantf(am_m), ma_v = __builtin_amdgcn_frexp_mantf(am_v);
        const int ea_m = __builtin_amdgcn_frexp_expf(am_m), ea_v = __builtin_amdgcn_frexp_expf(am_v);
        const float ma_m_ln2 = ma_m * kLn2, ma_v_ln2 = ma_v * kLn2;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            m1[i] = dequant_wide<true>((mw[i >> 2] >> (8 * (i & 3))) & 0xFFu, tab, ma_m, ma_m_ln2, ea_m, ihm, ilm);
            v1[i] = dequant_wide<false>((vw[i >> 2] >> (8 * (i & 3))) & 0xFFu, tab + 256, ma_v, ma_v_ln2, ea_v,
                                        ihv, ilv);
        }
    }

    // AdamW in FP32, group statistics of the new moments
    float mx_m = 0.0f, mx_v = 0.0f;
    uint32_t mn_m = ~0u, mn_v = ~0u;  // min over the bits of 2|x| - 2: zero wraps to the top
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float m0 = m1[i], v0 = v1[i];
        const float g = (i & 1) ? bf16_hi(gw[i >> 1]) : bf16_lo(gw[i >> 1]);

        const float m = __builtin_fmaf(p.beta1, m0, p.omb1 * g);
        // (1 - b2) g first: g^2 alone leaves FP32 for |g| > 1.8e19, (1 - b2) g^2 only when v must
        const float v = __builtin_fmaf(p.beta2, v0, (p.omb2 * g) * g);
        const float den = __builtin_fmaf(__builtin_amdgcn_sqrtf(v), p.inv_sqrt_bc2, p.eps);
        const float u = m * __builtin_amdgcn_rcpf(den);
        th[i] = __builtin_fmaf(th[i], p.decay, -p.step_size * u);
        m1[i] = m;
        v1[i] = v;

        mx_m = __builtin_fmaxf(mx_m, __builtin_fabsf(m));
        mx_v = __builtin_fmaxf(mx_v, v);
        mn_m = min(mn_m, (__float_as_uint(m) << 1) - 2u);
        mn_v = min(mn_v, (__float_as_uint(v) << 1) - 2u);
    }
    // Stores go through global-address-space pointers (as the loads do): a flat
    // store counts against the LDS counter too, and the group reductions below
    // would then wait for it.
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    if (act) {
        gmem<f32x4> *pp = reinterpret_cast<gmem<f32x4> *>(as_global(b.param + base)) + lane * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) pp[i] = f32x4{th[4 * i], th[4 * i + 1], th[4 * i + 2], th[4 * i + 3]};
        if constexpr (kBf16) {  // the working copy the next forward pass reads
            gmem<u32x4> *bp = reinterpret_cast<gmem<u32x4> *>(as_global(b.param_bf16 + base)) + lane * 2;
            bp[0] = u32x4{bf16x2(th[0], th[1]), bf16x2(th[2], th[3]), bf16x2(th[4], th[5]), bf16x2(th[6], th[7])};
            bp[1] = u32x4{bf16x2(th[8], th[9]), bf16x2(th[10], th[11]), bf16x2(th[12], th[13]),
                          bf16x2(th[14], th[15])};
        }
    }

    // group statistics (non-negative floats order like their bit patterns)
    const uint32_t gx_m = run_max<LPG>(__float_as_uint(mx_m));
    const uint32_t gx_v = run_max<LPG>(__float_as_uint(mx_v));
    const uint32_t gn_m = (run_min<LPG>(mn_m) + 2u) >> 1;
    const uint32_t gn_v = (run_min<LPG>(mn_v) + 2u) >> 1;

    // one evaluation per lane: lane 0 of a group for m, lane 1 for v, then broadcast
    const GroupQ q = group_q(v_lane ? gx_v : gx_m, v_lane ? gn_v : gn_m,
                             v_lane ? p.v_log2_range : p.m_log2_range);
    if (act && j < 2) {
        as_global(v_lane ? b.v_amax : b.m_amax)[gbase + lgrp] = q.amax;
        as_global(v_lane ? b.v_k : b.m_k)[gbase + lgrp] = q.k;
    }
    const float amq_m = run_bcast<LPG, 0>(q.amq), inv_m = run_bcast<LPG, 0>(q.invq);
    const float kq_m = run_bcast<LPG, 0>(q.k);
    const float amq_v = run_bcast<LPG, 1>(q.amq), inv_v = run_bcast<LPG, 1>(q.invq);
    const float kq_v = run_bcast<LPG, 1>(q.k);
    const int wide_m = __float_as_int(run_bcast<LPG, 0>(__int_as_float(q.wide)));
    const int wide_v = __float_as_int(run_bcast<LPG, 1>(__int_as_float(q.wide)));

    uint32_t om[4], ov[4];
    if ((wide_m | wide_v) == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float ym[4], yv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float xm = m1[4 * t + u];
                ym[u] = with_sign_of(expand<kE4M3>(__builtin_fabsf(xm), amq_m, inv_m, kq_m), xm);
                yv[u] = expand<VF>(v1[4 * t + u], amq_v, inv_v, kq_v);
            }
            om[t] = cvt4<kE4M3>(ym[0], ym[1], ym[2], ym[3]);
            ov[t] = cvt4<VF>(yv[0], yv[1], yv[2], yv[3]);
        }
    } else {  // a wide group in this lane: the log-domain form for both moments
        const int ea_m = __float_as_int(run_bcast<LPG, 0>(__int_as_float(q.ea)));
        const int ea_v = __float_as_int(run_bcast<LPG, 1>(__int_as_float(q.ea)));
        const float ma_m = wide_m ? amq_m : __builtin_amdgcn_frexp_mantf(amq_m);
        const float ma_v = wide_v ? amq_v : __builtin_amdgcn_frexp_mantf(amq_v);
        const float ia_m = wide_m ? inv_m : rcp_rn(ma_m), ia_v = wide_v ? inv_v : rcp_rn(ma_v);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float ym[4], yv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float xm = m1[4 * t + u];
                ym[u] = with_sign_of(expand_wide<kE4M3>(__builtin_fabsf(xm), ma_m, ia_m, ea_m, kq_m), xm);
                yv[u] = expand_wide<VF>(v1[4 * t + u], ma_v, ia_v, ea_v, kq_v);
            }
            om[t] = cvt4<kE4M3>(ym[0], ym[1], ym[2], ym[3]);
            ov[t] = cvt4<VF>(yv[0], yv[1], yv[2], yv[3]);
        }
    }
    if (act) {
        reinterpret_cast<gmem<u32x4> *>(as_global(b.m_codes + base))[lane] = u32x4{om[0], om[1], om[2], om[3]};
        reinterpret_cast<gmem<u32x4> *>(as_global(b.v_codes + base))[lane] = u32x4{ov[0], ov[1], ov[2], ov[3]};
    }
}

// The per-code dequantization table in LDS: [0, 256) m codes (E4M3), [256, 512)
// v codes, both signs of a code byte mapping to its magnitude's entry.
constexpr size_t kTabBytes = 512 * sizeof(float2);  // the kernels' static LDS

// A thread's two table entries, read from the kernel arguments before the
// chunk loads are issued (so waiting for them waits for nothing else) ...
struct TabIn {
    float2 m, v;
};
__device__ __forceinline__ TabIn read_tab(const StepParams &p) {
    const uint32_t t = threadIdx.x & 127u;
    return TabIn{p.log_tab[0][t], p.log_tab[1][t]};
}

// ... and written to LDS after.  Every thread of the workgroup takes part (the
// barrier).  The fences order LDS only, so the chunk loads stay in flight
// across the barrier.
__device__ __forceinline__ void fill_tab(float2 *tab, const TabIn &e) {
    tab[threadIdx.x] = e.m;
    tab[256 + threadIdx.x] = e.v;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A wave's chunk loads are issued first and the LDS table is filled while
// they are in flight (measured on the 7B-shaped arena: 19.6 -> 18.6 ms, and
// 18.4 ms with the raised issue priority).
template <int G, int VF, bool kBf16>
__global__ __launch_bounds__(kBlock) void adamw_fp8_step_kernel(const StepArgs a) {
    __shared__ float2 tab[512];
    const int lane = threadIdx.x & 63;
    const int64_t chunk = xcd_eighth(blockIdx.x, gridDim.x) * (kBlock / 64) +
                          __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const bool live = chunk < a.n_chunks;
    const int64_t base = live ? chunk * kWaveElems : 0;
    const bool act = live && base + lane * 16 < a.buf.n;
    const TabIn te = read_tab(a.p);
    ChunkIn in;
    // The wave issues its loads at raised priority, ahead of older waves'
    // arithmetic on the same SIMD, then drops back for its own.
    __builtin_amdgcn_s_setprio(3);
    load_chunk<G>(a.buf, base, lane, act, in);
    __builtin_amdgcn_s_setprio(0);
    fill_tab(tab, te);
    if (live) step_chunk<G, VF, kBf16>(a.p, a.buf, tab, base, lane, act, in);
}

// Tensor-list form: the launch numbers the chunks of all tensors in order; a
// wave finds its tensor by binary search over chunk_start (wave-uniform, so
// the loads are scalar and hit the scalar cache after the first waves), then
// runs the same per-chunk step on that tensor's buffers.  A tensor's last
// chunk is partial unless its size is a multiple of 1024.
template <int G, int VF, bool kBf16>
__global__ __launch_bounds__(kBlock) void adamw_fp8_step_list_kernel(const StepListArgs a) {
    __shared__ float2 tab[512];
    const int lane = threadIdx.x & 63;
    const int64_t chunk = xcd_eighth(blockIdx.x, gridDim.x) * (kBlock / 64) +
                          __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const bool live = chunk < a.total_chunks;
    int lo = 0;
    if (live) {
        int hi = a.n_tensors;  // chunk_start[lo] <= chunk < chunk_start[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.chunk_start[mid] <= chunk)
                lo = mid;
            else
                hi = mid;
        }
    }
    const StepBufs b = a.entries[lo];
    const int64_t base = live ? (chunk - a.chunk_start[lo]) * kWaveElems : 0;
    const bool act = live && base + lane * 16 < b.n;
    const TabIn te = read_tab(a.p);
    ChunkIn in;
    __builtin_amdgcn_s_setprio(3);
    load_chunk<G>(b, base, lane, act, in);
    __builtin_amdgcn_s_setprio(0);
    fill_tab(tab, te);
    if (live) step_chunk<G, VF, kBf16>(a.p, b, tab, base, lane, act, in);
}

template <int G, int VF, bool kBf16>
hipError_t launch(const StepArgs &a, hipStream_t stream, int /*num_cus*/) {
    constexpr auto kernel = &adamw_fp8_step_kernel<G, VF, kBf16>;
    const dim3 grid((unsigned)ceil_div(a.n_chunks, kBlock / 64));
    void *args[] = {const_cast<StepArgs *>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, dim3(kBlock), args,
                           stream_lds_bytes(kTabBytes), stream);
}

template <int G, int VF, bool kBf16>
hipError_t launch(const StepListArgs &a, hipStream_t stream, int) {
    constexpr auto kernel = &adamw_fp8_step_list_kernel<G, VF, kBf16>;
    const dim3 grid((unsigned)ceil_div(a.total_chunks, kBlock / 64));
    void *args[] = {const_cast<StepListArgs *>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, dim3(kBlock), args,
                           stream_lds_bytes(kTabBytes), stream);
}

template <int VF, bool kBf16, class Args>
hipError_t launch_g(const Args &a, int G, hipStream_t s, int cap) {
    switch (G) {
    case 32: return launch<32, VF, kBf16>(a, s, cap);
    case 64: return launch<64, VF, kBf16>(a, s, cap);
    case 128: return launch<128, VF, kBf16>(a, s, cap);
    case 256: return launch<256, VF, kBf16>(a, s, cap);
    case 512: return launch<512, VF, kBf16>(a, s, cap);
    case 1024: return launch<1024, VF, kBf16>(a, s, cap);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Host side: the dequantization table of each format, built once.
static void build_log_table(int fmt, float2 *tab) {
    const int mbits = fmt == kE5M2 ? 2 : 3;
    const int bias = fmt == kE5M2 ? 15 : 7;
    const double vmax = fmt == kE5M2 ? 57344.0 : 448.0;
    for (int c = 0; c < 128; ++c) {
        const int e = c >> mbits, m = c & ((1 << mbits) - 1);
        const bool special = fmt == kE5M2 ? e == 31 : (e == 15 && m == 7);
        if (c == 0 || special) {
            tab[c] = make_float2(-0x1p40f, 0.0f);  // 2^(-2^40 / k) is exactly 0 for every stored k
            continue;
        }
        const double d = e == 0 ? ldexp((double)m, 1 - bias - mbits)
                                : ldexp((double)((1 << mbits) | m), e - bias - mbits);
        const double L = log2(d) - log2(vmax);
        const float hi = (float)L;
        tab[c] = make_float2(hi, (float)(L - (double)hi));
    }
}

const float2 *fp8_log_table(int fmt) {
    static const struct Tables {
        float2 t[2][128];
        Tables() { build_log_table(kE4M3, t[0]); build_log_table(kE5M2, t[1]); }
    } tables;
    return tables.t[fmt == kE5M2 ? 1 : 0];
}

hipError_t launch_adamw_fp8_step(const StepArgs &a, int group_size, int v_format,
                                 hipStream_t stream, int num_cus) {
    if (a.buf.param_bf16)
        return v_format == kE5M2 ? launch_g<kE5M2, true>(a, group_size, stream, num_cus)
                                 : launch_g<kE4M3, true>(a, group_size, stream, num_cus);
    return v_format == kE5M2 ? launch_g<kE5M2, false>(a, group_size, stream, num_cus)
                             : launch_g<kE4M3, false>(a, group_size, stream, num_cus);
}

hipError_t launch_adamw_fp8_step_list(const StepListArgs &a, int group_size, int v_format, hipStream_t stream) {
    if (a.has_bf16)
        return v_format == kE5M2 ? launch_g<kE5M2, true>(a, group_size, stream, 0)
                                 : launch_g<kE4M3, true>(a, group_size, stream, 0);
    return v_format == kE5M2 ? launch_g<kE5M2, false>(a, group_size, stream, 0)
                             : launch_g<kE4M3, false>(a, group_size, stream, 0);
}

}  // namespace coat
