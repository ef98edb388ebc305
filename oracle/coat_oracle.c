/*
 * coat_oracle.c -- CPU oracle for COAT-style FP8 optimizer-state and
 * activation compression.  TEST INFRASTRUCTURE ONLY (see coat_oracle.h).
 *
 * Plain C, IEEE binary64 throughout, one element at a time.  Sources are cited
 * per function; the page keys [COAT], [ATLAS], [FP4N], [LPF] are defined in
 * coat_oracle.h.
 */
#include "coat_oracle.h"

#include <math.h>
#include <stddef.h>

/* ======================================================================== */
/* C1. Minifloat codec by enumeration                                        */
/* ======================================================================== */

/*
 * Field layout of a sign / exponent / mantissa minifloat ([ATLAS] section
 * "01 Number anatomy"; [FP4N] discussion of subnormals):
 *   exponent field 0        -> subnormal: (m / 2^M) * 2^(1 - bias)
 *   exponent field e > 0    -> normal:    (1 + m / 2^M) * 2^(e - bias)
 * Special codes:
 *   OCP E4M3 ("FN"): only exponent and mantissa all ones is NaN, no infinity;
 *                    so the largest finite value is 1.75 * 2^8 = 448 and the
 *                    smallest subnormal is 2^-9 ([ATLAS] section "03 FP8").
 *   OCP E5M2:        exponent all ones is reserved (inf / NaN), IEEE style;
 *                    largest finite 1.75 * 2^15 = 57344, smallest 2^-16.
 *   E2M2 (bias 2):   no special codes; the 16-value grid worked out in [FP4N].
 */
typedef struct {
    int ebits, mbits, bias;
    int special; /* 0 none, 1 OCP-FN (only all-ones code is NaN), 2 IEEE-style */
} orc_format;

static orc_format fmt_desc(int fmt)
{
    orc_format f;
    switch (fmt) {
    case ORC_E4M3: f.ebits = 4; f.mbits = 3; f.bias = 7;  f.special = 1; break;
    case ORC_E5M2: f.ebits = 5; f.mbits = 2; f.bias = 15; f.special = 2; break;
    default:       f.ebits = 2; f.mbits = 2; f.bias = 2;  f.special = 0; break;
    }
    return f;
}

/* Decode a sign-less code magnitude from the field definitions. */
static double decode_magnitude(const orc_format *f, uint32_t mag)
{
    uint32_t e = mag >> f->mbits;
    uint32_t m = mag & ((1u << f->mbits) - 1u);
    uint32_t emax_field = (1u << f->ebits) - 1u;
    double frac = (double)m / (double)(1u << f->mbits);

    if (f->special == 1 && e == emax_field && m == (1u << f->mbits) - 1u)
        return NAN;
    if (f->special == 2 && e == emax_field)
        return m == 0 ? INFINITY : NAN;
    if (e == 0)
        return ldexp(frac, 1 - f->bias);
    return ldexp(1.0 + frac, (int)e - f->bias);
}

double orc_fp8_decode(int fmt, uint32_t code)
{
    orc_format f = fmt_desc(fmt);
    int nbits = 1 + f.ebits + f.mbits;
    uint32_t sign = (code >> (nbits - 1)) & 1u;
    uint32_t mag = code & ((1u << (nbits - 1)) - 1u);
    double a = decode_magnitude(&f, mag);
    return sign ? -a : a;
}

/* Largest code magnitude whose value is finite.  Finite values grow strictly
 * with the code magnitude, so the grid is {decode(c) : c = 0 .. max_code}. */
uint32_t orc_fp8_max_code(int fmt)
{
    orc_format f = fmt_desc(fmt);
    uint32_t c = (1u << (f.ebits + f.mbits)) - 1u;
    while (!isfinite(decode_magnitude(&f, c)))
        --c;
    return c;
}

double orc_fp8_max(int fmt)
{
    orc_format f = fmt_desc(fmt);
    return decode_magnitude(&f, orc_fp8_max_code(fmt));
}

double orc_fp8_min_subnormal(int fmt)
{
    orc_format f = fmt_desc(fmt);
    return decode_magnitude(&f, 1u);
}

/*
 * The grid of each format, enumerated once from the field definitions:
 * grid[f][c] = decode(c) for c = 0 .. max_code (finite values grow strictly
 * with the code magnitude).
 */
#define ORC_NFMT 3
static double grid[ORC_NFMT][256];
static uint32_t grid_top[ORC_NFMT];

__attribute__((constructor)) static void build_grids(void)
{
    for (int fmt = 0; fmt < ORC_NFMT; ++fmt) {
        orc_format f = fmt_desc(fmt);
        grid_top[fmt] = orc_fp8_max_code(fmt);
        for (uint32_t c = 0; c <= grid_top[fmt]; ++c)
            grid[fmt][c] = decode_magnitude(&f, c);
    }
}

/*
 * Round-to-nearest-even with saturation ([ATLAS] "01 Number anatomy" separates
 * overflow from rounding; the method saturates rather than overflowing).
 * Find the pair of grid neighbours around |x| (bisection over the sorted
 * grid), take the nearer one, and on an exact tie take the code whose
 * mantissa LSB is 0.
 */
uint32_t orc_fp8_encode(int fmt, double x)
{
    orc_format f = fmt_desc(fmt);
    int nbits = 1 + f.ebits + f.mbits;
    const double *v = grid[fmt];
    uint32_t top = grid_top[fmt];
    double a = fabs(x);
    uint32_t c;

    if (a >= v[top]) {
        c = top;
    } else {
        /* largest c with v[c] <= a: invariant v[lo] <= a < v[hi] */
        uint32_t lo = 0, hi = top;
        while (hi - lo > 1) {
            uint32_t mid = (lo + hi) / 2;
            if (v[mid] <= a) lo = mid; else hi = mid;
        }
        c = lo;
        if (v[c] != a) {
            double d_lo = a - v[c], d_hi = v[c + 1] - a;
            if (d_hi < d_lo || (d_hi == d_lo && (c & 1u)))
                c = c + 1;
        }
    }
    if (c == 0)
        return 0u;
    return (x < 0 ? (1u << (nbits - 1)) : 0u) | c;
}

/* ======================================================================== */
/* C2 / C3. Dynamic-range expansion of a 1xG group                           */
/* ======================================================================== */

/*
 * [COAT] section "expansion function": before quantizing, each group is
 * stretched with f(x) = sign(x) |x|^k, which turns a group range R_X into
 * R_X^k.  k is chosen per group and per step so that the stretched group
 * covers the FP8 format's range, which [COAT] section "the second moment's
 * dynamic range is smaller" takes as max / smallest subnormal (448 / 2^-9 for
 * E4M3).  Hence R_X^k = R_fmt, k = ln R_fmt / ln R_X.
 *
 * Readings (where the page's display math was lost):
 *  - R_X is max|x| / min over the nonzero |x| of the group (zeros encode as 0);
 *  - an all-zero group stores amax = 0, k = 1; a group whose nonzero
 *    magnitudes are all equal stores k = 1 (ln 1 = 0);
 *  - the stored scale is the group absmax and the code is
 *    RNE_sat(sign(x) * MAX * (|x| / amax)^k); this is |x|^k / s with
 *    s = amax^k / MAX, written so that it stays inside the FP32 range;
 *  - k is rounded to FP32 (it is stored) before it is used for the codes;
 *  - the code is decided from the FP32 value of that product, the precision
 *    the update itself runs in.
 */
void orc_expand_quantize(int fmt, const float *x, int64_t G, double k_force,
                         uint8_t *codes, float *amax_out, float *k_out)
{
    double vmax = orc_fp8_max(fmt);
    double r_fmt = vmax / orc_fp8_min_subnormal(fmt);
    double amax = 0.0, amin = INFINITY;
    int64_t i;

    for (i = 0; i < G; ++i) {
        double a = fabs((double)x[i]);
        if (a > amax) amax = a;
        if (a != 0.0 && a < amin) amin = a;
    }

    if (amax == 0.0) {
        for (i = 0; i < G; ++i) codes[i] = 0;
        *amax_out = 0.0f;
        *k_out = 1.0f;
        return;
    }

    float k;
    if (k_force > 0.0)
        k = (float)k_force;
    else if (amin == amax)
        k = 1.0f;
    else
        k = (float)(log(r_fmt) / log(amax / amin));

    for (i = 0; i < G; ++i)
        codes[i] = (uint8_t)orc_expand_encode(fmt, (double)x[i], (float)amax, k);
    *amax_out = (float)amax; /* amax is an FP32 value, so this is exact */
    *k_out = k;
}

/* The last step of the group quantization on its own: the code of a value x
 * in a group stored with (amax, k), RNE_sat(sign(x) * MAX * (|x| / amax)^k)
 * with the power's value rounded to FP32 first.  x = 0 (or amax = 0) gives
 * code 0.  x need not be an FP32 value. */
uint32_t orc_expand_encode(int fmt, double x, float amax, float k)
{
    if (x == 0.0 || amax == 0.0f)
        return 0u;
    double y = orc_fp8_max(fmt) * pow(fabs(x) / (double)amax, (double)k);
    float y32 = (float)y;
    return orc_fp8_encode(fmt, x < 0 ? -(double)y32 : (double)y32);
}

void orc_expand_encode_each(int fmt, const double *x, const float *amax, const float *k, int64_t n,
                            uint8_t *codes)
{
    for (int64_t i = 0; i < n; ++i)
        codes[i] = (uint8_t)orc_expand_encode(fmt, x[i], amax[i], k[i]);
}

void orc_expand_encode_groups(int fmt, const double *x, int64_t g0, int64_t g1, int64_t G,
                              const float *amax, const float *k, uint8_t *codes)
{
    for (int64_t g = g0; g < g1; ++g)
        for (int64_t i = 0; i < G; ++i)
            codes[g * G + i] = (uint8_t)orc_expand_encode(fmt, x[g * G + i], amax[g], k[g]);
}

void orc_expand_quantize_groups(int fmt, const float *x, int64_t g0, int64_t g1, int64_t G,
                                const float *k_given, uint8_t *codes, float *amax, float *k)
{
    for (int64_t g = g0; g < g1; ++g)
        orc_expand_quantize(fmt, x + g * G, G, k_given ? (double)k_given[g] : 0.0,
                            codes + g * G, &amax[g], &k[g]);
}

/* [COAT] section "expansion function": dequantization applies the inverse
 * power 1/k to the decoded magnitude; the sign is carried by the code. */
double orc_expand_dequantize(int fmt, uint32_t code, float amax, float k)
{
    double d = orc_fp8_decode(fmt, code);
    if (d == 0.0 || amax == 0.0f)
        return 0.0;
    double mag = (double)amax * pow(fabs(d) / orc_fp8_max(fmt), 1.0 / (double)k);
    return d < 0 ? -mag : mag;
}

void orc_expand_dequantize_groups(int fmt, const uint8_t *codes, int64_t g0, int64_t g1, int64_t G,
                                  const float *amax, const float *k, double *out)
{
    for (int64_t g = g0; g < g1; ++g)
        for (int64_t i = 0; i < G; ++i)
            out[g * G + i] = orc_expand_dequantize(fmt, codes[g * G + i], amax[g], k[g]);
}

/* ======================================================================== */
/* BF16 rounding                                                             */
/* ======================================================================== */

/*
 * BF16 keeps FP32's sign and 8-bit exponent and 7 explicit mantissa bits
 * ([LPF]; [ATLAS] "01 Number anatomy"), i.e. an 8-bit significand.  Round to
 * nearest, ties to even, by scaling the significand to an integer: frexp
 * gives x = f 2^e with 0.5 <= |f| < 1, so f * 2^8 carries the 8 kept bits in
 * its integer part, and rint (round-half-even in the default rounding mode)
 * rounds the rest away.  Values below the smallest normal keep the normal
 * exponent floor (BF16 subnormals have the same spacing as FP32's exponent
 * floor allows: 2^-133).  The result is exact in binary64 and representable
 * in FP32, so its bit pattern's top half is the BF16 code.
 */
uint16_t orc_bf16_rne(float xf)
{
    double x = (double)xf;
    union { float f; uint32_t u; } cv;
    if (x == 0.0 || isnan(x) || isinf(x)) {
        cv.f = xf;
        return (uint16_t)(cv.u >> 16);
    }
    int e;
    double f = frexp(x, &e);               /* x = f * 2^e */
    if (e < -125) {                        /* below the normal range: fixed spacing 2^-133 */
        f = ldexp(x, 133);
        e = 0;
        cv.f = (float)ldexp(rint(f), -133);
        return (uint16_t)(cv.u >> 16);
    }
    double r = ldexp(rint(ldexp(f, 8)), e - 8);
    if (fabs(r) > 3.3895313892515355e38)   /* rounds past the largest BF16 value */
        r = x > 0 ? INFINITY : -INFINITY;
    cv.f = (float)r;
    return (uint16_t)(cv.u >> 16);
}

/* ======================================================================== */
/* C4. AdamW with FP8 moments                                                */
/* ======================================================================== */

static double bf16_to_double(uint16_t bits)
{
    /* BF16 keeps FP32's sign, 8-bit exponent and the top 7 mantissa bits
     * ([LPF]; [ATLAS] "01 Number anatomy"), so widening appends 16 zero bits. */
    union { uint32_t u; float f; } cv;
    cv.u = (uint32_t)bits << 16;
    return (double)cv.f;
}

/*
 * The update rule of [ATLAS] section "08 Adam -> AdamW" (the [COAT] page
 * names the same symbols but its display formula was lost):
 *   m_t = b1 m_{t-1} + (1 - b1) g_t
 *   v_t = b2 v_{t-1} + (1 - b2) g_t^2
 *   dtheta = -lr * mhat / (sqrt(vhat) + eps)
 *   theta <- (1 - lr * wd) theta + dtheta
 * with the standard Adam bias corrections mhat = m_t / (1 - b1^t),
 * vhat = v_t / (1 - b2^t), t the 1-based step.  Weight decay acts on theta
 * directly, never through m or v ([COAT] section on second-moment
 * sensitivity).
 */
typedef struct { double b1, b2, lr, eps, wd, bc1, bc2; } adamw_consts;

static adamw_consts adamw_setup(const orc_hparams *hp)
{
    adamw_consts c;
    c.b1 = (double)hp->beta1;
    c.b2 = (double)hp->beta2;
    c.lr = (double)hp->lr;
    c.eps = (double)hp->eps;
    c.wd = (double)hp->weight_decay;
    c.bc1 = 1.0 - pow(c.b1, (double)hp->step);
    c.bc2 = 1.0 - pow(c.b2, (double)hp->step);
    return c;
}

static double adamw_element(double theta, double g, double m0, double v0,
                            const adamw_consts *c, double *m1, double *v1)
{
    double b1 = c->b1, b2 = c->b2, lr = c->lr, eps = c->eps, wd = c->wd;

    *m1 = b1 * m0 + (1.0 - b1) * g;
    *v1 = b2 * v0 + (1.0 - b2) * g * g;
    double mhat = *m1 / c->bc1;
    double vhat = *v1 / c->bc2;
    double dtheta = -lr * mhat / (sqrt(vhat) + eps);
    return (1.0 - lr * wd) * theta + dtheta;
}

void orc_adamw_step_f64(double *param, const double *grad, double *m, double *v,
                        int64_t n, const orc_hparams *hp)
{
    adamw_consts c = adamw_setup(hp);
    for (int64_t i = 0; i < n; ++i) {
        double m1, v1;
        param[i] = adamw_element(param[i], grad[i], m[i], v[i], &c, &m1, &v1);
        m[i] = m1;
        v[i] = v1;
    }
}

/*
 * The fused step in the order the method takes it: dequantize both moments
 * with the group's stored (amax, k), run the AdamW update with FP32 master
 * weights ([LPF] on FP32 master copies), store theta as FP32, then recompute
 * (amax, k) per group from the new FP32 moments and requantize them.  m is
 * stored as E4M3; v as E4M3 or E5M2 ([COAT] allows both pairings).
 */
void orc_adamw_step(float *param, const uint16_t *grad,
                    uint8_t *m_codes, float *m_amax, float *m_k,
                    uint8_t *v_codes, float *v_amax, float *v_k,
                    int64_t g0, int64_t g1, int64_t G, int v_fmt,
                    const orc_hparams *hp, float *m_new_out, float *v_new_out)
{
    float m_new[1024], v_new[1024];  /* G <= 1024 */
    adamw_consts c = adamw_setup(hp);
    if (G > 1024) return;

    for (int64_t grp = g0; grp < g1; ++grp) {
        int64_t base = grp * G;
        for (int64_t i = 0; i < G; ++i) {
            int64_t e = base + i;
            double m0 = orc_expand_dequantize(ORC_E4M3, m_codes[e], m_amax[grp], m_k[grp]);
            double v0 = orc_expand_dequantize(v_fmt, v_codes[e], v_amax[grp], v_k[grp]);
            double m1, v1;
            double th = adamw_element((double)param[e], bf16_to_double(grad[e]),
                                      m0, v0, &c, &m1, &v1);
            param[e] = (float)th;
            m_new[i] = (float)m1;
            v_new[i] = (float)v1;
            if (m_new_out) m_new_out[e] = m_new[i];
            if (v_new_out) v_new_out[e] = v_new[i];
        }
        orc_expand_quantize(ORC_E4M3, m_new, G, 0.0, m_codes + base, &m_amax[grp], &m_k[grp]);
        orc_expand_quantize(v_fmt, v_new, G, 0.0, v_codes + base, &v_amax[grp], &v_k[grp]);
    }
}

/* The working copy the forward/backward pass computes with ([LPF]: FP32
 * master weights, BF16 for the matrix products) taken right after the update. */
void orc_adamw_step_bf16(float *param, const uint16_t *grad,
                         uint8_t *m_codes, float *m_amax, float *m_k,
                         uint8_t *v_codes, float *v_amax, float *v_k,
                         int64_t g0, int64_t g1, int64_t G, int v_fmt,
                         const orc_hparams *hp, uint16_t *param_bf16)
{
    orc_adamw_step(param, grad, m_codes, m_amax, m_k, v_codes, v_amax, v_k, g0, g1, G, v_fmt, hp,
                   NULL, NULL);
    for (int64_t e = g0 * G; e < g1 * G; ++e)
        param_bf16[e] = orc_bf16_rne(param[e]);
}

/* ======================================================================== */
/* C5. Group Scaling and activation quantization                             */
/* ======================================================================== */

/*
 * [COAT] section "mixed granularity": the per-tensor max is split into two
 * stages -- a max over every 1xG slice along the channel axis (cached), then a
 * max over that G-times-smaller tensor.
 */
void orc_group_absmax(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                      int64_t G, float *partial, float *amax)
{
    int64_t gpr = cols / G;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < gpr; ++j) {
            double mx = 0.0;
            for (int64_t i = 0; i < G; ++i) {
                double a = fabs(bf16_to_double(x_bf16[r * cols + j * G + i]));
                if (a > mx) mx = a;
            }
            partial[r * gpr + j] = (float)mx;
        }
    *amax = orc_absmax_reduce(partial, rows * gpr);
}

float orc_absmax_reduce(const float *partial, int64_t n)
{
    double mx = 0.0;
    for (int64_t i = 0; i < n; ++i)
        if ((double)partial[i] > mx) mx = (double)partial[i];
    return (float)mx;
}

/*
 * Scaled E4M3 cast: the scale maps the absmax onto the format's max (448),
 * current scaling from the tensor's own statistics ([COAT] "mixed
 * granularity").  The quotient 448 x / a is formed exactly in binary64 and
 * rounded once to FP32 (a quotient of two <=24-bit numbers is never close
 * enough to an FP32 rounding boundary for the binary64 step to matter); the
 * FP8 code is decided from that FP32 value.
 */
static uint8_t scaled_e4m3(double x, double a)
{
    float y = (float)(x * 448.0 / a);
    return (uint8_t)orc_fp8_encode(ORC_E4M3, (double)y);
}

void orc_quant_per_tensor(const uint16_t *x_bf16, int64_t n, float amax,
                          uint8_t *codes, float *scale)
{
    double a = (double)amax;
    if (a == 0.0) {
        for (int64_t i = 0; i < n; ++i) codes[i] = 0;
        *scale = 1.0f;
        return;
    }
    for (int64_t i = 0; i < n; ++i)
        codes[i] = scaled_e4m3(bf16_to_double(x_bf16[i]), a);
    *scale = (float)(a / 448.0);
}

/* [COAT] "mixed granularity": nonlinear-layer inputs are quantized in 1xG
 * groups along the channel axis, never across tokens. */
void orc_quant_group(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                     int64_t G, uint8_t *codes, float *scales, float *partial)
{
    int64_t gpr = cols / G;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < gpr; ++j) {
            int64_t base = r * cols + j * G;
            double a = 0.0;
            for (int64_t i = 0; i < G; ++i) {
                double ax = fabs(bf16_to_double(x_bf16[base + i]));
                if (ax > a) a = ax;
            }
            if (partial) partial[r * gpr + j] = (float)a;
            if (a == 0.0) {
                for (int64_t i = 0; i < G; ++i) codes[base + i] = 0;
                scales[r * gpr + j] = 1.0f;
                continue;
            }
            for (int64_t i = 0; i < G; ++i)
                codes[base + i] = scaled_e4m3(bf16_to_double(x_bf16[base + i]), a);
            scales[r * gpr + j] = (float)(a / 448.0);
        }
}

/*
 * The consumer half of activation compression ([COAT] "mixed granularity"
 * and "why activations are hard": compressed activations are saved for the
 * backward pass and read back there): decode the E4M3 code, multiply by the
 * stored scale in FP32 (the product of a 4-bit and a 24-bit significand is
 * exact in binary64, then rounded once to FP32), round to BF16.
 */
static uint16_t dequant_one(uint8_t code, float scale)
{
    float y = (float)(orc_fp8_decode(ORC_E4M3, code) * (double)scale);
    return orc_bf16_rne(y);
}

void orc_dequant_per_tensor(const uint8_t *codes, int64_t n, float scale, uint16_t *out_bf16)
{
    for (int64_t i = 0; i < n; ++i)
        out_bf16[i] = dequant_one(codes[i], scale);
}

void orc_dequant_group(const uint8_t *codes, int64_t rows, int64_t cols, int64_t G,
                       const float *scales, uint16_t *out_bf16)
{
    int64_t gpr = cols / G;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < gpr; ++j)
            for (int64_t i = 0; i < G; ++i) {
                int64_t e = r * cols + j * G + i;
                out_bf16[e] = dequant_one(codes[e], scales[r * gpr + j]);
            }
}

/* ======================================================================== */
/* SwiGLU producer with Group Scaling stage 1 in its epilogue                */
/* ======================================================================== */

/* The GLU-type activation of [COAT] "why activations are hard": SiLU of the
 * gate times the up projection.  Its output is a linear layer's input, whose
 * per-tensor scale needs the Group Scaling absmax; [COAT] "mixed granularity"
 * has stage 1 fused into the op that produces the tensor. */
double orc_silu(double x)
{
    return x / (1.0 + exp(-x));
}

void orc_swiglu_absmax(const uint16_t *gate, const uint16_t *up, int64_t rows, int64_t cols, int64_t G,
                       uint16_t *h_bf16, float *partial)
{
    int64_t gpr = cols / G;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < gpr; ++j) {
            double mx = 0.0;
            for (int64_t i = 0; i < G; ++i) {
                int64_t e = r * cols + j * G + i;
                double h = orc_silu(bf16_to_double(gate[e])) * bf16_to_double(up[e]);
                uint16_t b = orc_bf16_rne((float)h);
                h_bf16[e] = b;
                double a = fabs(bf16_to_double(b));
                if (a > mx) mx = a;
            }
            partial[r * gpr + j] = (float)mx;
        }
}

/* ======================================================================== */
/* RMSNorm producer with Group Scaling stage 1 in its epilogue               */
/* [COAT] "why activations are hard": the normalization layers are among the */
/* nonlinear layers that hold most of the activation memory; "mixed          */
/* granularity": stage 1 of the following linear layer's per-tensor scale is */
/* taken where its input is produced.  RMSNorm as usually defined:           */
/*   rstd = 1 / sqrt(mean_i x_i^2 + eps),  y_i = x_i * rstd * w_i.           */
/* ======================================================================== */

void orc_rmsnorm_absmax(const uint16_t *x, const uint16_t *weight, int64_t rows, int64_t cols, int64_t G,
                        float eps, uint16_t *y_bf16, float *partial, float *rstd)
{
    int64_t gpr = cols / G;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * cols;
        double ss = 0.0;
        for (int64_t i = 0; i < cols; ++i) {
            double v = bf16_to_double(xr[i]);
            ss += v * v;
        }
        double rs = 1.0 / sqrt(ss / (double)cols + (double)eps);
        if (rstd) rstd[r] = (float)rs;
        for (int64_t j = 0; j < gpr; ++j) {
            double mx = 0.0;
            for (int64_t i = j * G; i < (j + 1) * G; ++i) {
                double y = bf16_to_double(xr[i]) * rs;
                if (weight) y *= bf16_to_double(weight[i]);
                uint16_t b = orc_bf16_rne((float)y);
                y_bf16[r * cols + i] = b;
                double a = fabs(bf16_to_double(b));
                if (a > mx) mx = a;
            }
            partial[r * gpr + j] = (float)mx;
        }
    }
}
