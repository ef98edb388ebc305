/*
 * coat_oracle.h -- CPU oracle for COAT-style FP8 optimizer-state and
 * activation compression.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * reference that the GPU path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It shares
 * no code, header, table or constant with the HIP library, and the HIP library
 * never calls it.
 *
 * Everything is computed in IEEE binary64 and rounded only where the method
 * stores a value (FP32 master weights, FP32 per-group metadata, FP8 codes).
 *
 * Sources (the pages the method is described on):
 *   [COAT]  "COAT: compressing optimizer states and activations for
 *           memory-efficient FP8 training" explainer, blog.daoxuan.cc/posts/57954
 *   [ATLAS] "LLM atlas -- systems / numerics", llm-atlas.k1412.top/systems/numerics
 *   [FP4N]  FP8/FP4/MoFQ reading notes, 53ai.com/news/qianyanjishu/2200.html
 *   [LPF]   "AI low-precision formats (bfloat16/FP8/TF32)" interview notes,
 *           codechuan.com/interview/1/948.html
 *
 * Parity status: every function here is pinned by the CPU tests (codec brute
 * force and page constants, the E2M2 worked grid, the k = 1 reduction, the
 * expansion invariants and error bound, AdamW against torch.optim.AdamW, the
 * step-1 closed form, Group Scaling against torch.amax and torch's FP8 casts,
 * BF16 rounding against torch's cast, dequantization against torch's E4M3
 * decode times the scale, SwiGLU against torch's float64 silu, RMSNorm against
 * torch's float64 rms_norm and its closed forms), and the pins are checked by
 * planting mistakes in a copy of this oracle.
 * The 1.63x quantization-error figure of [COAT] is "parity unpinned": it needs
 * real optimizer states that are not available.
 */
#ifndef COAT_ORACLE_H
#define COAT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Minifloat formats known to the oracle's generic ExMy codec. */
enum {
    ORC_E4M3 = 0, /* OCP E4M3 ("FN"): bias 7, only S.1111.111 is NaN, no inf   */
    ORC_E5M2 = 1, /* OCP E5M2: bias 15, exponent 11111 reserved for inf / NaN    */
    ORC_E2M2 = 2  /* the 4-bit worked example of [FP4N]: bias 2, no specials    */
};

/* ---- C1: codec (by enumeration of the format's grid) -------------------- */

/* Decode one code.  NaN codes return NaN, E5M2 infinities return +-inf. */
double orc_fp8_decode(int fmt, uint32_t code);

/* Round-to-nearest-even onto the format's grid, saturating at +-MAX.
 * A result of magnitude zero is returned as code 0x00 (no negative zero). */
uint32_t orc_fp8_encode(int fmt, double x);

/* Format constants read off the enumerated grid. */
double orc_fp8_max(int fmt);            /* largest finite value             */
double orc_fp8_min_subnormal(int fmt);  /* smallest positive value          */
uint32_t orc_fp8_max_code(int fmt);     /* code magnitude of the max value  */

/* ---- C2 / C3: dynamic-range expansion of one 1xG group ------------------ */

/* Quantize the FP32 group x[0..G) (COAT, section "expansion function").
 * k_force <= 0: k is recomputed so that the expanded group fills the format's
 * range; k_force > 0: that k is used instead (k_force = 1 is plain absmax
 * scaling).  Writes codes[0..G), *amax and *k (both FP32, as stored). */
void orc_expand_quantize(int fmt, const float *x, int64_t G, double k_force,
                         uint8_t *codes, float *amax, float *k);

/* orc_expand_quantize over groups [g0, g1) of x (G elements each); k_given
 * (may be NULL) supplies each group's k instead of recomputing it. */
void orc_expand_quantize_groups(int fmt, const float *x, int64_t g0, int64_t g1, int64_t G,
                                const float *k_given, uint8_t *codes, float *amax, float *k);

/* The code of a value x (any binary64 value) in a group stored with (amax,
 * k): the last step of orc_expand_quantize on its own. */
uint32_t orc_expand_encode(int fmt, double x, float amax, float k);

/* orc_expand_encode of x[i] with its own (amax[i], k[i]), i < n. */
void orc_expand_encode_each(int fmt, const double *x, const float *amax, const float *k, int64_t n,
                            uint8_t *codes);

/* orc_expand_encode of every x of groups [g0, g1) with its group's (amax, k). */
void orc_expand_encode_groups(int fmt, const double *x, int64_t g0, int64_t g1, int64_t G,
                              const float *amax, const float *k, uint8_t *codes);

/* Inverse expansion of one code with its group's stored (amax, k). */
double orc_expand_dequantize(int fmt, uint32_t code, float amax, float k);

/* orc_expand_dequantize of every code of groups [g0, g1) (G codes each). */
void orc_expand_dequantize_groups(int fmt, const uint8_t *codes, int64_t g0, int64_t g1, int64_t G,
                                  const float *amax, const float *k, double *out);

/* Round-to-nearest-even of an FP32 value to BF16, returned as its bit pattern. */
uint16_t orc_bf16_rne(float x);

/* ---- C4: AdamW step with FP8 first/second moments ----------------------- */

typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int64_t step; /* 1-based index of the update being made */
} orc_hparams;

/* One AdamW step over groups [g0, g1) of a flat parameter arena of G-element
 * groups.  m is E4M3; v is ORC_E4M3 or ORC_E5M2.  param, codes and per-group
 * (amax, k) are updated in place; grad holds BF16 bit patterns.  m_new and
 * v_new (each may be NULL) receive the new FP32 moments before they are
 * requantized, indexed like param. */
void orc_adamw_step(float *param, const uint16_t *grad,
                    uint8_t *m_codes, float *m_amax, float *m_k,
                    uint8_t *v_codes, float *v_amax, float *v_k,
                    int64_t g0, int64_t g1, int64_t G, int v_fmt,
                    const orc_hparams *hp, float *m_new, float *v_new);

/* The same step, also writing the BF16 working copy of the updated FP32
 * master weights (round to nearest even) to param_bf16 (indexed like param). */
void orc_adamw_step_bf16(float *param, const uint16_t *grad,
                         uint8_t *m_codes, float *m_amax, float *m_k,
                         uint8_t *v_codes, float *v_amax, float *v_k,
                         int64_t g0, int64_t g1, int64_t G, int v_fmt,
                         const orc_hparams *hp, uint16_t *param_bf16);

/* The same AdamW arithmetic with unquantized binary64 moments (used to pin
 * the update rule against an independent implementation). */
void orc_adamw_step_f64(double *param, const double *grad, double *m, double *v,
                        int64_t n, const orc_hparams *hp);

/* ---- C5: Group Scaling and activation quantization ---------------------- */

/* Stage 1 and stage 2 of Group Scaling: partial[r*(cols/G)+j] is the max |x|
 * over the j-th 1xG group of row r; *amax is the max over all partials. */
void orc_group_absmax(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                      int64_t G, float *partial, float *amax);

/* Stage 2 alone: max over an array of non-negative partial maxima. */
float orc_absmax_reduce(const float *partial, int64_t n);

/* Per-tensor E4M3 cast with the tensor absmax A (current scaling):
 * code = RNE_sat(fp32(448 x / A)), scale = fp32(A / 448); A = 0 -> scale 1. */
void orc_quant_per_tensor(const uint16_t *x_bf16, int64_t n, float amax,
                          uint8_t *codes, float *scale);

/* 1xG group E4M3 quantization: per group a = max|x|, scale = fp32(a / 448),
 * code = RNE_sat(fp32(448 x / a)); a = 0 -> scale 1, codes 0.  partial (may
 * be NULL) receives a. */
void orc_quant_group(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                     int64_t G, uint8_t *codes, float *scales, float *partial);

/* Dequantization of E4M3 activations for the backward pass: per element the
 * FP32 product decode(code) * scale, rounded to BF16 (nearest even).
 * Per-tensor: one scale; group: scales[r*(cols/G)+j] for slice j of row r. */
void orc_dequant_per_tensor(const uint8_t *codes, int64_t n, float scale, uint16_t *out_bf16);
void orc_dequant_group(const uint8_t *codes, int64_t rows, int64_t cols, int64_t G,
                       const float *scales, uint16_t *out_bf16);

/* SwiGLU with Group Scaling stage 1 fused into its epilogue: per element
 * h = silu(gate) * up (silu(x) = x / (1 + e^-x)), formed in binary64, rounded
 * to FP32 and then to BF16 (nearest even); partial[r*(cols/G)+j] = max |h| over
 * slice j of row r (h as stored). */
double orc_silu(double x);
void orc_swiglu_absmax(const uint16_t *gate, const uint16_t *up, int64_t rows, int64_t cols, int64_t G,
                       uint16_t *h_bf16, float *partial);

/* RMSNorm with Group Scaling stage 1 fused into its epilogue: per row
 * rstd = 1 / sqrt(mean x^2 + eps) and y = x * rstd * w (w = 1 when weight is
 * NULL), in binary64, y rounded to FP32 and then BF16 (nearest even);
 * partial[r*(cols/G)+j] = max |y| over slice j of row r (y as stored);
 * rstd (may be NULL) receives fp32(rstd) per row. */
void orc_rmsnorm_absmax(const uint16_t *x, const uint16_t *weight, int64_t rows, int64_t cols, int64_t G,
                        float eps, uint16_t *y_bf16, float *partial, float *rstd);

#ifdef __cplusplus
}
#endif
#endif
