/*
 * coat.h -- C ABI of the MI355X (gfx950) kernels for COAT-style FP8
 * compression of AdamW optimizer states and activations.
 *
 * Sources (the pages the method is described on):
 *   [COAT]  "COAT: compressing optimizer states and activations for
 *           memory-efficient FP8 training" explainer, blog.daoxuan.cc/posts/57954
 *   [ATLAS] "LLM atlas -- systems / numerics", llm-atlas.k1412.top/systems/numerics
 *   [LPF]   "AI low-precision formats (bfloat16/FP8/TF32)" interview notes,
 *           codechuan.com/interview/1/948.html
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *   allocates no device memory, keeps no state between calls and never
 *   synchronizes: all work is enqueued on `stream` (a hipStream_t passed as
 *   void*, NULL for the default stream) and every result, including
 *   per-tensor statistics, is written to device memory.
 * - Arguments are validated before anything is enqueued.  On any error the
 *   call returns a non-zero coat_status, enqueues nothing and leaves every
 *   buffer untouched.  Launch failures return COAT_ERR_HIP.  Device faults
 *   surface at the caller's next synchronization of `stream`.
 * - Distinct arrays must not overlap.  Calls on disjoint buffers may run
 *   concurrently from any host thread.  No C++ exception crosses the ABI.
 * - BF16 values are passed as their 16-bit patterns (uint16_t); FP8 codes as
 *   uint8_t in the OCP encodings: E4M3 (bias 7, max 448, smallest subnormal
 *   2^-9, only S.1111.111 is NaN) and E5M2 (bias 15, max 57344, smallest
 *   subnormal 2^-16) -- [ATLAS] sections "01 Number anatomy" and "03 FP8".
 *   Codes 0x00 and 0x80 both mean zero.  No NaN or infinity code is produced.
 * - FP8 rounding is round-to-nearest-even with saturation at +-MAX.
 * - Group size G: a power of two in [32, 1024].  Groups are 1xG runs of
 *   contiguous elements ([COAT] section "mixed granularity": along the channel
 *   axis, never across tokens); the optimizer groups are consecutive runs of
 *   the flat parameter arena, so a tensor whose size is a multiple of G never
 *   shares a group with its neighbour.
 * - Sizes: one launch covers at most (2^31 - 1) * 4096 elements (about
 *   8.8e12; the launch grid's limit); larger sizes return COAT_ERR_SHAPE.
 * - NaN or infinite inputs are outside the contract.
 */
#ifndef COAT_H
#define COAT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    COAT_OK = 0,
    COAT_ERR_NULL = 1,   /* a required pointer is NULL                          */
    COAT_ERR_ALIGN = 2,  /* a pointer misses its required alignment             */
    COAT_ERR_SHAPE = 3,  /* n / rows / cols out of range or not divisible       */
    COAT_ERR_GROUP = 4,  /* group size not a power of two in [32, 1024]         */
    COAT_ERR_FORMAT = 5, /* unknown FP8 format                                  */
    COAT_ERR_HPARAM = 6, /* beta outside [0,1), eps below FLT_MIN (2^-126),
                            step < 1, non-finite lr / wd / eps, or
                            lr / (1 - beta1^step) or 1 - lr * wd not finite
                            in FP32                                             */
    COAT_ERR_HIP = 7,    /* the HIP runtime refused the launch                  */
    COAT_ERR_SCRATCH = 8 /* the request exceeds the library's static device
                            scratch (coat_adamw_step_list_noalloc only)        */
} coat_status;

typedef enum {
    COAT_FP8_E4M3 = 0,
    COAT_FP8_E5M2 = 1
} coat_fp8_format;

/* AdamW hyper-parameters, FP32 as the caller holds them.  `step` is the
 * 1-based index of the update being made (the caller increments it before
 * each call); it drives the bias corrections 1 - beta^step. */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int64_t step;
} coat_adamw_hparams;

/*
 * coat_adamw_step -- one fused AdamW update of n parameters whose moments are
 * stored in FP8 with per-group dynamic-range expansion.
 *
 * Per 1xG group and per step ([COAT] sections on second-moment sensitivity,
 * on the smaller dynamic range of v, and "expansion function"; the update rule
 * of [ATLAS] section "08 Adam -> AdamW"; FP32 master weights per [LPF]):
 *   1. dequantize m and v:  x = sign(c) * amax * (|dec(c)| / MAX)^(1/k)
 *      with the group's stored (amax, k) -- the inverse of f(x) = sign(x)|x|^k;
 *   2. AdamW in FP32 on the FP32 master weights:
 *        m' = b1 m + (1-b1) g,   v' = b2 v + (1-b2) g^2,
 *        theta' = (1 - lr wd) theta - lr (m'/(1-b1^t)) / (sqrt(v'/(1-b2^t)) + eps);
 *   3. per group, amax = max|x| and amin = min over nonzero |x| of the new
 *      moment, k = ln(MAX / min_subnormal) / ln(amax / amin) so that the
 *      expanded group fills the FP8 range (k = 1 when amax = amin or amax = 0;
 *      k < 1 is allowed for groups wider than the format);
 *   4. requantize: c = RNE_sat(sign(x) * MAX * (|x| / amax)^k); store the codes
 *      and the new (amax, k).
 *
 * param      FP32 [n], read and written.                  16-byte aligned.
 * grad_bf16  BF16 bit patterns [n], read only.            16-byte aligned.
 * m_codes    E4M3 codes [n], read and written.            16-byte aligned.
 * m_amax     FP32 [n/G] group absmax of m, read/written.  4-byte aligned.
 * m_k        FP32 [n/G] expansion exponent of m.          4-byte aligned.
 * v_codes    codes [n] in `v_format`, read and written.   16-byte aligned.
 * v_amax, v_k  as for m.
 * n          number of parameters, > 0, a multiple of G.  A parameter set is
 *            passed as one flat arena (one launch for the whole model).
 * group_size G.   v_format  COAT_FP8_E4M3 or COAT_FP8_E5M2 (m is always E4M3).
 * hp         host pointer, read during the call only.
 * A never-updated state is codes 0, amax 0, k 1; any other state must be
 * one a previous call wrote (or a byte copy of it: a checkpoint).
 * Range: any finite moments, including groups whose max / min spans more
 * than FP32's own ratio range (k down to about 0.064); the new moments must
 * be finite in FP32, which bounds |g| by about sqrt(FLT_MAX / (1 - b2))
 * (5.8e20 at b2 = 0.999).
 */
coat_status coat_adamw_step(float *param, const uint16_t *grad_bf16,
                            uint8_t *m_codes, float *m_amax, float *m_k,
                            uint8_t *v_codes, float *v_amax, float *v_k,
                            int64_t n, int32_t group_size, coat_fp8_format v_format,
                            const coat_adamw_hparams *hp, void *stream);

/*
 * coat_adamw_step_bf16 -- coat_adamw_step that also writes the BF16 working
 * copy of the updated master weights, round to nearest even, from the same
 * pass ([LPF]: FP32 master weights are updated, the BF16 copy is what the
 * forward and backward passes compute with).  2 extra bytes per parameter
 * instead of a separate cast kernel's 6.
 *
 * param_bf16  BF16 bit patterns [n], written.  16-byte aligned; must not
 *             overlap any other argument.  All other arguments, layout and
 *             errors as coat_adamw_step (NULL param_bf16 -> COAT_ERR_NULL).
 */
coat_status coat_adamw_step_bf16(float *param, const uint16_t *grad_bf16,
                                 uint8_t *m_codes, float *m_amax, float *m_k,
                                 uint8_t *v_codes, float *v_amax, float *v_k,
                                 uint16_t *param_bf16,
                                 int64_t n, int32_t group_size, coat_fp8_format v_format,
                                 const coat_adamw_hparams *hp, void *stream);

/*
 * Tensor-list form of the step: the parameters live in separate allocations
 * (one per tensor, as a training framework keeps them) instead of one arena,
 * and all of them are updated by ONE launch.  Each tensor follows exactly the
 * per-group arithmetic of coat_adamw_step (the same update rule and expansion,
 * [COAT] and [ATLAS] as cited there); since groups never straddle tensors,
 * the result is bit for bit that of one coat_adamw_step call per tensor.
 *
 * Use: describe the tensors with coat_adamw_tensor entries; pack them once into
 * a host table of coat_adamw_list_bytes(n) bytes (coat_adamw_list_pack
 * validates every entry as coat_adamw_step would); copy that table, unchanged,
 * into device memory the caller owns (16-byte aligned); then call
 * coat_adamw_step_list with both copies every step.  The tables stay valid
 * while the tensors stay where they are; the library keeps no pointer to them
 * after a call returns, and the device copy must stay alive until the launch
 * has run (stream order).
 */
typedef struct {
    float *param;              /* FP32 [n], 16-byte aligned                    */
    const uint16_t *grad_bf16; /* BF16 [n], 16-byte aligned                    */
    uint8_t *m_codes;          /* E4M3 [n], 16-byte aligned                    */
    float *m_amax, *m_k;       /* FP32 [n/G] each, 4-byte aligned              */
    uint8_t *v_codes;          /* [n] in the list's v format, 16-byte aligned  */
    float *v_amax, *v_k;       /* FP32 [n/G] each                              */
    uint16_t *param_bf16;      /* BF16 working copy [n], or NULL: all entries of
                                  a list NULL or all set (else COAT_ERR_NULL)   */
    int64_t n;                 /* parameters, > 0, a multiple of G             */
} coat_adamw_tensor;

/* Size in bytes of the packed table for n_tensors tensors (0 if n_tensors <= 0). */
int64_t coat_adamw_list_bytes(int32_t n_tensors);

/* Validate tensors[0..n_tensors) for group size G and write the packed table to
 * table_host (coat_adamw_list_bytes(n_tensors) bytes, any alignment).  Errors:
 * COAT_ERR_NULL, _ALIGN, _GROUP, _SHAPE as coat_adamw_step per entry;
 * n_tensors <= 0 -> COAT_ERR_SHAPE.  Nothing is written on error. */
coat_status coat_adamw_list_pack(const coat_adamw_tensor *tensors, int32_t n_tensors, int32_t group_size,
                                 void *table_host);

/* One fused step over every tensor of a packed list.  table_host: the table
 * coat_adamw_list_pack wrote (read during the call: launch size, G, whether a
 * BF16 copy is written); table_device: its byte-identical device copy, read by
 * the kernel.  v_format and hp as coat_adamw_step.  A table that does not carry
 * the packer's header -> COAT_ERR_SHAPE. */
coat_status coat_adamw_step_list(const void *table_host, const void *table_device, coat_fp8_format v_format,
                                 const coat_adamw_hparams *hp, void *stream);

/*
 * coat_adamw_step_list_noalloc -- coat_adamw_step_list for callers that cannot
 * allocate device memory: code that must not call hipMalloc (tight training
 * or serving loops, harnesses that forbid allocation) and so has no device
 * copy of the table to pass.  The table is copied, on `stream`, into a device
 * array the library owns -- COAT_LIST_NOALLOC_MAX_BYTES (64 KiB, enough for
 * 744 tensors; coat_adamw_list_bytes gives a table's size), held by every GPU
 * the library runs on until the process ends -- and the same kernel then
 * reads it there.  The call allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine.
 *
 * table_host  the table coat_adamw_list_pack wrote.  It is read by the copy
 *             the call enqueues: keep it unchanged until `stream` has run
 *             that copy (as for any asynchronous copy from host memory).
 * v_format, hp, stream  as coat_adamw_step_list; the result is identical.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (other streams, other host threads) race, and must be ordered by
 * the caller.  A table larger than COAT_LIST_NOALLOC_MAX_BYTES ->
 * COAT_ERR_SCRATCH; other errors as coat_adamw_step_list.  A call rejected by
 * its argument checks enqueues nothing; if the launch itself fails
 * (COAT_ERR_HIP), the table copy may already be enqueued.
 */
#define COAT_LIST_NOALLOC_MAX_BYTES 65536
coat_status coat_adamw_step_list_noalloc(const void *table_host, coat_fp8_format v_format,
                                         const coat_adamw_hparams *hp, void *stream);

/*
 * coat_group_absmax -- both stages of Group Scaling ([COAT] section "mixed
 * granularity"): stage 1 writes the max |x| of every 1xG slice of each row,
 * stage 2 reduces that G-times-smaller tensor to the tensor absmax.
 *
 * x_bf16        BF16 [rows x cols] row-major, read only.  16-byte aligned.
 * rows, cols    rows > 0; cols > 0, a multiple of G.
 * partial_amax  FP32 [rows * cols / G], written (row r, slice j at r*(cols/G)+j).
 *               4-byte aligned.
 * amax          FP32 [1], written: max over partial_amax (exact; both are
 *               BF16 values held in FP32).
 */
coat_status coat_group_absmax(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                              int32_t group_size, float *partial_amax, float *amax,
                              void *stream);

/*
 * coat_absmax_reduce -- stage 2 of Group Scaling alone, for partial maxima
 * produced elsewhere (for example by coat_quant_group): amax = max partial.
 *
 * partial  FP32 [n] non-negative values, read only.  4-byte aligned.  n > 0.
 * amax     FP32 [1], written.
 */
coat_status coat_absmax_reduce(const float *partial, int64_t n, float *amax, void *stream);

/*
 * coat_quant_per_tensor -- per-tensor E4M3 cast of a linear-layer input with
 * current (just-in-time) scaling from the tensor's own absmax ([COAT] section
 * "mixed granularity"):
 *   A = *amax (device scalar, e.g. from coat_group_absmax, read on device);
 *   code = RNE_sat(y) with y the FP32 value of 448 * x / A (correctly
 *   rounded quotient); *scale = FP32(A / 448), the dequantization scale.
 *   A = 0 gives scale 1 and all codes 0.  A need not be max |x| (a scale
 *   kept from an earlier step, say): larger values saturate to +-448, also
 *   where 448 x / A exceeds FP32.
 *
 * x_bf16  BF16 [n], read only.  16-byte aligned.  n > 0, a multiple of 8.
 * amax    FP32 [1] device scalar, read only.
 * codes   E4M3 [n], written.  16-byte aligned.
 * scale   FP32 [1], written.
 */
coat_status coat_quant_per_tensor(const uint16_t *x_bf16, int64_t n, const float *amax,
                                  uint8_t *codes, float *scale, void *stream);

/*
 * coat_quant_group -- 1xG E4M3 quantization of a nonlinear-layer input
 * ([COAT] section "mixed granularity"): per slice a = max |x|,
 * code = RNE_sat(FP32(448 * x / a)), scale = FP32(a / 448); a = 0 gives
 * scale 1 and codes 0.  When partial_amax_or_null is not NULL it also
 * receives a -- stage 1 of Group Scaling from the same pass.
 *
 * x_bf16   BF16 [rows x cols] row-major, read only.  16-byte aligned.
 * codes    E4M3 [rows x cols], written.  16-byte aligned.
 * scales   FP32 [rows * cols / G], written.  4-byte aligned.
 * partial_amax_or_null  FP32 [rows * cols / G] or NULL.
 */
coat_status coat_quant_group(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                             int32_t group_size, uint8_t *codes, float *scales,
                             float *partial_amax_or_null, void *stream);

/*
 * coat_dequant_per_tensor / coat_dequant_group -- E4M3 activations back to
 * BF16 for the backward pass, the consumer half of activation compression
 * ([COAT] sections "why activations are hard" and "mixed granularity":
 * compressed activations are saved for, and read back in, the backward pass).
 * Per element: y = FP32(decode(code) * scale) (the correctly rounded FP32
 * product), stored as BF16, round to nearest even.
 *
 * codes     E4M3 [n] or [rows x cols], read only.  16-byte aligned.
 * scale     FP32 [1] device scalar (per-tensor), as written by
 *           coat_quant_per_tensor.  4-byte aligned.
 * scales    FP32 [rows * cols / G] (group), as written by coat_quant_group.
 * out_bf16  BF16 bit patterns, same count as codes, written.  16-byte aligned.
 * n         > 0, a multiple of 8.  rows, cols, G as for coat_quant_group.
 */
coat_status coat_dequant_per_tensor(const uint8_t *codes, int64_t n, const float *scale,
                                    uint16_t *out_bf16, void *stream);
coat_status coat_dequant_group(const uint8_t *codes, int64_t rows, int64_t cols, int32_t group_size,
                               const float *scales, uint16_t *out_bf16, void *stream);

/*
 * coat_swiglu_fused -- SwiGLU with Group Scaling stage 1 fused into its
 * epilogue ([COAT] "mixed granularity": the per-slice max is cached by the op
 * that produces the tensor, so stage 1 costs no second read; [COAT] "why
 * activations are hard": GLU-type activations are the outlier-heavy ones).
 *   h = silu(gate) * up, silu(x) = x / (1 + e^-x), in FP32, stored as BF16
 *   (round to nearest even); h_partial_amax[r*(cols/G)+j] = max |h| over
 *   slice j of row r (as stored).  coat_absmax_reduce then gives the tensor
 *   absmax for coat_quant_per_tensor of h (the down projection's input).
 * Optionally, in the same pass, SwiGLU's own inputs are saved for the
 * backward pass as 1xG E4M3 exactly as coat_quant_group would write them.
 *
 * gate_bf16, up_bf16  BF16 [rows x cols] row-major, read only.  16-byte aligned.
 * h_bf16              BF16 [rows x cols], written.  16-byte aligned.
 * h_partial_amax      FP32 [rows * cols / G], written.  4-byte aligned.
 * gate_codes, up_codes    E4M3 [rows x cols] or NULL; 16-byte aligned.
 * gate_scales, up_scales  FP32 [rows * cols / G] or NULL; all four NULL or
 *                     all four set (else COAT_ERR_NULL).
 * rows, cols, G as for coat_quant_group.  h agrees with a binary64 evaluation
 * rounded to FP32 and then BF16 to within one BF16 step (FP32 exp and
 * reciprocal).
 */
coat_status coat_swiglu_fused(const uint16_t *gate_bf16, const uint16_t *up_bf16, int64_t rows, int64_t cols,
                              int32_t group_size, uint16_t *h_bf16, float *h_partial_amax,
                              uint8_t *gate_codes, float *gate_scales, uint8_t *up_codes, float *up_scales,
                              void *stream);

/*
 * coat_rmsnorm_fused -- RMSNorm with Group Scaling stage 1 fused into its
 * epilogue ([COAT] "why activations are hard": normalization layers are among
 * the nonlinear layers that dominate activation memory; [COAT] "mixed
 * granularity": stage 1 is taken by the op that produces the tensor, and the
 * normalization's input is saved in 1xG groups along the channel axis).
 *   rstd = 1 / sqrt(mean_c x^2 + eps) per row, y = x * rstd * w, FP32, y
 *   stored as BF16 (round to nearest even); y_partial_amax[r*(cols/G)+j] =
 *   max |y| over slice j of row r (as stored).  coat_absmax_reduce then gives
 *   the tensor absmax for coat_quant_per_tensor of y (the next linear layer's
 *   input).  Optionally, in the same pass, x is saved for the backward pass as
 *   1xG E4M3 exactly as coat_quant_group would write it, and rstd per row.
 *
 * x_bf16        BF16 [rows x cols] row-major, read only.  16-byte aligned.
 * weight_bf16   BF16 [cols] gain, or NULL for none.  16-byte aligned.
 * eps           > 0 and finite (else COAT_ERR_HPARAM).
 * y_bf16        BF16 [rows x cols], written.  16-byte aligned.
 * y_partial_amax  FP32 [rows * cols / G], written.
 * rstd          FP32 [rows] or NULL.
 * x_codes, x_scales  E4M3 [rows x cols] (16-byte aligned) and FP32
 *               [rows * cols / G], both NULL or both set (else COAT_ERR_NULL).
 * rows > 0; cols % G == 0 and cols <= 8192 (one row is held by one wave),
 * else COAT_ERR_SHAPE.  The row's sum of squares is taken in FP32, so y
 * agrees with a binary64 evaluation rounded to FP32 and then BF16 to within
 * one BF16 step.
 */
coat_status coat_rmsnorm_fused(const uint16_t *x_bf16, const uint16_t *weight_bf16, int64_t rows, int64_t cols,
                               float eps, int32_t group_size, uint16_t *y_bf16, float *y_partial_amax,
                               float *rstd, uint8_t *x_codes, float *x_scales, void *stream);

/* Static, human-readable name of a status code. */
const char *coat_status_string(coat_status s);

#ifdef __cplusplus
}
#endif
#endif /* COAT_H */
