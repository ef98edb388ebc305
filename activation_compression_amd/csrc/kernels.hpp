// kernels.hpp -- internal launch interface between the C ABI (abi.hip) and
// the kernel translation units.  Host code; no torch, no oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coat {

// One tensor's (or one arena's) buffers for the fused FP8-state AdamW step.
// Also the device layout of one entry of a tensor-list table (80 bytes).
struct StepBufs {
    float *param;
    const uint16_t *grad;
    uint8_t *m_codes;
    float *m_amax, *m_k;
    uint8_t *v_codes;
    float *v_amax, *v_k;
    uint16_t *param_bf16;  // BF16 working copy of the updated weights, or null
    int64_t n;             // parameters, a multiple of the group size
};
static_assert(sizeof(StepBufs) == 80, "tensor-list entry layout");

// Per-step scalars, folded on the host (binary64, rounded once to FP32).
struct StepParams {
    float beta1, omb1;    // beta1 and 1 - beta1 (exact in FP32 for beta1 in [0.5, 1))
    float beta2, omb2;
    float step_size;      // lr / (1 - beta1^t)
    float inv_sqrt_bc2;   // 1 / sqrt(1 - beta2^t)
    float eps;
    float decay;          // 1 - lr * weight_decay
    float m_log2_range;   // log2(MAX / smallest subnormal) of m's format
    float v_log2_range;   // ... of v's format
    // log2(|decode(c)| / MAX) for every code magnitude c, as an FP32 hi + lo
    // pair (code 0 and non-finite codes hold -2^40): m's format, then v's.
    float2 log_tab[2][128];
};

// One flat arena, one launch.
struct StepArgs {
    StepBufs buf;
    int64_t n_chunks;  // ceil(n / 1024): one wave handles 1024 per pass
    StepParams p;
};

// A list of separately allocated tensors, one launch.  The table lives in
// device memory: chunk_start[t] is the first 1024-parameter chunk of tensor t
// in the launch's chunk numbering (chunk_start[0] = 0, chunk_start[n_tensors]
// = total_chunks); entries[t] holds its buffers.
struct StepListArgs {
    const int64_t *chunk_start;
    const StepBufs *entries;
    int64_t total_chunks;
    int32_t n_tensors;
    int32_t has_bf16;  // every entry has a BF16 copy (else none has)
    StepParams p;
};

// Fill tab[c] = log2(|decode(c)| / MAX) for the 128 code magnitudes of an OCP
// FP8 format (0: E4M3, 1: E5M2), computed once per format in binary64.
const float2 *fp8_log_table(int fmt);

// Residency cap of the streaming kernels.  With fewer requests in flight
// HBM serves this many-stream traffic better: measured on MI355X, the
// optimizer step ran 20.66 ms at its register-limited 6 workgroups per CU,
// 20.18 at 5 and 20.16 at 4, 20.5 at 3; SwiGLU 4% and the dequantization 2%
// faster at 5 than at 8.  The casts and stage 1 ran up to 9% slower capped
// and are left uncapped.  A kernel is held to kStreamBlocksPerCu by
// requesting dynamic LDS it does not use: stream_lds_bytes(static) bytes on
// top of its static LDS (abi.hip; 0 when the device cannot be queried).
constexpr int kStreamBlocksPerCu = 5;
size_t stream_lds_bytes(size_t static_lds);

// Streaming kernels give each wave one 1024-element chunk (no grid-stride
// loop: the hardware dispatcher then sweeps the arrays in order, which keeps
// DRAM pages open); the small reduction kernel of stage 2 is grid-stride and
// sizes its grid from the device's compute-unit count (num_cus).
hipError_t launch_adamw_fp8_step(const StepArgs &a, int group_size, int v_format,
                                 hipStream_t stream, int num_cus);
hipError_t launch_adamw_fp8_step_list(const StepListArgs &a, int group_size, int v_format, hipStream_t stream);

hipError_t launch_group_absmax(const uint16_t *x, int64_t n, int group_size, float *partial,
                               float *amax, hipStream_t stream, int num_cus);
hipError_t launch_absmax_reduce(const float *partial, int64_t n, float *amax,
                                hipStream_t stream, int num_cus);
hipError_t launch_quant_per_tensor(const uint16_t *x, int64_t n, const float *amax,
                                   uint8_t *codes, float *scale, hipStream_t stream, int num_cus);
hipError_t launch_quant_group(const uint16_t *x, int64_t n, int group_size, uint8_t *codes,
                              float *scales, float *partial, hipStream_t stream, int num_cus);
hipError_t launch_dequant_per_tensor(const uint8_t *codes, int64_t n, const float *scale, uint16_t *out,
                                     hipStream_t stream);
constexpr int kRmsNormMaxCols = 8192;  // one row per wave, held in registers
hipError_t launch_rmsnorm_fused(const uint16_t *x, const uint16_t *weight, int64_t rows, int cols, int group_size,
                                float eps, uint16_t *y, float *y_partial, float *rstd, uint8_t *x_codes,
                                float *x_scales, hipStream_t stream);
hipError_t launch_swiglu_fused(const uint16_t *gate, const uint16_t *up, int64_t n, int group_size, uint16_t *h,
                               float *h_partial, uint8_t *gate_codes, float *gate_scales, uint8_t *up_codes,
                               float *up_scales, hipStream_t stream);
hipError_t launch_dequant_group(const uint8_t *codes, int64_t n, int group_size, const float *scales,
                                uint16_t *out, hipStream_t stream);

constexpr int kBlock = 256;       // threads per workgroup: 4 wave64s
constexpr int kWaveElems = 1024;  // elements per wave pass: 64 lanes x 16

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups of `Kernel` resident on one CU (looked up once per kernel; the
// answer depends only on the kernel's resources and the architecture).
template <auto Kernel>
inline int resident_blocks_per_cu() {
    static int cached = 0;
    const int v = __atomic_load_n(&cached, __ATOMIC_RELAXED);
    if (v > 0) return v;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void *>(Kernel), kBlock, 0) !=
            hipSuccess || occ <= 0)
        occ = 1;
    __atomic_store_n(&cached, occ, __ATOMIC_RELAXED);
    return occ;
}

// Grid for a grid-stride kernel needing `want` workgroups' worth of work.
template <auto Kernel>
inline dim3 resident_grid(int64_t want, int num_cus) {
    const int64_t cap = (int64_t)resident_blocks_per_cu<Kernel>() * num_cus;
    const int64_t g = want < cap ? want : cap;
    return dim3((unsigned)(g > 0 ? g : 1));
}

}  // namespace coat
