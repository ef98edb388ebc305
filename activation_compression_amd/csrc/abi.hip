// abi.hip -- the C ABI of include/coat.h: argument validation, per-step
// scalar folding and kernel dispatch.  Nothing is enqueued unless every
// argument is valid; no device memory is allocated; no call synchronizes.
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/coat.h"
#include "kernels.hpp"

namespace {

using coat::kBlock;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_group(int32_t G) { return G >= 32 && G <= 1024 && (G & (G - 1)) == 0; }

// Streaming launches give each 256-thread workgroup 4096 elements; the grid's
// x dimension must stay below 2^31.
constexpr int64_t kMaxElems = (int64_t)0x7FFFFFFF * coat::kWaveElems * (coat::kBlock / 64);
bool fits_grid(int64_t n) { return n <= kMaxElems; }

// Compute units of the current device, looked up once per device.
int num_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

coat_status from_hip(hipError_t e) { return e == hipSuccess ? COAT_OK : COAT_ERR_HIP; }

}  // namespace

namespace coat {

size_t stream_lds_bytes(size_t static_lds) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    int lds = dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (lds <= 0) {
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            lds <= 0)
            return 0;
        if (dev < 64) cache[dev].store(lds, std::memory_order_relaxed);
    }
    const size_t per_block = (size_t)lds / kStreamBlocksPerCu;
    return per_block > static_lds ? per_block - static_lds : 0;
}

}  // namespace coat

extern "C" {

const char *coat_status_string(coat_status s) {
    switch (s) {
    case COAT_OK: return "ok";
    case COAT_ERR_NULL: return "null pointer argument";
    case COAT_ERR_ALIGN: return "misaligned pointer argument";
    case COAT_ERR_SHAPE: return "invalid size: n, rows or cols out of range or not a multiple of the group";
    case COAT_ERR_GROUP: return "group size must be a power of two in [32, 1024]";
    case COAT_ERR_FORMAT: return "unknown FP8 format";
    case COAT_ERR_HPARAM: return "invalid AdamW hyper-parameters";
    case COAT_ERR_HIP: return "HIP runtime error while enqueueing";
    case COAT_ERR_SCRATCH: return "the request exceeds the library's static device scratch";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

// eps must be a normal float so that the kernel's reciprocal of the
// denominator sqrt(v) / sqrt(1 - b2^t) + eps >= eps stays finite (a zero
// moment over a zero second moment is then 0, not 0 * inf); the per-step
// factors lr / (1 - b1^t) and 1 - lr wd must be finite in FP32.
bool valid_hparams(const coat_adamw_hparams *hp) {
    const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps, wd = hp->weight_decay;
    if (!(isfinite(lr) && isfinite(wd) && isfinite(eps) && b1 >= 0.0 && b1 < 1.0 && b2 >= 0.0 && b2 < 1.0 &&
          eps >= (double)FLT_MIN && hp->step >= 1))
        return false;
    const double bc1 = 1.0 - pow(b1, (double)hp->step);
    return isfinite((float)(lr / bc1)) && isfinite((float)(1.0 - lr * wd));
}

// Per-step scalars in binary64, rounded once.
void make_params(const coat_adamw_hparams *hp, coat_fp8_format v_format, coat::StepParams &p) {
    const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, wd = hp->weight_decay;
    const double t = (double)hp->step;
    const double bc1 = 1.0 - pow(b1, t), bc2 = 1.0 - pow(b2, t);
    p.beta1 = hp->beta1; p.omb1 = (float)(1.0 - b1);
    p.beta2 = hp->beta2; p.omb2 = (float)(1.0 - b2);
    p.step_size = (float)(lr / bc1);
    p.inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
    p.eps = hp->eps;
    p.decay = (float)(1.0 - lr * wd);
    // log2 of each format's range MAX / smallest subnormal
    p.m_log2_range = (float)(log2(448.0) + 9.0);
    p.v_log2_range = v_format == COAT_FP8_E5M2 ? (float)(log2(57344.0) + 16.0) : p.m_log2_range;
    memcpy(p.log_tab[0], coat::fp8_log_table(COAT_FP8_E4M3), sizeof p.log_tab[0]);
    memcpy(p.log_tab[1], coat::fp8_log_table((int)v_format), sizeof p.log_tab[1]);
}

// One tensor's buffers: shared by the arena and tensor-list forms.
coat_status check_bufs(const coat::StepBufs &b, int32_t group_size) {
    if (!b.param || !b.grad || !b.m_codes || !b.m_amax || !b.m_k || !b.v_codes || !b.v_amax || !b.v_k)
        return COAT_ERR_NULL;
    if (!aligned(b.param, 16) || !aligned(b.grad, 16) || !aligned(b.m_codes, 16) || !aligned(b.v_codes, 16) ||
        !aligned(b.m_amax, 4) || !aligned(b.m_k, 4) || !aligned(b.v_amax, 4) || !aligned(b.v_k, 4) ||
        (b.param_bf16 && !aligned(b.param_bf16, 16)))
        return COAT_ERR_ALIGN;
    if (!valid_group(group_size)) return COAT_ERR_GROUP;
    if (b.n <= 0 || b.n % group_size != 0 || !fits_grid(b.n)) return COAT_ERR_SHAPE;
    return COAT_OK;
}

coat_status adamw_step_impl(float *param, const uint16_t *grad_bf16, uint8_t *m_codes, float *m_amax, float *m_k,
                            uint8_t *v_codes, float *v_amax, float *v_k, int64_t n, int32_t group_size,
                            coat_fp8_format v_format, const coat_adamw_hparams *hp, uint16_t *param_bf16,
                            void *stream) {
    coat::StepArgs a;
    a.buf = coat::StepBufs{param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k, param_bf16, n};
    if (!hp) return COAT_ERR_NULL;
    const coat_status s = check_bufs(a.buf, group_size);
    if (s != COAT_OK) return s;
    if (v_format != COAT_FP8_E4M3 && v_format != COAT_FP8_E5M2) return COAT_ERR_FORMAT;
    if (!valid_hparams(hp)) return COAT_ERR_HPARAM;
    a.n_chunks = coat::ceil_div(n, coat::kWaveElems);
    make_params(hp, v_format, a.p);
    return from_hip(coat::launch_adamw_fp8_step(a, group_size, (int)v_format, (hipStream_t)stream, num_cus()));
}

// Packed tensor-list table: header | int64 chunk_start[n + 1] (padded to 16
// bytes) | StepBufs entries[n].  Written on the host by coat_adamw_list_pack;
// the kernel reads the caller's device copy.
struct ListHeader {
    uint32_t magic;
    uint32_t version;
    int32_t n_tensors;
    int32_t group_size;
    int32_t has_bf16;
    int32_t reserved;
    int64_t total_chunks;
};
static_assert(sizeof(ListHeader) == 32, "list header layout");
constexpr uint32_t kListMagic = 0x4C54414Fu;
constexpr uint32_t kListVersion = 1;

int64_t list_starts_bytes(int32_t n) { return (8 * ((int64_t)n + 1) + 15) / 16 * 16; }

coat::StepBufs to_bufs(const coat_adamw_tensor &x) {
    return coat::StepBufs{x.param, x.grad_bf16, x.m_codes, x.m_amax, x.m_k, x.v_codes, x.v_amax, x.v_k,
                          x.param_bf16, x.n};
}

}  // namespace

extern "C" {

coat_status coat_adamw_step(float *param, const uint16_t *grad_bf16, uint8_t *m_codes, float *m_amax,
                            float *m_k, uint8_t *v_codes, float *v_amax, float *v_k, int64_t n,
                            int32_t group_size, coat_fp8_format v_format, const coat_adamw_hparams *hp,
                            void *stream) {
    return adamw_step_impl(param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k, n, group_size, v_format,
                           hp, nullptr, stream);
}

coat_status coat_adamw_step_bf16(float *param, const uint16_t *grad_bf16, uint8_t *m_codes, float *m_amax,
                                 float *m_k, uint8_t *v_codes, float *v_amax, float *v_k, uint16_t *param_bf16,
                                 int64_t n, int32_t group_size, coat_fp8_format v_format,
                                 const coat_adamw_hparams *hp, void *stream) {
    if (!param_bf16) return COAT_ERR_NULL;
    return adamw_step_impl(param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k, n, group_size, v_format,
                           hp, param_bf16, stream);
}

coat_status coat_group_absmax(const uint16_t *x_bf16, int64_t rows, int64_t cols, int32_t group_size,
                              float *partial_amax, float *amax, void *stream) {
    if (!x_bf16 || !partial_amax || !amax) return COAT_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(partial_amax, 4) || !aligned(amax, 4)) return COAT_ERR_ALIGN;
    if (!valid_group(group_size)) return COAT_ERR_GROUP;
    if (rows <= 0 || cols <= 0 || cols % group_size != 0 || rows > INT64_MAX / cols || !fits_grid(rows * cols))
        return COAT_ERR_SHAPE;
    return from_hip(coat::launch_group_absmax(x_bf16, rows * cols, group_size, partial_amax, amax,
                                              (hipStream_t)stream, num_cus()));
}

coat_status coat_absmax_reduce(const float *partial, int64_t n, float *amax, void *stream) {
    if (!partial || !amax) return COAT_ERR_NULL;
    if (!aligned(partial, 4) || !aligned(amax, 4)) return COAT_ERR_ALIGN;
    if (n <= 0) return COAT_ERR_SHAPE;
    return from_hip(coat::launch_absmax_reduce(partial, n, amax, (hipStream_t)stream, num_cus()));
}

coat_status coat_quant_per_tensor(const uint16_t *x_bf16, int64_t n, const float *amax, uint8_t *codes,
                                  float *scale, void *stream) {
    if (!x_bf16 || !amax || !codes || !scale) return COAT_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(codes, 16) || !aligned(amax, 4) || !aligned(scale, 4))
        return COAT_ERR_ALIGN;
    if (n <= 0 || n % 8 != 0 || !fits_grid(n)) return COAT_ERR_SHAPE;
    return from_hip(coat::launch_quant_per_tensor(x_bf16, n, amax, codes, scale, (hipStream_t)stream,
                                                  num_cus()));
}

coat_status coat_quant_group(const uint16_t *x_bf16, int64_t rows, int64_t cols, int32_t group_size,
                             uint8_t *codes, float *scales, float *partial_amax_or_null, void *stream) {
    if (!x_bf16 || !codes || !scales) return COAT_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(codes, 16) || !aligned(scales, 4) ||
        (partial_amax_or_null && !aligned(partial_amax_or_null, 4)))
        return COAT_ERR_ALIGN;
    if (!valid_group(group_size)) return COAT_ERR_GROUP;
    if (rows <= 0 || cols <= 0 || cols % group_size != 0 || rows > INT64_MAX / cols || !fits_grid(rows * cols))
        return COAT_ERR_SHAPE;
    return from_hip(coat::launch_quant_group(x_bf16, rows * cols, group_size, codes, scales,
                                             partial_amax_or_null, (hipStream_t)stream, num_cus()));
}

coat_status coat_dequant_per_tensor(const uint8_t *codes, int64_t n, const float *scale, uint16_t *out_bf16,
                                    void *stream) {
    if (!codes || !scale || !out_bf16) return COAT_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(out_bf16, 16) || !aligned(scale, 4)) return COAT_ERR_ALIGN;
    if (n <= 0 || n % 8 != 0 || !fits_grid(n)) return COAT_ERR_SHAPE;
    return from_hip(coat::launch_dequant_per_tensor(codes, n, scale, out_bf16, (hipStream_t)stream));
}

coat_status coat_dequant_group(const uint8_t *codes, int64_t rows, int64_t cols, int32_t group_size,
                               const float *scales, uint16_t *out_bf16, void *stream) {
    if (!codes || !scales || !out_bf16) return COAT_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(out_bf16, 16) || !aligned(scales, 4)) return COAT_ERR_ALIGN;
    if (!valid_group(group_size)) return COAT_ERR_GROUP;
    if (rows <= 0 || cols <= 0 || cols % group_size != 0 || rows > INT64_MAX / cols || !fits_grid(rows * cols))
        return COAT_ERR_SHAPE;
    return from_hip(coat::launch_dequant_group(codes, rows * cols, group_size, scales, out_bf16,
                                               (hipStream_t)stream));
}

coat_status coat_swiglu_fused(const uint16_t *gate_bf16, const uint16_t *up_bf16, int64_t rows, int64_t cols,
                              int32_t group_size, uint16_t *h_bf16, float *h_partial_amax, uint8_t *gate_codes,
                              float *gate_scales, uint8_t *up_codes, float *up_scales, void *stream) {
    if (!gate_bf16 || !up_bf16 || !h_bf16 || !h_partial_amax) return COAT_ERR_NULL;
    const int saved = !!gate_codes + !!gate_scales + !!up_codes + !!up_scales;
    if (saved != 0 && saved != 4) return COAT_ERR_NULL;
    if (!aligned(gate_bf16, 16) || !aligned(up_bf16, 16) || !aligned(h_bf16, 16) || !aligned(h_partial_amax, 4) ||
        (saved && (!aligned(gate_codes, 16) || !aligned(up_codes, 16) || !aligned(gate_scales, 4) ||
                   !aligned(up_scales, 4))))
        return COAT_ERR_ALIGN;
    if (!valid_group(group_size)) return COAT_ERR_GROUP;
    if (rows <= 0 || cols <= 0 || cols % group_size != 0 || rows > INT64_MAX / cols || !fits_grid(rows * cols))
        return COAT_ERR_SHAPE;
    return from_hip(coat::launch_swiglu_fused(gate_bf16, up_bf16, rows * cols, group_size, h_bf16, h_partial_amax,
                                              gate_codes, gate_scales, up_codes, up_scales, (hipStream_t)stream));
}

coat_status coat_rmsnorm_fused(const uint16_t *x_bf16, const uint16_t *weight_bf16, int64_t rows, int64_t cols,
                               float eps, int32_t group_size, uint16_t *y_bf16, float *y_partial_amax, float *rstd,
                               uint8_t *x_codes, float *x_scales, void *stream) {
    if (!x_bf16 || !y_bf16 || !y_partial_amax) return COAT_ERR_NULL;
    if (!x_codes != !x_scales) return COAT_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(y_bf16, 16) || !aligned(y_partial_amax, 4) ||
        (weight_bf16 && !aligned(weight_bf16, 16)) || (rstd && !aligned(rstd, 4)) ||
        (x_codes && (!aligned(x_codes, 16) || !aligned(x_scales, 4))))
        return COAT_ERR_ALIGN;
    if (!valid_group(group_size)) return COAT_ERR_GROUP;
    if (rows <= 0 || cols <= 0 || cols % group_size != 0 || cols > coat::kRmsNormMaxCols ||
        rows > (int64_t)0x7FFFFFFF * (coat::kBlock / 64))
        return COAT_ERR_SHAPE;
    if (!(eps > 0.0f) || !(eps < INFINITY)) return COAT_ERR_HPARAM;
    return from_hip(coat::launch_rmsnorm_fused(x_bf16, weight_bf16, rows, (int)cols, group_size, eps, y_bf16,
                                               y_partial_amax, rstd, x_codes, x_scales, (hipStream_t)stream));
}

int64_t coat_adamw_list_bytes(int32_t n_tensors) {
    if (n_tensors <= 0) return 0;
    return (int64_t)sizeof(ListHeader) + list_starts_bytes(n_tensors) + (int64_t)sizeof(coat::StepBufs) * n_tensors;
}

coat_status coat_adamw_list_pack(const coat_adamw_tensor *tensors, int32_t n_tensors, int32_t group_size,
                                 void *table_host) {
    if (!tensors || !table_host) return COAT_ERR_NULL;
    if (n_tensors <= 0) return COAT_ERR_SHAPE;
    if (!valid_group(group_size)) return COAT_ERR_GROUP;
    int64_t chunks = 0;
    const bool bf16 = tensors[0].param_bf16 != nullptr;
    for (int32_t t = 0; t < n_tensors; ++t) {
        const coat_status s = check_bufs(to_bufs(tensors[t]), group_size);
        if (s != COAT_OK) return s;
        if ((tensors[t].param_bf16 != nullptr) != bf16) return COAT_ERR_NULL;
        chunks += coat::ceil_div(tensors[t].n, coat::kWaveElems);
        if (!fits_grid(chunks * coat::kWaveElems)) return COAT_ERR_SHAPE;
    }
    unsigned char *out = static_cast<unsigned char *>(table_host);
    unsigned char *starts = out + sizeof(ListHeader);
    unsigned char *entries = starts + list_starts_bytes(n_tensors);
    int64_t c = 0;
    for (int32_t t = 0; t < n_tensors; ++t) {
        const coat::StepBufs b = to_bufs(tensors[t]);
        memcpy(starts + 8 * t, &c, sizeof c);
        memcpy(entries + sizeof b * t, &b, sizeof b);
        c += coat::ceil_div(b.n, coat::kWaveElems);
    }
    memcpy(starts + 8 * (int64_t)n_tensors, &c, sizeof c);
    const ListHeader h{kListMagic, kListVersion, n_tensors, group_size, bf16 ? 1 : 0, 0, c};
    memcpy(out, &h, sizeof h);
    return COAT_OK;
}

coat_status coat_adamw_step_list(const void *table_host, const void *table_device, coat_fp8_format v_format,
                                 const coat_adamw_hparams *hp, void *stream) {
    if (!table_host || !table_device || !hp) return COAT_ERR_NULL;
    if (!aligned(table_device, 16)) return COAT_ERR_ALIGN;
    ListHeader h;
    memcpy(&h, table_host, sizeof h);
    if (h.magic != kListMagic || h.version != kListVersion || h.n_tensors <= 0 || h.total_chunks <= 0)
        return COAT_ERR_SHAPE;
    if (!valid_group(h.group_size)) return COAT_ERR_GROUP;
    if (v_format != COAT_FP8_E4M3 && v_format != COAT_FP8_E5M2) return COAT_ERR_FORMAT;
    if (!valid_hparams(hp)) return COAT_ERR_HPARAM;
    const unsigned char *dev = static_cast<const unsigned char *>(table_device);
    coat::StepListArgs a;
    a.chunk_start = reinterpret_cast<const int64_t *>(dev + sizeof(ListHeader));
    a.entries = reinterpret_cast<const coat::StepBufs *>(dev + sizeof(ListHeader) + list_starts_bytes(h.n_tensors));
    a.total_chunks = h.total_chunks;
    a.n_tensors = h.n_tensors;
    a.has_bf16 = h.has_bf16;
    make_params(hp, v_format, a.p);
    return from_hip(coat::launch_adamw_fp8_step_list(a, h.group_size, (int)v_format, (hipStream_t)stream));
}

}  // extern "C"

// ---- the tensor-list step without allocation ------------------------------
//
// coat_adamw_step_list reads its packed table from device memory the caller
// owns.  The variant below keeps that table in `scratch`, a file-scope device
// array that every GPU the library runs on holds until the process ends; the
// call copies the host table into it on the caller's stream and launches the
// same kernel on it, so it allocates nothing.  Host code never passes the
// array's name itself (on the host that is only a stand-in for the symbol):
// its address on each device comes from hipGetSymbolAddress, taken once per
// device with that device current.

namespace {

constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[COAT_LIST_NOALLOC_MAX_BYTES];

// The current device's address of `scratch` (nullptr if it cannot be had).
void *scratch_on_current_device() {
    static std::atomic<void *> addr[kMaxDevices];
    static std::mutex lock;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> g(lock);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        addr[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace

extern "C" {

coat_status coat_adamw_step_list_noalloc(const void *table_host, coat_fp8_format v_format,
                                         const coat_adamw_hparams *hp, void *stream) {
    if (!table_host || !hp) return COAT_ERR_NULL;
    ListHeader h;
    memcpy(&h, table_host, sizeof h);
    if (h.magic != kListMagic || h.version != kListVersion || h.n_tensors <= 0 || h.total_chunks <= 0)
        return COAT_ERR_SHAPE;
    if (!valid_group(h.group_size)) return COAT_ERR_GROUP;
    if (v_format != COAT_FP8_E4M3 && v_format != COAT_FP8_E5M2) return COAT_ERR_FORMAT;
    if (!valid_hparams(hp)) return COAT_ERR_HPARAM;
    const int64_t bytes = coat_adamw_list_bytes(h.n_tensors);
    if (bytes <= 0 || bytes > (int64_t)COAT_LIST_NOALLOC_MAX_BYTES) return COAT_ERR_SCRATCH;
    unsigned char *dev = static_cast<unsigned char *>(scratch_on_current_device());
    if (!dev) return COAT_ERR_HIP;
    if (hipMemcpyAsync(dev, table_host, (size_t)bytes, hipMemcpyHostToDevice, (hipStream_t)stream) != hipSuccess)
        return COAT_ERR_HIP;
    coat::StepListArgs a;
    a.chunk_start = reinterpret_cast<const int64_t *>(dev + sizeof(ListHeader));
    a.entries = reinterpret_cast<const coat::StepBufs *>(dev + sizeof(ListHeader) + list_starts_bytes(h.n_tensors));
    a.total_chunks = h.total_chunks;
    a.n_tensors = h.n_tensors;
    a.has_bf16 = h.has_bf16;
    make_params(hp, v_format, a.p);
    return from_hip(coat::launch_adamw_fp8_step_list(a, h.group_size, (int)v_format, (hipStream_t)stream));
}

}  // extern "C"
