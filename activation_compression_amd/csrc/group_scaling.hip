// group_scaling.hip -- COAT Group Scaling and activation FP8 casts for gfx950.
//
// Method: "COAT: compressing optimizer states and activations for
// memory-efficient FP8 training" explainer (blog.daoxuan.cc/posts/57954),
// section "mixed granularity": linear-layer inputs take one per-tensor E4M3
// scale, whose absmax is found in two stages (a max per 1xG slice, cached,
// then a max over that G-times-smaller tensor); nonlinear-layer inputs take
// one scale per 1xG slice along the channel axis.
//
// All kernels are HBM-streaming: each lane owns 16 consecutive BF16 values
// (two 16-byte loads) and writes 16 codes with one 16-byte store; each wave
// handles one 1024-element chunk.  |x| maxima
// are integer maxima of the BF16 bit patterns with the sign cleared (two per
// v_pk_max_u16), which is exact for every finite value, denormals included.
// A 1xG slice is G/16 adjacent lanes, reduced with DPP.
//
// Every cast evaluates y = FP32(448 x / a) exactly rounded: a is prescaled by
// a power of two into [1, 2) (exact), 448 x by the same power (exact: a BF16
// value times 7 * 2^j has at most 11 significant bits), and the quotient is
// the RN-reciprocal product plus one Markstein correction.  The code is then
// the round-to-nearest-even of y, clamped to +-448.
#include "cast.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace coat {
namespace {

// ---- stage 1: per-slice absmax; also clears the stage-2 target, which the
// stage-2 kernel (next on the same stream) max-reduces into.
template <int G>
__global__ __launch_bounds__(kBlock) void absmax_stage1_kernel(const uint16_t *__restrict__ x, int64_t n,
                                                               int64_t n_chunks, float *__restrict__ partial,
                                                               float *__restrict__ amax) {
    constexpr int LPG = G / 16;
    if (blockIdx.x == 0 && threadIdx.x == 0) *amax = 0.0f;
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);  // one chunk per wave
    if (chunk < n_chunks) {
        const int64_t e0 = chunk * kWaveElems + lane * 16;
        const bool act = e0 < n;
        uint32_t m = 0u;
        if (act) {
            uint32_t w[8];
            load16(x + e0, w);
            m = absmax16(w);
        }
        m = run_max<LPG>(m);
        if (act && (lane % LPG) == 0) partial[e0 / G] = __uint_as_float(m << 16);
    }
}

// ---- stage 2: max over the partial tensor.  Multi-workgroup; each
// workgroup folds its maximum into *amax with an atomic max on the bit
// pattern (order-independent and exact for non-negative floats).
__global__ __launch_bounds__(kBlock) void absmax_stage2_kernel(const float *__restrict__ partial, int64_t n,
                                                               float *__restrict__ amax) {
    __shared__ uint32_t red[kBlock / 64];
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    uint32_t acc[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};  // eight loads in flight per thread
    for (; i + 7 * stride < n; i += 8 * stride) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = max(acc[j], __float_as_uint(partial[i + j * stride]) & 0x7FFFFFFFu);
    }
    for (; i < n; i += stride) acc[0] = max(acc[0], __float_as_uint(partial[i]) & 0x7FFFFFFFu);
    uint32_t m = max(max(max(acc[0], acc[1]), max(acc[2], acc[3])), max(max(acc[4], acc[5]), max(acc[6], acc[7])));
    m = run_max<64>(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = red[0];
#pragma unroll
        for (int i = 1; i < kBlock / 64; ++i) b = max(b, red[i]);
        // Atomics on one address serialize in L2: skip those that cannot raise
        // the value.  The load may be stale, which only costs an atomic.
        unsigned int *dst = reinterpret_cast<unsigned int *>(amax);
        if (b > __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(dst, b);
    }
}

__global__ void zero_scalar_kernel(float *p) { *p = 0.0f; }

// ---- per-tensor cast with the device-resident tensor absmax.  A wave issues
// its input loads before it reads the absmax (which the stage-2 kernel before
// it has just written), so the scalar's latency overlaps the loads'.
__global__ __launch_bounds__(kBlock) void quant_per_tensor_kernel(const uint16_t *__restrict__ x, int64_t n,
                                                                  int64_t n_chunks, const float *__restrict__ amax,
                                                                  uint8_t *__restrict__ codes,
                                                                  float *__restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t chunk = xcd_block(blockIdx.x, gridDim.x) * (kBlock / 64) + (threadIdx.x >> 6);  // one chunk per wave
    const int64_t e0 = chunk * kWaveElems + lane * 16;
    const bool live = chunk < n_chunks;
    const bool full = live && e0 + 16 <= n;
    const bool tail = live && !full && e0 < n;  // n % 16 == 8: the last lane holds 8 values
    uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (full) {
        load16(x + e0, w);
    } else if (tail) {
        const uint4 a = reinterpret_cast<const uint4 *>(x + e0)[0];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    }
    const float A = *amax;
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale = A > 0.0f ? A / 448.0f : 1.0f;
    if (!(full || tail)) return;
    const uint4 c = cast16<true>(w, cast_q(A));
    if (full)
        *reinterpret_cast<uint4 *>(codes + e0) = c;
    else
        *reinterpret_cast<uint2 *>(codes + e0) = make_uint2(c.x, c.y);
}

// ---- 1xG group cast (+ optional stage-1 partials from the same pass).
template <int G>
__global__ __launch_bounds__(kBlock) void quant_group_kernel(const uint16_t *__restrict__ x, int64_t n,
                                                             int64_t n_chunks, uint8_t *__restrict__ codes,
                                                             float *__restrict__ scales,
                                                             float *__restrict__ partial) {
    constexpr int LPG = G / 16;
    const int lane = threadIdx.x & 63;
    const int64_t chunk = xcd_block(blockIdx.x, gridDim.x) * (kBlock / 64) + (threadIdx.x >> 6);  // one chunk per wave
    if (chunk < n_chunks) {
        const int64_t e0 = chunk * kWaveElems + lane * 16;
        const bool act = e0 < n;
        uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        if (act) load16(x + e0, w);
        const uint32_t mb = run_max<LPG>(absmax16(w));
        const float a = __uint_as_float(mb << 16);
        const CastQ q = cast_q(a);
        const uint4 c = cast16(w, q);
        if (act) {
            *reinterpret_cast<uint4 *>(codes + e0) = c;
            if ((lane % LPG) == 0) {
                const int64_t grp = e0 / G;
                scales[grp] = a > 0.0f ? a / 448.0f : 1.0f;
                if (partial) partial[grp] = a;
            }
        }
    }
}

template <typename K, typename... Args>
hipError_t launch_k(K kernel, dim3 grid, hipStream_t s, Args... args) {
    void *ptrs[] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, dim3(kBlock), ptrs, 0, s);
}

// One 1024-element chunk per wave.
template <auto Kernel>
dim3 chunk_grid(int64_t n_chunks, int /*num_cus*/) {
    return dim3((unsigned)ceil_div(n_chunks, kBlock / 64));
}

template <int G>
hipError_t launch_stage1(const uint16_t *x, int64_t n, int64_t nc, float *partial, float *amax, hipStream_t s,
                         int num_cus) {
    constexpr auto k = &absmax_stage1_kernel<G>;
    return launch_k(k, chunk_grid<k>(nc, num_cus), s, x, n, nc, partial, amax);
}

template <int G>
hipError_t launch_qg(const uint16_t *x, int64_t n, int64_t nc, uint8_t *codes, float *scales, float *partial,
                     hipStream_t s, int num_cus) {
    constexpr auto k = &quant_group_kernel<G>;
    return launch_k(k, chunk_grid<k>(nc, num_cus), s, x, n, nc, codes, scales, partial);
}

// About 32 partials per thread: few workgroups, so few atomics on the target.
hipError_t launch_stage2(const float *partial, int64_t n, float *amax, hipStream_t s, int num_cus) {
    constexpr auto k = &absmax_stage2_kernel;
    return launch_k(k, resident_grid<k>(ceil_div(n, (int64_t)kBlock * 32), num_cus), s, partial, n, amax);
}

}  // namespace

hipError_t launch_absmax_reduce(const float *partial, int64_t n, float *amax, hipStream_t s, int num_cus) {
    hipError_t e = launch_k(&zero_scalar_kernel, dim3(1), s, amax);
    if (e != hipSuccess) return e;
    return launch_stage2(partial, n, amax, s, num_cus);
}

hipError_t launch_group_absmax(const uint16_t *x, int64_t n, int G, float *partial, float *amax,
                               hipStream_t s, int num_cus) {
    const int64_t nc = ceil_div(n, kWaveElems);
    hipError_t e;
    switch (G) {
    case 32: e = launch_stage1<32>(x, n, nc, partial, amax, s, num_cus); break;
    case 64: e = launch_stage1<64>(x, n, nc, partial, amax, s, num_cus); break;
    case 128: e = launch_stage1<128>(x, n, nc, partial, amax, s, num_cus); break;
    case 256: e = launch_stage1<256>(x, n, nc, partial, amax, s, num_cus); break;
    case 512: e = launch_stage1<512>(x, n, nc, partial, amax, s, num_cus); break;
    case 1024: e = launch_stage1<1024>(x, n, nc, partial, amax, s, num_cus); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    return launch_stage2(partial, n / G, amax, s, num_cus);
}

hipError_t launch_quant_per_tensor(const uint16_t *x, int64_t n, const float *amax, uint8_t *codes,
                                   float *scale, hipStream_t s, int num_cus) {
    const int64_t nc = ceil_div(n, kWaveElems);
    constexpr auto k = &quant_per_tensor_kernel;
    return launch_k(k, chunk_grid<k>(nc, num_cus), s, x, n, nc, amax, codes, scale);
}

hipError_t launch_quant_group(const uint16_t *x, int64_t n, int G, uint8_t *codes, float *scales,
                              float *partial, hipStream_t s, int num_cus) {
    const int64_t nc = ceil_div(n, kWaveElems);
    switch (G) {
    case 32: return launch_qg<32>(x, n, nc, codes, scales, partial, s, num_cus);
    case 64: return launch_qg<64>(x, n, nc, codes, scales, partial, s, num_cus);
    case 128: return launch_qg<128>(x, n, nc, codes, scales, partial, s, num_cus);
    case 256: return launch_qg<256>(x, n, nc, codes, scales, partial, s, num_cus);
    case 512: return launch_qg<512>(x, n, nc, codes, scales, partial, s, num_cus);
    case 1024: return launch_qg<1024>(x, n, nc, codes, scales, partial, s, num_cus);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace coat
