// dequant.hip -- E4M3 activations back to BF16 for the backward pass, gfx950.
//
// The consumer half of activation compression ("COAT: compressing optimizer
// states and activations for memory-efficient FP8 training" explainer,
// blog.daoxuan.cc/posts/57954, sections "why activations are hard" and
// "mixed granularity"): activations saved in FP8 for the backward pass are
// read back there.  Per element y = FP32(decode(code) * scale), then BF16
// (round to nearest even).  The FP32 product is exact-then-rounded
// (v_mul_f32), the decode and the BF16 rounding are the native
// v_cvt_pk_f32_fp8 and v_cvt_pk_bf16_f32.  Each lane turns 16 codes (one
// 16-byte load) into 16 BF16 values (two 16-byte stores); one 1024-element
// chunk per wave.
#include "device.hpp"
#include "kernels.hpp"

namespace coat {
namespace {

// 16 codes (4 dwords) times one scale, to 8 dwords of packed BF16.
__device__ __forceinline__ void dequant16(const uint32_t c[4], float scale, uint32_t out[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const v2f lo = decode2_e4m3<false>(c[j]), hi = decode2_e4m3<true>(c[j]);
        out[2 * j] = bf16x2(lo.x * scale, lo.y * scale);
        out[2 * j + 1] = bf16x2(hi.x * scale, hi.y * scale);
    }
}

// A wave issues its code loads before it reads the scale, so the scalar's
// latency overlaps the loads'.
__global__ __launch_bounds__(kBlock) void dequant_per_tensor_kernel(const uint8_t *__restrict__ codes, int64_t n,
                                                                    int64_t n_chunks,
                                                                    const float *__restrict__ scale_p,
                                                                    uint16_t *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t chunk = xcd_block(blockIdx.x, gridDim.x) * (kBlock / 64) + (threadIdx.x >> 6);
    if (chunk >= n_chunks) return;
    const int64_t e0 = chunk * kWaveElems + lane * 16;
    if (e0 + 16 <= n) {
        const uint4 cv = *reinterpret_cast<const uint4 *>(codes + e0);
        const float scale = *scale_p;
        const uint32_t c[4] = {cv.x, cv.y, cv.z, cv.w};
        uint32_t o[8];
        dequant16(c, scale, o);
        uint4 *op = reinterpret_cast<uint4 *>(out + e0);
        op[0] = make_uint4(o[0], o[1], o[2], o[3]);
        op[1] = make_uint4(o[4], o[5], o[6], o[7]);
    } else if (e0 < n) {  // n % 16 == 8: the last lane holds 8 codes
        const uint2 cv = *reinterpret_cast<const uint2 *>(codes + e0);
        const float scale = *scale_p;
        const uint32_t c[4] = {cv.x, cv.y, 0u, 0u};
        uint32_t o[8];
        dequant16(c, scale, o);
        *reinterpret_cast<uint4 *>(out + e0) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

template <int G>
__global__ __launch_bounds__(kBlock) void dequant_group_kernel(const uint8_t *__restrict__ codes, int64_t n,
                                                               int64_t n_chunks, const float *__restrict__ scales,
                                                               uint16_t *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t chunk = xcd_block(blockIdx.x, gridDim.x) * (kBlock / 64) + (threadIdx.x >> 6);
    if (chunk >= n_chunks) return;
    const int64_t e0 = chunk * kWaveElems + lane * 16;
    if (e0 >= n) return;  // n % G == 0 and G >= 32: lanes are all in or all out
    const float scale = scales[e0 / G];
    const uint4 cv = *reinterpret_cast<const uint4 *>(codes + e0);
    const uint32_t c[4] = {cv.x, cv.y, cv.z, cv.w};
    uint32_t o[8];
    dequant16(c, scale, o);
    uint4 *op = reinterpret_cast<uint4 *>(out + e0);
    op[0] = make_uint4(o[0], o[1], o[2], o[3]);
    op[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

template <typename K, typename... Args>
hipError_t launch_k(K kernel, int64_t n_chunks, hipStream_t s, Args... args) {
    void *ptrs[] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)ceil_div(n_chunks, kBlock / 64)),
                           dim3(kBlock), ptrs, stream_lds_bytes(0), s);
}

}  // namespace

hipError_t launch_dequant_per_tensor(const uint8_t *codes, int64_t n, const float *scale, uint16_t *out,
                                     hipStream_t s) {
    const int64_t nc = ceil_div(n, kWaveElems);
    return launch_k(&dequant_per_tensor_kernel, nc, s, codes, n, nc, scale, out);
}

hipError_t launch_dequant_group(const uint8_t *codes, int64_t n, int G, const float *scales, uint16_t *out,
                                hipStream_t s) {
    const int64_t nc = ceil_div(n, kWaveElems);
    switch (G) {
    case 32: return launch_k(&dequant_group_kernel<32>, nc, s, codes, n, nc, scales, out);
    case 64: return launch_k(&dequant_group_kernel<64>, nc, s, codes, n, nc, scales, out);
    case 128: return launch_k(&dequant_group_kernel<128>, nc, s, codes, n, nc, scales, out);
    case 256: return launch_k(&dequant_group_kernel<256>, nc, s, codes, n, nc, scales, out);
    case 512: return launch_k(&dequant_group_kernel<512>, nc, s, codes, n, nc, scales, out);
    case 1024: return launch_k(&dequant_group_kernel<1024>, nc, s, codes, n, nc, scales, out);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace coat
