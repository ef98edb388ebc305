// ceiling.hip -- memory-only reference kernels for the benchmark's roofline
// context (built into libcoat_ceiling.so, separate from the product library).
//
// step_skeleton moves exactly the bytes of the fused FP8-state AdamW step, with
// the same launch shape (one 1024-parameter chunk per wave, 256-thread
// workgroups, the same XCD-aware workgroup order and residency cap) and the same per-lane layout (16 consecutive parameters: 64 B of
// FP32 master weights, 32 B of BF16 gradient, 16 B of each FP8 moment, the
// group's (amax, k) of both moments), but replaces the arithmetic with a
// trivial dependence on every loaded byte.  copy_stream is a plain 16-byte-
// per-lane copy.  Their GB/s are what this device's HBM delivers for the
// step's traffic pattern and for a single read + write stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

struct SkelArgs {
    float *param;
    const uint32_t *grad;  // BF16 pairs
    uint32_t *m_codes, *v_codes;
    float *m_amax, *m_k, *v_amax, *v_k;
    int64_t n_chunks;
};

// The step's XCD-aware workgroup order: the dispatcher deals workgroups to the
// eight XCDs round-robin; each XCD sweeps runs of 256 consecutive logical
// workgroups (blocks past the last whole run of 8 x 256 keep their index).
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t nb) {
    if (b >= nb / 2048 * 2048) return b;
    const int64_t q = b >> 3;
    return (q / 256) * 2048 + (b & 7) * 256 + q % 256;
}

__global__ __launch_bounds__(256) void step_skeleton(SkelArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t c = xcd_order(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
    if (c >= a.n_chunks) return;
    const int64_t base = c * 1024;
    f4 *tp = reinterpret_cast<f4 *>(a.param + base) + lane * 4;
    const u4 *gp = reinterpret_cast<const u4 *>(a.grad + base / 2) + lane * 2;
    u4 *mp = reinterpret_cast<u4 *>(a.m_codes + base / 4) + lane;
    u4 *vp = reinterpret_cast<u4 *>(a.v_codes + base / 4) + lane;
    f4 t0 = tp[0], t1 = tp[1], t2 = tp[2], t3 = tp[3];
    u4 g0 = gp[0], g1 = gp[1], m = mp[0], v = vp[0];
    const int64_t grp = (base + lane * 16) / 128;
    const float am = a.m_amax[grp], km = a.m_k[grp], av = a.v_amax[grp], kv = a.v_k[grp];
    const float s = __uint_as_float((g0.x ^ g1.w) & 0x007FFFFFu) + am + km + av + kv;
    t0.x += s; t1.y += s; t2.z += s; t3.w += s;
    m.x ^= g0.y; v.y ^= g1.z; m.z ^= g0.w; v.w ^= g1.x;
    tp[0] = t0; tp[1] = t1; tp[2] = t2; tp[3] = t3;
    mp[0] = m; vp[0] = v;
    if ((lane & 7) == 0) {
        a.m_amax[grp] = am + 1.0f; a.m_k[grp] = km;
        a.v_amax[grp] = av + 1.0f; a.v_k[grp] = kv;
    }
}

__global__ __launch_bounds__(64) void copy_stream(const f4 *__restrict__ src, f4 *__restrict__ dst, int64_t nvec) {
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (i < nvec) dst[i] = __builtin_nontemporal_load(src + i);
}

}  // namespace

extern "C" {

// n: parameters, a multiple of 1024 (group size 128).  blocks_per_cu > 0 caps
// the workgroups resident per CU (by reserving LDS), as the step does; 0
// leaves residency to the hardware.  Returns a hipError_t.
int coat_ceiling_step_skeleton(float *param, const uint16_t *grad, uint8_t *m_codes, float *m_amax, float *m_k,
                               uint8_t *v_codes, float *v_amax, float *v_k, int64_t n, int blocks_per_cu,
                               void *stream) {
    if (n <= 0 || n % 1024 != 0) return (int)hipErrorInvalidValue;
    size_t lds = 0;
    if (blocks_per_cu > 0) {
        int dev = 0, per_cu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
            per_cu > 0)
            lds = (size_t)per_cu / (size_t)blocks_per_cu;
    }
    SkelArgs a{param, reinterpret_cast<const uint32_t *>(grad), reinterpret_cast<uint32_t *>(m_codes),
               reinterpret_cast<uint32_t *>(v_codes), m_amax, m_k, v_amax, v_k, n / 1024};
    void *args[] = {&a};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&step_skeleton), dim3((unsigned)((a.n_chunks + 3) / 4)),
                                dim3(256), args, lds, (hipStream_t)stream);
}

// nbytes: a multiple of 16.
int coat_ceiling_copy(const void *src, void *dst, int64_t nbytes, void *stream) {
    if (nbytes <= 0 || nbytes % 16 != 0) return (int)hipErrorInvalidValue;
    const f4 *s = reinterpret_cast<const f4 *>(src);
    f4 *d = reinterpret_cast<f4 *>(dst);
    int64_t nvec = nbytes / 16;
    void *args[] = {&s, &d, &nvec};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&copy_stream), dim3((unsigned)((nvec + 63) / 64)),
                                dim3(64), args, 0, (hipStream_t)stream);
}

}  // extern "C"
