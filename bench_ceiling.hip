// bench_ceiling.hip -- memory-only reference kernels that bench.py times beside
// the fused FP8-state AdamW step, to report what this device's HBM delivers
// for the step's own traffic.  Measurement tooling, not part of the library:
// bench.py builds it into _build/libbench_ceiling.so.
//
// step_skeleton moves exactly the bytes of the step (14 + 32/G B per
// parameter at G = 128) with the step's launch shape -- one 1024-parameter
// chunk per wave, 256-thread workgroups in the same XCD-aware order (each XCD
// sweeping its own eighth of the launch), the same residency cap -- and lane
// layout (16 consecutive parameters: 64 B of FP32
// master weights, 32 B of BF16 gradient, 16 B of each FP8 moment, the group's
// (amax, k) of both moments), with a trivial dependence on every loaded byte
// in place of the arithmetic.  With meta = 0 it leaves out the per-group
// (amax, k) traffic.  copy_1r1w is a plain 16-byte-per-lane copy; copy_4r3w
// reads four equal streams and writes three.
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
// eight XCDs round-robin (workgroup b on XCD b % 8); XCD x sweeps logical
// workgroups [x per, (x + 1) per) in order, per = nb / 8 (blocks past 8 per
// keep their index).
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t nb) {
    const int64_t per = nb >> 3;
    return b < 8 * per ? (b & 7) * per + (b >> 3) : b;
}

template <bool kMeta>
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
    float s = __uint_as_float((g0.x ^ g1.w) & 0x007FFFFFu);
    float am = 0.0f, km = 0.0f, av = 0.0f, kv = 0.0f;
    if constexpr (kMeta) {
        am = a.m_amax[grp]; km = a.m_k[grp]; av = a.v_amax[grp]; kv = a.v_k[grp];
        s += am + km + av + kv;
    }
    t0.x += s; t1.y += s; t2.z += s; t3.w += s;
    m.x ^= g0.y; v.y ^= g1.z; m.z ^= g0.w; v.w ^= g1.x;
    tp[0] = t0; tp[1] = t1; tp[2] = t2; tp[3] = t3;
    mp[0] = m; vp[0] = v;
    if (kMeta && (lane & 7) == 0) {
        a.m_amax[grp] = am + 1.0f; a.m_k[grp] = km;
        a.v_amax[grp] = av + 1.0f; a.v_k[grp] = kv;
    }
}

__global__ __launch_bounds__(256) void copy_1r1w(const f4 *__restrict__ src, f4 *__restrict__ dst, int64_t nvec) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < nvec) dst[i] = src[i];
}

// Four read streams and three write streams of nvec 16-byte vectors each.
__global__ __launch_bounds__(256) void copy_4r3w(const f4 *__restrict__ r0, const f4 *__restrict__ r1,
                                                 const f4 *__restrict__ r2, const f4 *__restrict__ r3,
                                                 f4 *__restrict__ w0, f4 *__restrict__ w1, f4 *__restrict__ w2,
                                                 int64_t nvec) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nvec) return;
    const f4 a = r0[i], b = r1[i], c = r2[i], d = r3[i];
    w0[i] = a + d;
    w1[i] = b + d;
    w2[i] = c + d;
}

size_t cap_lds(int blocks_per_cu) {
    if (blocks_per_cu <= 0) return 0;
    int dev = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        per_cu <= 0)
        return 0;
    return (size_t)per_cu / (size_t)blocks_per_cu;  // this many workgroups fit exactly
}

}  // namespace

extern "C" {

// n: parameters, a multiple of 1024 (group size 128).  blocks_per_cu > 0 caps
// the workgroups resident per CU (by reserving LDS), as the step does; 0
// leaves residency to the hardware.  meta = 0 leaves out the (amax, k)
// traffic.  Returns a hipError_t.
int ceiling_step_skeleton(float *param, const uint16_t *grad, uint8_t *m_codes, float *m_amax, float *m_k,
                          uint8_t *v_codes, float *v_amax, float *v_k, int64_t n, int blocks_per_cu, int meta,
                          void *stream) {
    if (n <= 0 || n % 1024 != 0) return (int)hipErrorInvalidValue;
    SkelArgs a{param, reinterpret_cast<const uint32_t *>(grad), reinterpret_cast<uint32_t *>(m_codes),
               reinterpret_cast<uint32_t *>(v_codes), m_amax, m_k, v_amax, v_k, n / 1024};
    void *args[] = {&a};
    const void *k = meta ? reinterpret_cast<const void *>(&step_skeleton<true>)
                         : reinterpret_cast<const void *>(&step_skeleton<false>);
    return (int)hipLaunchKernel(k, dim3((unsigned)((a.n_chunks + 3) / 4)), dim3(256), args,
                                cap_lds(blocks_per_cu), (hipStream_t)stream);
}

// nbytes: a multiple of 16.
int ceiling_copy_1r1w(const void *src, void *dst, int64_t nbytes, void *stream) {
    if (nbytes <= 0 || nbytes % 16 != 0) return (int)hipErrorInvalidValue;
    const f4 *s = reinterpret_cast<const f4 *>(src);
    f4 *d = reinterpret_cast<f4 *>(dst);
    int64_t nvec = nbytes / 16;
    void *args[] = {&s, &d, &nvec};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&copy_1r1w), dim3((unsigned)((nvec + 255) / 256)),
                                dim3(256), args, 0, (hipStream_t)stream);
}

// Seven disjoint streams of nbytes each (a multiple of 16): four read, three written.
int ceiling_copy_4r3w(const void *r0, const void *r1, const void *r2, const void *r3, void *w0, void *w1, void *w2,
                      int64_t nbytes, void *stream) {
    if (nbytes <= 0 || nbytes % 16 != 0) return (int)hipErrorInvalidValue;
    const void *rs[4] = {r0, r1, r2, r3};
    void *ws[3] = {w0, w1, w2};
    int64_t nvec = nbytes / 16;
    void *args[] = {&rs[0], &rs[1], &rs[2], &rs[3], &ws[0], &ws[1], &ws[2], &nvec};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&copy_4r3w), dim3((unsigned)((nvec + 255) / 256)),
                                dim3(256), args, 0, (hipStream_t)stream);
}

}  // extern "C"
