// device.hpp -- gfx950 device primitives shared by the COAT kernels:
// format traits, native OCP FP8 conversions, wave64 group reductions and
// small exact-arithmetic helpers.  Header-only, device code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coat {

enum Fmt : int { kE4M3 = 0, kE5M2 = 1 };

// OCP FP8 formats ("LLM atlas -- systems / numerics", sections "01 Number
// anatomy" and "03 FP8"): E4M3 max 448, smallest subnormal 2^-9;
// E5M2 max 57344, smallest subnormal 2^-16.
template <int F> struct Fp8;
template <> struct Fp8<kE4M3> {
    static constexpr float kMax = 448.0f;
    static constexpr double kMinSub = 0x1p-9;
};
template <> struct Fp8<kE5M2> {
    static constexpr float kMax = 57344.0f;
    static constexpr double kMinSub = 0x1p-16;
};

typedef float v2f __attribute__((ext_vector_type(2)));

// ---- native FP8 conversions (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 and the
// reverse).  Rounding is to nearest even.  Callers pass values within a few
// ulps of +-MAX or below (clamped, or bounded by construction), which the
// rounding takes to at most MAX whatever the overflow mode.

// Pack four FP32 values into four FP8 codes (byte i <- value i).
template <int F>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    int w;
    if constexpr (F == kE4M3) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    }
    return (uint32_t)w;
}

// Decode code byte 0 of `c` to FP32.
template <int F>
__device__ __forceinline__ float decode1(uint32_t c) {
    if constexpr (F == kE4M3)
        return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
    else
        return __builtin_amdgcn_cvt_f32_bf8((int)c, 0);
}

// Two FP32 values to a packed pair of BF16 (round to nearest even, native
// v_cvt_pk_bf16_f32): a in the low half, b in the high half.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const v2f v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// Decode E4M3 code bytes 0,1 (kHi = false) or 2,3 (kHi = true) of w to FP32.
template <bool kHi>
__device__ __forceinline__ v2f decode2_e4m3(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
}

// ---- XCD-aware block order.  The dispatcher deals workgroups to the eight
// XCDs round-robin (workgroup b runs on XCD b % 8), so in launch order the
// XCDs interleave at single-workgroup granularity.  Streaming kernels remap
// the workgroup index so that each XCD sweeps runs of kXcdRun consecutive
// logical workgroups instead: XCD x takes logical blocks [s*8R + x*R,
// s*8R + (x+1)*R) of super-run s.  Blocks past the last whole super-run keep
// their index.  A bijection on [0, nblocks).  Measured on MI355X: a
// memory-only model of the optimizer step 5.19 -> 5.32 TB/s with R = 256
// (32 .. 8192 all gained, 256 most); the 1xG cast 4%, the dequantization 2%
// faster; SwiGLU unchanged.  The row-per-wave RMSNorm and the read-only
// stage-1 pass lost 1-7% and keep the launch order; the optimizer step takes
// xcd_eighth below.
constexpr int64_t kXcdRun = 256;

__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t nblocks) {
    constexpr int64_t W = 8 * kXcdRun;
    if (b >= nblocks / W * W) return b;
    const int64_t q = b >> 3;
    return (q / kXcdRun) * W + (b & 7) * kXcdRun + q % kXcdRun;
}

// The optimizer step's order: XCD x (= b % 8) sweeps its own contiguous
// eighth of the launch, logical blocks [x per, (x + 1) per) in order, per =
// nblocks / 8; blocks past 8 per keep their index.  A bijection on [0,
// nblocks).  At any moment the eight XCDs then stream eight regions of every
// array an eighth of the arena apart instead of one shared window.  Measured
// on the 7B-shaped arena over 25 buffer placements on three MI355X: faster in
// 22, by 0.65% on average (the runs of kXcdRun above: the reference).
__device__ __forceinline__ int64_t xcd_eighth(int64_t b, int64_t nblocks) {
    const int64_t per = nblocks >> 3;
    return b < 8 * per ? (b & 7) * per + (b >> 3) : b;
}

// ---- bit helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Magnitude of `mag` with the sign bit of `sgn` (one v_bfi_b32).
__device__ __forceinline__ float with_sign_of(float mag, float sgn) {
    return __uint_as_float((__float_as_uint(mag) & 0x7FFFFFFFu) | (__float_as_uint(sgn) & 0x80000000u));
}

// ---- wave64 reductions over aligned runs of W lanes (W a power of two <= 64).
// Every lane of a run receives the run's result.  Runs of up to 16 lanes stay
// inside a DPP row; 32 uses ds_swizzle, 64 ds_bpermute.

template <int W>
__device__ __forceinline__ uint32_t run_max(uint32_t v) {
    if constexpr (W >= 2) v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    if constexpr (W >= 4) v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    if constexpr (W >= 8) v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
    if constexpr (W >= 16) v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true)); // row_mirror
    if constexpr (W >= 32) v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));             // xor 16
    if constexpr (W >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

template <int W>
__device__ __forceinline__ uint32_t run_min(uint32_t v) {
    if constexpr (W >= 2) v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
    if constexpr (W >= 4) v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
    if constexpr (W >= 8) v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));
    if constexpr (W >= 16) v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));
    if constexpr (W >= 32) v = min(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
    if constexpr (W >= 64) v = min(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// Max of the packed |bf16| magnitudes of one dword pair-wise (v_pk_max_u16
// on the bit patterns with the sign bits cleared: for non-negative IEEE
// values the integer order is the numeric order, denormals included).
__device__ __forceinline__ uint32_t pk_absmax_u16(uint32_t acc, uint32_t w) {
    typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
    uint32_t a = w & 0x7FFF7FFFu;
    v2u16 x = __builtin_bit_cast(v2u16, acc), y = __builtin_bit_cast(v2u16, a);
    v2u16 r = __builtin_elementwise_max(x, y);
    return __builtin_bit_cast(uint32_t, r);
}

// Device memory seen as the global address space: the compiler then uses
// global rather than flat memory instructions for a pointer it cannot trace to
// a kernel argument (one read from a table in memory).  A flat load counts
// against the LDS counter as well, so an LDS-only wait would wait for it too.
template <class T> using gmem = __attribute__((address_space(1))) T;
template <class T> __device__ __forceinline__ gmem<T> *as_global(T *p) { return (gmem<T> *)p; }

// Correctly rounded quotient a / b from the correctly rounded reciprocal
// y = RN(1/b): one product and one FMA-based correction (Markstein's
// theorem; no overflow or underflow in the operands' range).
__device__ __forceinline__ float div_rn_from_rcp(float a, float b, float y) {
    float q = a * y;
    float r = __builtin_fmaf(-q, b, a);
    return __builtin_fmaf(r, y, q);
}

}  // namespace coat
