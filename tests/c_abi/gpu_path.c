/* gpu_path.c -- the hot path driven from plain C through the C ABI alone:
 * device buffers from hipMalloc, a stream from hipStreamCreate, no Python.
 * It runs one fused FP8-state AdamW step (coat_adamw_step) on 32768
 * parameters and the Group Scaling path (coat_group_absmax ->
 * coat_quant_per_tensor, and coat_quant_group) on a [64 x 1024] BF16 tensor,
 * then writes its inputs and every result to a file that the test suite
 * checks against the oracle.
 *
 * The HIP runtime entry points are taken with dlsym from the library that
 * libcoat.so itself loads, so this file needs no HIP header.
 *
 * Usage: gpu_path <libcoat.so> <output file>; exit status 0 when every call
 * returned success.  Output: the arrays below, in order, raw little-endian. */
#include <dlfcn.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/coat.h"

#define N_PARAM 32768
#define GROUP 128
#define ROWS 64
#define COLS 1024
#define N_ACT (ROWS * COLS)

#define LOAD(lib, name, var)                    \
    do {                                        \
        void *sym_ = dlsym(lib, #name);         \
        memcpy(&(var), &sym_, sizeof(var));     \
        if (!sym_) {                            \
            fprintf(stderr, "missing %s\n", #name); \
            return 2;                           \
        }                                       \
    } while (0)

typedef int (*hip_malloc_fn)(void **, size_t);
typedef int (*hip_free_fn)(void *);
typedef int (*hip_memcpy_fn)(void *, const void *, size_t, int);
typedef int (*hip_stream_create_fn)(void **);
typedef int (*hip_stream_sync_fn)(void *);
typedef int (*hip_stream_destroy_fn)(void *);
enum { H2D = 1, D2H = 2 }; /* hipMemcpyHostToDevice, hipMemcpyDeviceToHost */

typedef coat_status (*step_fn)(float *, const uint16_t *, uint8_t *, float *, float *, uint8_t *, float *,
                               float *, int64_t, int32_t, coat_fp8_format, const coat_adamw_hparams *, void *);
typedef coat_status (*absmax_fn)(const uint16_t *, int64_t, int64_t, int32_t, float *, float *, void *);
typedef coat_status (*qpt_fn)(const uint16_t *, int64_t, const float *, uint8_t *, float *, void *);
typedef coat_status (*qg_fn)(const uint16_t *, int64_t, int64_t, int32_t, uint8_t *, float *, float *, void *);
typedef const char *(*sstr_fn)(coat_status);

/* xorshift64*: the inputs are written out with the results, so any
 * generator will do. */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}

/* FP32 -> BF16 bit pattern, round to nearest even (finite inputs). */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static float theta0[N_PARAM], theta1[N_PARAM];
static uint16_t grad[N_PARAM];
static uint8_t m_codes[N_PARAM], v_codes[N_PARAM];
static float m_amax[N_PARAM / GROUP], m_k[N_PARAM / GROUP], v_amax[N_PARAM / GROUP], v_k[N_PARAM / GROUP];
static uint16_t x[N_ACT];
static float partial[N_ACT / GROUP], amax[1], scale[1], gscales[N_ACT / GROUP];
static uint8_t codes[N_ACT], gcodes[N_ACT];

int main(int argc, char **argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s libcoat.so out.bin\n", argv[0]);
        return 2;
    }
    void *lib = dlopen(argv[1], RTLD_NOW | RTLD_LOCAL);
    void *hip = dlopen("libamdhip64.so.7", RTLD_NOW | RTLD_LOCAL);
    if (!lib || !hip) {
        fprintf(stderr, "dlopen: %s\n", dlerror());
        return 2;
    }
    hip_malloc_fn hmalloc;
    hip_free_fn hfree;
    hip_memcpy_fn hmemcpy;
    hip_stream_create_fn hscreate;
    hip_stream_sync_fn hssync;
    hip_stream_destroy_fn hsdestroy;
    step_fn step;
    absmax_fn absmax;
    qpt_fn qpt;
    qg_fn qg;
    sstr_fn sstr;
    LOAD(hip, hipMalloc, hmalloc);
    LOAD(hip, hipFree, hfree);
    LOAD(hip, hipMemcpy, hmemcpy);
    LOAD(hip, hipStreamCreate, hscreate);
    LOAD(hip, hipStreamSynchronize, hssync);
    LOAD(hip, hipStreamDestroy, hsdestroy);
    LOAD(lib, coat_adamw_step, step);
    LOAD(lib, coat_group_absmax, absmax);
    LOAD(lib, coat_quant_per_tensor, qpt);
    LOAD(lib, coat_quant_group, qg);
    LOAD(lib, coat_status_string, sstr);

    /* inputs: theta ~ U(-0.05, 0.05); |g| log-uniform over four decades with
     * a random sign; x ~ a sum of four uniforms with one channel x100 */
    for (int i = 0; i < N_PARAM; ++i) {
        theta0[i] = (float)(0.1 * uniform() - 0.05);
        double mag = 1e-5;
        for (double e = 4.0 * uniform(); e > 0.0; e -= 1.0) mag *= e >= 1.0 ? 10.0 : 1.0 + 9.0 * e;
        grad[i] = to_bf16((float)(uniform() < 0.5 ? -mag : mag));
    }
    for (int i = 0; i < N_ACT; ++i) {
        double s = uniform() + uniform() + uniform() + uniform() - 2.0;
        if (i % COLS == 7) s *= 100.0;
        x[i] = to_bf16((float)s);
    }

    void *stream = NULL;
    void *d_th, *d_g, *d_mc, *d_ma, *d_mk, *d_vc, *d_va, *d_vk, *d_x, *d_p, *d_a, *d_c, *d_s, *d_gc, *d_gs;
    const size_t ng = N_PARAM / GROUP, na = N_ACT / GROUP;
    int herr = hscreate(&stream);
    herr |= hmalloc(&d_th, sizeof theta0) | hmalloc(&d_g, sizeof grad);
    herr |= hmalloc(&d_mc, N_PARAM) | hmalloc(&d_vc, N_PARAM);
    herr |= hmalloc(&d_ma, 4 * ng) | hmalloc(&d_mk, 4 * ng) | hmalloc(&d_va, 4 * ng) | hmalloc(&d_vk, 4 * ng);
    herr |= hmalloc(&d_x, sizeof x) | hmalloc(&d_p, 4 * na) | hmalloc(&d_a, 4) | hmalloc(&d_c, N_ACT);
    herr |= hmalloc(&d_s, 4) | hmalloc(&d_gc, N_ACT) | hmalloc(&d_gs, 4 * na);
    if (herr) {
        fprintf(stderr, "hip allocation failed\n");
        return 1;
    }
    /* a never-updated state: codes 0, amax 0, k 1 */
    for (size_t g = 0; g < ng; ++g) {
        m_amax[g] = v_amax[g] = 0.0f;
        m_k[g] = v_k[g] = 1.0f;
    }
    herr |= hmemcpy(d_th, theta0, sizeof theta0, H2D) | hmemcpy(d_g, grad, sizeof grad, H2D);
    herr |= hmemcpy(d_mc, m_codes, N_PARAM, H2D) | hmemcpy(d_vc, v_codes, N_PARAM, H2D);
    herr |= hmemcpy(d_ma, m_amax, 4 * ng, H2D) | hmemcpy(d_mk, m_k, 4 * ng, H2D);
    herr |= hmemcpy(d_va, v_amax, 4 * ng, H2D) | hmemcpy(d_vk, v_k, 4 * ng, H2D);
    herr |= hmemcpy(d_x, x, sizeof x, H2D);

    const coat_adamw_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.1f, 1};
    coat_status st[4];
    st[0] = step((float *)d_th, (const uint16_t *)d_g, (uint8_t *)d_mc, (float *)d_ma, (float *)d_mk,
                 (uint8_t *)d_vc, (float *)d_va, (float *)d_vk, N_PARAM, GROUP, COAT_FP8_E4M3, &hp, stream);
    st[1] = absmax((const uint16_t *)d_x, ROWS, COLS, GROUP, (float *)d_p, (float *)d_a, stream);
    st[2] = qpt((const uint16_t *)d_x, N_ACT, (const float *)d_a, (uint8_t *)d_c, (float *)d_s, stream);
    st[3] = qg((const uint16_t *)d_x, ROWS, COLS, GROUP, (uint8_t *)d_gc, (float *)d_gs, NULL, stream);
    for (int i = 0; i < 4; ++i)
        if (st[i] != COAT_OK) {
            fprintf(stderr, "call %d: %s\n", i, sstr(st[i]));
            return 1;
        }
    herr |= hssync(stream);
    herr |= hmemcpy(theta1, d_th, sizeof theta1, D2H);
    herr |= hmemcpy(m_codes, d_mc, N_PARAM, D2H) | hmemcpy(v_codes, d_vc, N_PARAM, D2H);
    herr |= hmemcpy(m_amax, d_ma, 4 * ng, D2H) | hmemcpy(m_k, d_mk, 4 * ng, D2H);
    herr |= hmemcpy(v_amax, d_va, 4 * ng, D2H) | hmemcpy(v_k, d_vk, 4 * ng, D2H);
    herr |= hmemcpy(partial, d_p, 4 * na, D2H) | hmemcpy(amax, d_a, 4, D2H) | hmemcpy(codes, d_c, N_ACT, D2H);
    herr |= hmemcpy(scale, d_s, 4, D2H) | hmemcpy(gcodes, d_gc, N_ACT, D2H) | hmemcpy(gscales, d_gs, 4 * na, D2H);
    void *bufs[] = {d_th, d_g, d_mc, d_ma, d_mk, d_vc, d_va, d_vk, d_x, d_p, d_a, d_c, d_s, d_gc, d_gs};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) herr |= hfree(bufs[i]);
    herr |= hsdestroy(stream);
    if (herr) {
        fprintf(stderr, "a HIP runtime call failed\n");
        return 1;
    }

    FILE *f = fopen(argv[2], "wb");
    if (!f) return 1;
    const void *out[] = {theta0, grad, theta1, m_codes, m_amax, m_k, v_codes, v_amax, v_k,
                         x, partial, amax, codes, scale, gcodes, gscales};
    const size_t len[] = {sizeof theta0, sizeof grad, sizeof theta1, sizeof m_codes, sizeof m_amax, sizeof m_k,
                          sizeof v_codes, sizeof v_amax, sizeof v_k, sizeof x, sizeof partial, sizeof amax,
                          sizeof codes, sizeof scale, sizeof gcodes, sizeof gscales};
    for (size_t i = 0; i < sizeof out / sizeof out[0]; ++i)
        if (fwrite(out[i], 1, len[i], f) != len[i]) return 1;
    return fclose(f) == 0 ? 0 : 1;
}
