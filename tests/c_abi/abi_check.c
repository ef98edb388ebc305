/* abi_check.c -- the C ABI consumed from plain C: include/coat.h compiles as
 * C99 and every entry point's host-side validation answers as documented.
 * No call here is valid, so nothing reaches a GPU; it runs on any host.
 * Usage: abi_check <path to libcoat.so>; exit status 0 when every check holds. */
#include <dlfcn.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/coat.h"

static int failures = 0;

#define CHECK(expr, want)                                                                  \
    do {                                                                                   \
        int got_ = (int)(expr);                                                            \
        if (got_ != (int)(want)) {                                                         \
            fprintf(stderr, "%s:%d: %s = %d, want %d\n", __FILE__, __LINE__, #expr, got_,  \
                    (int)(want));                                                          \
            ++failures;                                                                    \
        }                                                                                  \
    } while (0)

/* dlsym returns an object pointer; POSIX guarantees it converts to a
 * function pointer, ISO C does not, so the bits are copied. */
#define LOAD(lib, name, var)                    \
    do {                                        \
        void *sym_ = dlsym(lib, #name);         \
        memcpy(&(var), &sym_, sizeof(var));     \
    } while (0)

typedef coat_status (*coat_adamw_step_fn)(float *, const uint16_t *, uint8_t *, float *, float *, uint8_t *,
                                          float *, float *, int64_t, int32_t, coat_fp8_format,
                                          const coat_adamw_hparams *, void *);
typedef coat_status (*coat_group_absmax_fn)(const uint16_t *, int64_t, int64_t, int32_t, float *, float *, void *);
typedef coat_status (*coat_quant_per_tensor_fn)(const uint16_t *, int64_t, const float *, uint8_t *, float *,
                                                void *);
typedef coat_status (*coat_quant_group_fn)(const uint16_t *, int64_t, int64_t, int32_t, uint8_t *, float *,
                                           float *, void *);
typedef int64_t (*coat_adamw_list_bytes_fn)(int32_t);
typedef coat_status (*coat_adamw_list_pack_fn)(const coat_adamw_tensor *, int32_t, int32_t, void *);
typedef const char *(*coat_status_string_fn)(coat_status);

int main(int argc, char **argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s libcoat.so\n", argv[0]);
        return 2;
    }
    void *lib = dlopen(argv[1], RTLD_NOW | RTLD_LOCAL);
    if (!lib) {
        fprintf(stderr, "dlopen: %s\n", dlerror());
        return 2;
    }
    coat_adamw_step_fn step;
    coat_group_absmax_fn absmax;
    coat_quant_per_tensor_fn qpt;
    coat_quant_group_fn qg;
    coat_adamw_list_bytes_fn lbytes;
    coat_adamw_list_pack_fn lpack;
    coat_status_string_fn sstr;
    LOAD(lib, coat_adamw_step, step);
    LOAD(lib, coat_group_absmax, absmax);
    LOAD(lib, coat_quant_per_tensor, qpt);
    LOAD(lib, coat_quant_group, qg);
    LOAD(lib, coat_adamw_list_bytes, lbytes);
    LOAD(lib, coat_adamw_list_pack, lpack);
    LOAD(lib, coat_status_string, sstr);
    if (!step || !absmax || !qpt || !qg || !lbytes || !lpack || !sstr) {
        fprintf(stderr, "missing symbol\n");
        return 2;
    }

    /* aligned, never-dereferenced addresses */
    float *f = (float *)(uintptr_t)0x100000;
    uint8_t *u8 = (uint8_t *)(uintptr_t)0x200000;
    uint16_t *u16 = (uint16_t *)(uintptr_t)0x300000;
    coat_adamw_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.1f, 1};
    coat_adamw_hparams bad = hp;

    CHECK(step(NULL, u16, u8, f, f, u8, f, f, 1024, 128, COAT_FP8_E4M3, &hp, NULL), COAT_ERR_NULL);
    CHECK(step(f, u16, u8, f, f, u8, f, f, 1024, 128, COAT_FP8_E4M3, NULL, NULL), COAT_ERR_NULL);
    CHECK(step((float *)((char *)f + 4), u16, u8, f, f, u8, f, f, 1024, 128, COAT_FP8_E4M3, &hp, NULL),
          COAT_ERR_ALIGN);
    CHECK(step(f, u16, u8, f, f, u8, f, f, 1000, 128, COAT_FP8_E4M3, &hp, NULL), COAT_ERR_SHAPE);
    CHECK(step(f, u16, u8, f, f, u8, f, f, 1024, 100, COAT_FP8_E4M3, &hp, NULL), COAT_ERR_GROUP);
    CHECK(step(f, u16, u8, f, f, u8, f, f, 1024, 128, (coat_fp8_format)9, &hp, NULL), COAT_ERR_FORMAT);
    bad.beta2 = 1.0f;
    CHECK(step(f, u16, u8, f, f, u8, f, f, 1024, 128, COAT_FP8_E4M3, &bad, NULL), COAT_ERR_HPARAM);
    bad = hp;
    bad.step = 0;
    CHECK(step(f, u16, u8, f, f, u8, f, f, 1024, 128, COAT_FP8_E5M2, &bad, NULL), COAT_ERR_HPARAM);

    CHECK(absmax(u16, 16, 4096, 128, f, NULL, NULL), COAT_ERR_NULL);
    CHECK(absmax(u16, 16, 4000, 128, f, f, NULL), COAT_ERR_SHAPE);
    CHECK(qpt(u16, 12, f, u8, f, NULL), COAT_ERR_SHAPE);
    CHECK(qg(u16 + 1, 16, 4096, 128, u8, f, NULL, NULL), COAT_ERR_ALIGN);

    CHECK(lbytes(2), 32 + 32 + 2 * 80);
    {
        coat_adamw_tensor t[2];
        unsigned char table[32 + 32 + 2 * 80];
        memset(t, 0, sizeof t);
        t[0].param = f; t[0].grad_bf16 = u16; t[0].m_codes = u8; t[0].m_amax = f; t[0].m_k = f;
        t[0].v_codes = u8; t[0].v_amax = f; t[0].v_k = f; t[0].n = 2048;
        t[1] = t[0];
        t[1].n = 200;
        CHECK(lpack(t, 2, 128, table), COAT_ERR_SHAPE);
        t[1].n = 256;
        CHECK(lpack(t, 2, 128, table), COAT_OK);
    }
    if (strlen(sstr(COAT_ERR_SHAPE)) == 0) ++failures;

    dlclose(lib);
    if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
    return failures ? 1 : 0;
}
