/*
 * Driver for the sanitizer build of the library's host layer (test
 * infrastructure; no GPU needed, no kernel is launched).
 *
 * tests/test_sanitize.py compiles the host code of the library with
 * AddressSanitizer and UndefinedBehaviorSanitizer (device code unchanged) and
 * links this driver against it. The driver takes every host-side path that
 * ends before a launch: the size, workspace, codebook and setup queries
 * (including sizes whose products overflow 64 bits), the descriptor check,
 * and the argument validation of every entry point, plus the empty-batch
 * no-ops. Stand-in device pointers point into one small heap buffer, so any
 * host read or write through them past its end stops the run. Each call's
 * status is compared with the one the header documents.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/qlora_amd.h"

static int g_fail = 0;

#define EXPECT(call, want)                                                          \
    do {                                                                            \
        const long long got_ = (long long)(call);                                   \
        if (got_ != (long long)(want)) {                                            \
            fprintf(stderr, "line %d: %s = %lld, expected %lld\n", __LINE__, #call, \
                    got_, (long long)(want));                                       \
            g_fail = 1;                                                             \
        }                                                                           \
    } while (0)

static unsigned char* g_fake; /* 4 KiB, 256-byte aligned: never read by a valid path */

static void* fake(size_t off) { return g_fake + off; }

static qlora_nf4 desc(int64_t N, int64_t K, int fmt) {
    qlora_nf4 d;
    memset(&d, 0, sizeof d);
    d.N = N;
    d.K = K;
    d.codes = (uint8_t*)fake(0);
    d.absmax_q = (int8_t*)fake(256);
    d.absmax_scale = (float*)fake(512);
    d.dq_format = fmt;
    d.format_version = QLORA_FORMAT_VERSION;
    d.setup_id = qlora_setup_id(fmt);
    d.reserved = 0;
    return d;
}

static void queries(void) {
    for (int s = -2; s <= 12; ++s) {
        const char* t = qlora_strerror(s);
        if (!t || !t[0]) g_fail = 1;
    }
    size_t a = 0, b = 0, c = 0;
    EXPECT(qlora_nf4_sizes(4096, 4096, &a, &b, &c), QLORA_OK);
    EXPECT(a, 4096u * 2048u);
    EXPECT(qlora_nf4_sizes(1, 96, &a, &b, &c), QLORA_ERR_SHAPE);
    EXPECT(qlora_nf4_sizes(0, 64, &a, &b, &c), QLORA_ERR_SHAPE);
    /* products past 64 bits are refused, not wrapped */
    EXPECT(qlora_nf4_sizes(INT64_MAX / 64 * 64, INT64_MAX / 64 * 64, &a, &b, &c) != QLORA_OK, 1);
    EXPECT(qlora_nf4_sizes((int64_t)1 << 40, (int64_t)1 << 40, &a, &b, &c) != QLORA_OK, 1);

    float lv[16], th[15], tq[15];
    EXPECT(qlora_codebook(lv, th), QLORA_OK);
    EXPECT(qlora_codebook_quotient_thresholds(tq), QLORA_OK);
    EXPECT(qlora_codebook_quotient_thresholds(NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_codebook_id() == qlora_setup_id(QLORA_DQ_INT8), 1);
    EXPECT(qlora_setup_id(3), 0);
    EXPECT(qlora_setup_id(-1), 0);

    const int64_t Ms[] = {0, 1, 16, 17, 511, 512, 4096, (int64_t)1 << 40, INT64_MAX};
    const int64_t NKs[][2] = {{4096, 4096}, {1, 64}, {28672, 8192}, {(int64_t)1 << 40, 1 << 20},
                              {INT64_MAX, 64}, {64, INT64_MAX / 64 * 64}};
    const int rs[] = {0, 16, 24, 64, 256, 272};
    for (int op = -1; op <= 5; ++op)
        for (size_t i = 0; i < sizeof Ms / sizeof Ms[0]; ++i)
            for (size_t j = 0; j < sizeof NKs / sizeof NKs[0]; ++j)
                for (size_t k = 0; k < sizeof rs / sizeof rs[0]; ++k)
                    (void)qlora_workspace_bytes(op, Ms[i], NKs[j][0], NKs[j][1], rs[k]);
    EXPECT(qlora_workspace_bytes(0, 16, 4096, 4000, 16), 0);
    EXPECT(qlora_workspace_bytes(0, (int64_t)1 << 40, (int64_t)1 << 40, 1 << 20, 16), 0);
}

static void descriptor(void) {
    qlora_nf4 d = desc(64, 128, QLORA_DQ_INT8);
    EXPECT(qlora_nf4_check(&d), QLORA_OK);
    EXPECT(qlora_nf4_check(NULL), QLORA_ERR_INVALID_ARG);
    d.codes = NULL;
    EXPECT(qlora_nf4_check(&d), QLORA_ERR_INVALID_ARG);
    d = desc(64, 96, QLORA_DQ_INT8);
    EXPECT(qlora_nf4_check(&d), QLORA_ERR_SHAPE);
    d = desc(64, 128, QLORA_DQ_INT8);
    d.absmax_scale = (float*)fake(516);
    EXPECT(qlora_nf4_check(&d), QLORA_ERR_ALIGN);
    d = desc(64, 128, QLORA_DQ_INT8);
    d.format_version = 2;
    EXPECT(qlora_nf4_check(&d), QLORA_ERR_SETUP);
    d = desc(64, 128, QLORA_DQ_E4M3);
    d.dq_format = QLORA_DQ_UINT8;
    EXPECT(qlora_nf4_check(&d), QLORA_ERR_SETUP);
    d = desc(64, 128, 7);
    EXPECT(qlora_nf4_check(&d), QLORA_ERR_INVALID_ARG);
    d = desc(64, 128, QLORA_DQ_INT8);
    d.reserved = 1;
    EXPECT(qlora_nf4_check(&d), QLORA_ERR_INVALID_ARG);
}

static void entry_points(void) {
    const uint16_t* x = fake(1024);
    const uint16_t* A = fake(1280);
    const uint16_t* B = fake(1536);
    void* y = fake(2048);
    void* ws = fake(3072);
    const size_t big = (size_t)1 << 40;
    qlora_nf4 d = desc(64, 128, QLORA_DQ_INT8);
    qlora_nf4 out;
    memset(&out, 0, sizeof out);
    out.codes = (uint8_t*)fake(0);
    out.absmax_q = (int8_t*)fake(256);
    out.absmax_scale = (float*)fake(512);

    /* quantize: every rejection leaves the descriptor untouched */
    EXPECT(qlora_quantize_nf4_dq(NULL, QLORA_DTYPE_BF16, 4, 64, 0, &out, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_quantize_nf4_dq(fake(0), QLORA_DTYPE_BF16, 4, 96, 0, &out, NULL), QLORA_ERR_SHAPE);
    EXPECT(qlora_quantize_nf4_dq(fake(0), 7, 4, 64, 0, &out, NULL), QLORA_ERR_DTYPE);
    EXPECT(qlora_quantize_nf4_dq(fake(2), QLORA_DTYPE_BF16, 4, 64, 0, &out, NULL), QLORA_ERR_ALIGN);
    EXPECT(qlora_quantize_nf4_dq(fake(0), QLORA_DTYPE_BF16, 4, 64, 3, &out, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_quantize_nf4_dq(fake(0), QLORA_DTYPE_BF16, (int64_t)1 << 40, (int64_t)1 << 40, 0, &out,
                                 NULL) != QLORA_OK, 1);
    EXPECT(out.N == 0 && out.format_version == 0 && out.setup_id == 0, 1);

    /* dequant */
    EXPECT(qlora_dequant_bf16(&d, NULL, 0, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_dequant_bf16(&d, fake(2), 0, NULL), QLORA_ERR_ALIGN);
    EXPECT(qlora_dequant_bf16(&d, fake(0), 2, NULL), QLORA_ERR_INVALID_ARG);
    qlora_nf4 huge = desc((int64_t)1 << 22, (int64_t)1 << 16, QLORA_DQ_INT8);
    EXPECT(qlora_dequant_bf16(&huge, fake(0), QLORA_LAYOUT_KSLAB32, NULL), QLORA_ERR_SHAPE);

    /* forward */
    EXPECT(qlora_linear_fwd(&d, NULL, 32, A, B, 16, 32.f, y, 0, NULL, ws, big, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_linear_fwd(&d, x, -1, A, B, 16, 32.f, y, 0, NULL, ws, big, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_linear_fwd(&d, x, 32, A, B, 16, 32.f, y, 5, NULL, ws, big, NULL), QLORA_ERR_DTYPE);
    EXPECT(qlora_linear_fwd(&d, x, 32, A, B, 24, 32.f, y, 0, NULL, ws, big, NULL), QLORA_ERR_RANK);
    EXPECT(qlora_linear_fwd(&d, x, 32, A, fake(1544), 16, 32.f, y, 0, NULL, ws, big, NULL), QLORA_ERR_ALIGN);
    EXPECT(qlora_linear_fwd(&d, x, 32, A, B, 16, 32.f, y, 0, NULL, ws, 16, NULL), QLORA_ERR_WORKSPACE);
    EXPECT(qlora_linear_fwd(&d, x, INT64_MAX, A, B, 16, 32.f, y, 0, NULL, ws, big, NULL) != QLORA_OK, 1);
    EXPECT(qlora_linear_fwd(&d, x, 0, A, B, 16, 32.f, y, 0, NULL, ws, big, NULL), QLORA_OK);
    EXPECT(qlora_linear_fwd(NULL, x, 32, A, B, 16, 32.f, y, 0, NULL, ws, big, NULL), QLORA_ERR_INVALID_ARG);

    /* the allocation-free forward */
    EXPECT(qlora_linear_fwd_noalloc(&d, x, (int64_t)1 << 30, A, B, 16, 32.f, y, 0, NULL, NULL),
           QLORA_ERR_TOO_LARGE);
    EXPECT(qlora_linear_fwd_noalloc(&d, x, 0, A, B, 16, 32.f, y, 0, NULL, NULL), QLORA_OK);
    EXPECT(qlora_linear_fwd_noalloc(&d, x, 32, A, B, 8, 32.f, y, 0, NULL, NULL), QLORA_ERR_RANK);
    EXPECT(qlora_linear_fwd_noalloc(&d, x, -3, A, B, 16, 32.f, y, 0, NULL, NULL), QLORA_ERR_INVALID_ARG);

    /* backward */
    const uint16_t* dY = fake(1792);
    EXPECT(qlora_linear_bwd(&d, x, NULL, 32, A, B, 16, 32.f, NULL, y, 0, y, y, 0, ws, big, NULL),
           QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_linear_bwd(&d, NULL, dY, 32, A, B, 16, 32.f, NULL, y, 0, y, y, 0, ws, big, NULL),
           QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_linear_bwd(&d, x, dY, 32, A, B, 16, 32.f, NULL, y, 3, y, y, 0, ws, big, NULL),
           QLORA_ERR_DTYPE);
    EXPECT(qlora_linear_bwd(&d, x, dY, 32, A, B, 0, 32.f, NULL, y, 0, y, y, 0, ws, big, NULL),
           QLORA_ERR_RANK);
    EXPECT(qlora_linear_bwd(&d, x, dY, 32, A, B, 16, 32.f, NULL, y, 0, y, y, 0, ws, 64, NULL),
           QLORA_ERR_WORKSPACE);
    EXPECT(qlora_linear_bwd(&d, x, dY, INT64_MAX, A, B, 16, 32.f, NULL, y, 0, y, y, 0, ws, big, NULL)
               != QLORA_OK, 1);

    /* merge */
    EXPECT(qlora_merge_lora(&d, NULL, 64, 100, A, B, 16, 32.f, y, ws, big, NULL), QLORA_ERR_SHAPE);
    EXPECT(qlora_merge_lora(NULL, NULL, 64, 128, A, B, 16, 32.f, y, ws, big, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_merge_lora(&d, NULL, 32, 128, A, B, 16, 32.f, y, ws, big, NULL), QLORA_ERR_SHAPE);
    EXPECT(qlora_merge_lora(&d, NULL, 64, 128, A, B, 16, 32.f, y, ws, 64, NULL), QLORA_ERR_WORKSPACE);

    /* dense stage */
    EXPECT(qlora_gemm_bf16_nt(x, 64, A, 64, 0, y, B, -1, 128, 64, 16, y, 0, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_gemm_bf16_nt(x, 64, A, 64, 0, y, B, 8, 128, 48, 16, y, 0, NULL), QLORA_ERR_SHAPE);
    EXPECT(qlora_gemm_bf16_nt(x, (int64_t)1 << 22, A, 64, 0, y, B, 8, 128, 64, 16, y, 0, NULL),
           QLORA_ERR_SHAPE);
    EXPECT(qlora_gemm_bf16_nt(x, 64, A, 64, 0, y, B, 0, 128, 64, 16, y, 0, NULL), QLORA_OK);

    /* optimizer step */
    float* p = fake(0);
    EXPECT(qlora_adamw_step(p, fake(256), 1, fake(512), fake(768), NULL, -1, 1e-4, 0.9, 0.999, 1e-8,
                            0.0, 1, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_adamw_step(p, fake(256), 1, fake(512), fake(768), NULL, 1000, 1e-4, 0.9, 0.999, 1e-8,
                            0.0, 0, NULL), QLORA_ERR_INVALID_ARG);
    EXPECT(qlora_adamw_step(p, fake(256), 7, fake(512), fake(768), NULL, 1000, 1e-4, 0.9, 0.999, 1e-8,
                            0.0, 1, NULL), QLORA_ERR_DTYPE);
    EXPECT(qlora_adamw_step(p, fake(256), 1, fake(512), fake(768), NULL, 0, 1e-4, 0.9, 0.999, 1e-8,
                            0.0, 1, NULL), QLORA_OK);
}

int main(void) {
    g_fake = aligned_alloc(256, 4096);
    if (!g_fake) return 3;
    memset(g_fake, 0, 4096);
    queries();
    descriptor();
    entry_points();
    free(g_fake);
    if (g_fail) return 1;
    printf("host sanitize driver: every status as documented\n");
    return 0;
}
