/* Validation and error paths of every liblact entry point, for a build of
 * the library's host code with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_abi_sanitizers.py).  No GPU is needed: every case returns
 * before any device work (valid argument sets stop at the device check).
 * Exit status 0 when every status code is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lact.h"

static int failures = 0, checks = 0;

#define EXPECT(call, code)                                                                     \
    do {                                                                                       \
        lact_status s_ = (call);                                                               \
        ++checks;                                                                              \
        if (s_ != (code)) {                                                                    \
            ++failures;                                                                        \
            fprintf(stderr, "line %d: %s -> %d, expected %d (%s)\n", __LINE__, #call, (int)s_, \
                    (int)(code), lact_last_error());                                           \
        }                                                                                      \
    } while (0)

/* an aligned address that validation never dereferences */
#define F ((void*)(uintptr_t)(1u << 20))
#define FF ((float*)(uintptr_t)(1u << 20))

static lact_problem prob(int d, int dh, int io, int opt) {
    lact_problem p;
    memset(&p, 0, sizeof(p));
    p.n_inst = 2;
    p.d = d;
    p.dh = dh;
    p.io_dtype = io;
    p.opt = opt;
    p.ns_iters = 5;
    return p;
}

static lact_status fwd(const lact_problem* p, int64_t L, int64_t chunk, int32_t order, const int64_t* b,
                       const uint8_t* f, int32_t nc, void* q, size_t ws) {
    return lact_layer_forward(p, q, F, F, FF, FF, L, chunk, order, b, f, nc, FF, FF, FF, FF, FF, FF, F, F, ws, NULL);
}

static lact_status bwd(const lact_problem* p, int64_t L, void* dq, float* dW1, const float* oz, float* doz,
                       size_t ws) {
    return lact_layer_backward(p, F, F, F, FF, FF, oz, L, 128, LACT_APPLY_THEN_UPDATE, NULL, NULL, 0, FF, FF, FF, FF,
                               FF, FF, F, FF, FF, FF, FF, FF, FF, (float*)dq, FF, FF, FF, FF, doz, dW1, FF, FF, FF, FF,
                               FF, F, ws, NULL);
}

int main(void) {
    const size_t BIG = (size_t)1 << 40;
    lact_problem p = prob(128, 128, LACT_DTYPE_BF16, LACT_OPT_MOMENTUM);
    const int ok_or_nodev = LACT_ERR_NO_DEVICE;   /* valid arguments on a machine without a GPU */

    /* status text */
    for (int s = -5; s <= 0; ++s) {
        ++checks;
        if (!lact_status_str((lact_status)s) || !lact_status_str((lact_status)s)[0]) ++failures;
    }

    /* problems */
    EXPECT(fwd(NULL, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    lact_problem b = p;
    b.d = 96;
    EXPECT(fwd(&b, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_UNSUPPORTED);
    b = p;
    b.dh = 2048;
    EXPECT(fwd(&b, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_UNSUPPORTED);
    b = p;
    b.io_dtype = 5;
    EXPECT(fwd(&b, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    b = p;
    b.opt = 9;
    EXPECT(fwd(&b, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    b = p;
    b.opt = LACT_OPT_MUON;
    b.ns_iters = 0;
    EXPECT(fwd(&b, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    b = p;
    b.rec_planes = 4;
    EXPECT(fwd(&b, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    b = p;
    b.n_inst = -1;
    EXPECT(fwd(&b, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    b = p;
    b.flags = 0x40;
    EXPECT(fwd(&b, 512, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);

    /* schedules */
    const int64_t b_dec[] = {0, 300, 200, 512}, b_bad0[] = {1, 100, 512}, b_ok[] = {0, 100, 512},
                  b_short[] = {0, 100, 500};
    const uint8_t f3[] = {3, 3, 3}, f2[] = {3, 3}, f_bad[] = {3, 4};
    EXPECT(fwd(&p, 512, 128, 2, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, 512, 0, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, -1, 128, 0, NULL, NULL, 0, F, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, 512, 0, 0, b_dec, f3, 3, F, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, 512, 0, 0, b_bad0, f2, 2, F, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, 512, 0, 0, b_short, f2, 2, F, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, 512, 0, 0, b_ok, f_bad, 2, F, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, 512, 0, 0, b_ok, NULL, 2, F, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, 512, 0, 0, b_ok, f2, 2, F, BIG), ok_or_nodev);

    /* pointers and workspace */
    EXPECT(fwd(&p, 512, 128, 0, NULL, NULL, 0, NULL, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(fwd(&p, 512, 128, 0, NULL, NULL, 0, (char*)F + 2, BIG), LACT_ERR_INVALID_ARG);
    const size_t need = lact_workspace_size(&p, 512, 128, 0, NULL, NULL, 0);
    ++checks;
    if (need == 0) ++failures;
    EXPECT(fwd(&p, 512, 128, 0, NULL, NULL, 0, F, need - 1), LACT_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(fwd(&p, 512, 128, 0, NULL, NULL, 0, F, need), ok_or_nodev);
    b = p;
    b.d = 96;
    ++checks;
    if (lact_workspace_size(&b, 512, 128, 0, NULL, NULL, 0) != 0) ++failures;

    /* the other forward entry points */
    EXPECT(lact_layer_forward_scaled(&p, F, F, F, FF, FF, NULL, 512, 128, 0, NULL, NULL, 0, FF, FF, FF, FF, FF, FF, F,
                                     F, BIG, NULL),
           LACT_ERR_INVALID_ARG);   /* oz missing with APPLY chunks */
    EXPECT(lact_layer_forward_scaled(&p, F, F, F, FF, FF, FF, 512, 128, 0, NULL, NULL, 0, FF, FF, FF, FF, FF, FF, F,
                                     F, BIG, NULL),
           ok_or_nodev);
    EXPECT(lact_chunk_update(&p, F, F, FF, FF, -1, 16, FF, FF, FF, FF, FF, FF, F, BIG, NULL), LACT_ERR_INVALID_ARG);
    EXPECT(lact_chunk_update(&p, F, F, FF, FF, 32, 16, FF, FF, FF, FF, FF, FF, F, BIG, NULL), LACT_ERR_INVALID_ARG);
    EXPECT(lact_chunk_update(&p, F, F, FF, NULL, 16, 16, FF, FF, FF, FF, FF, FF, F, BIG, NULL),
           LACT_ERR_INVALID_ARG);   /* momentum needs beta */
    EXPECT(lact_chunk_update(&p, F, F, FF, FF, 16, 16, FF, FF, FF, FF, FF, FF, F, BIG, NULL), ok_or_nodev);
    EXPECT(lact_apply(&p, F, 16, 8, FF, FF, FF, F, F, BIG, NULL), LACT_ERR_INVALID_ARG);
    EXPECT(lact_apply(&p, NULL, 16, 16, FF, FF, FF, F, F, BIG, NULL), LACT_ERR_INVALID_ARG);
    EXPECT(lact_apply(&p, F, 16, 16, FF, FF, FF, F, F, BIG, NULL), ok_or_nodev);

    /* the backward */
    EXPECT(bwd(&p, 512, F, FF, FF, FF, BIG), ok_or_nodev);
    EXPECT(bwd(&p, 512, NULL, FF, FF, FF, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(bwd(&p, 512, F, NULL, FF, FF, BIG), LACT_ERR_INVALID_ARG);
    EXPECT(bwd(&p, 512, F, FF, FF, NULL, BIG), LACT_ERR_INVALID_ARG);       /* oz without doz */
    EXPECT(bwd(&p, 512, F, FF, NULL, NULL, BIG), ok_or_nodev);
    const size_t bneed = lact_backward_workspace_size(&p, 512, 128, 0, NULL, NULL, 0);
    ++checks;
    if (bneed < need) ++failures;
    EXPECT(bwd(&p, 512, F, FF, FF, FF, bneed - 1), LACT_ERR_WORKSPACE_TOO_SMALL);
    b = p;
    b.flags = LACT_QK_PREP;
    EXPECT(bwd(&b, 512, F, FF, FF, FF, BIG), ok_or_nodev);
    b = prob(64, 192, LACT_DTYPE_F32, LACT_OPT_MUON_MOMENTUM);
    EXPECT(bwd(&b, 300, F, FF, NULL, NULL, BIG), ok_or_nodev);
    ++checks;
    if (lact_backward_workspace_size(&b, 300, 128, 0, NULL, NULL, 0) == 0) ++failures;

    /* timing */
    EXPECT(lact_timing_enable(-1, 1), LACT_ERR_INVALID_ARG);
    EXPECT(lact_timing_enable(LACT_K_COUNT, 1), LACT_ERR_INVALID_ARG);
    EXPECT(lact_timing_read(0, NULL, NULL), LACT_ERR_INVALID_ARG);
    {
        double ms = -1;
        int64_t n = -1;
        EXPECT(lact_timing_enable(LACT_K_UPD, 1), LACT_OK);
        EXPECT(lact_timing_read(LACT_K_UPD, &ms, &n), LACT_OK);
        EXPECT(lact_timing_enable(LACT_K_UPD, 0), LACT_OK);
        ++checks;
        if (ms != 0.0 || n != 0) ++failures;
    }

    printf("abi driver: %d checks, %d failures\n", checks, failures);
    return failures ? 1 : 0;
}
