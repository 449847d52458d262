/*
 * abi_sanitize_driver.c -- drives the host-side argument checks of libdsc's C
 * ABI (include/dsc.h) for a build of its ABI layer with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_abi_sanitized.py).  Every call below
 * fails validation, which the library performs before any HIP call, so no GPU
 * is needed; the workspace-size queries are host arithmetic.  Extreme sizes
 * probe the overflow guards.  Exits 0 when every call returns the expected
 * status; the sanitizers abort on any invalid access or undefined operation.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dsc.h"

static int failures = 0;

static void expect(int got, int want, const char *what) {
    if (got != want) {
        fprintf(stderr, "%s: returned %d, expected %d (%s)\n", what, got, want, dsc_last_error());
        ++failures;
    }
}

/* fake device addresses, 16-byte aligned, 1 GiB apart (never dereferenced) */
static void *P(int k) { return (void *)((uintptr_t)k << 30); }
static void *ODD(int k) { return (void *)(((uintptr_t)k << 30) + 2); }

int main(void) {
    const int64_t big = (int64_t)1 << 40, huge = INT64_MAX;
    const int32_t cu_ok[3] = {0, 4, 8};

    /* head-wise: every stage of the checks */
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 64, 4, 8, NULL, P(2), NULL, 0, 0, P(3)), DSC_ERR_NULL, "hw null");
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 64, 0, 8, P(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_SHAPE, "hw W");
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 60, 4, 4, P(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_SHAPE, "hw D");
    /* any H dividing D passes the shape checks: y in place is then rejected */
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 48, 4, 24, P(1), P(2), NULL, 0, 0, P(1)), DSC_ERR_ALIAS, "hw H");
    expect(dsc_headwise_fwd(0, 7, 1, 8, 64, 4, 8, P(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_UNSUPPORTED, "hw dtype");
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 64, 4, 8, ODD(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_ALIGNMENT, "hw align");
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 64, 4, 8, P(1), P(2), NULL, 0, 0, P(1)), DSC_ERR_ALIAS, "hw alias");
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 64, 4, 8, P(1), P(2), P(9), 0, 0, P(3)), DSC_ERR_SHAPE, "hw cu count");
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 64, 4, 8, P(1), P(2), NULL, 0, 2, P(3)), DSC_ERR_SHAPE, "hw residual");
    /* extreme sizes: rejected without overflowing */
    expect(dsc_headwise_fwd(0, DSC_BF16, big, big, 64, 4, 8, P(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_SHAPE, "hw B*T");
    expect(dsc_headwise_fwd(0, DSC_BF16, huge, 2, 64, 4, 8, P(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_SHAPE, "hw B max");
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, huge - 7, 4, 8, P(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_SHAPE, "hw D max");
    expect(dsc_headwise_fwd(0, DSC_BF16, -1, 8, 64, 4, 8, P(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_SHAPE, "hw B<0");
    expect(dsc_headwise_bwd(0, DSC_BF16, 1, 8, 64, 4, 8, P(1), P(2), P(3), NULL, 0, 0, P(3), P(5)), DSC_ERR_ALIAS,
           "hw bwd alias");
    expect(dsc_headwise_bwd(0, DSC_FP32, 1, 8, 64, 4, 8, P(1), P(2), P(3), NULL, 0, 0, P(4), NULL), DSC_ERR_NULL,
           "hw bwd null");
    /* the message buffer: a long error text is cut, never overrun */
    expect(dsc_headwise_fwd(0, DSC_BF16, 1, 8, 64, 4, 8, P(1), P(2), cu_ok, 2, 0, P(1)), DSC_ERR_ALIAS, "hw cu alias");
    if (strlen(dsc_last_error()) >= 512) { fprintf(stderr, "message too long\n"); ++failures; }

    /* rotary embedding */
    expect(dsc_rope_table(0, 16, 3, 10000.0, (float *)P(1)), DSC_ERR_SHAPE, "rope table odd");
    expect(dsc_rope_table(0, 16, 64, -1.0, (float *)P(1)), DSC_ERR_SHAPE, "rope table base");
    expect(dsc_rope_table(0, huge, 64, 10000.0, (float *)P(1)), DSC_ERR_SHAPE, "rope table max_pos");
    expect(dsc_headwise_rope_fwd(0, DSC_BF16, 1, 8, 64, 4, 8, P(1), P(2), NULL, 0, 0, 48, 32, (const float *)P(4),
                                 16, P(3)), DSC_ERR_SHAPE, "rope rot");
    expect(dsc_headwise_rope_fwd(0, DSC_BF16, 1, 8, 64, 4, 8, P(1), P(2), NULL, 0, 0, 64, 32, (const float *)P(4),
                                 4, P(3)), DSC_ERR_SHAPE, "rope max_pos < T");
    expect(dsc_headwise_rope_bwd(0, DSC_BF16, 1, 8, 64, 4, 8, P(1), P(2), P(3), NULL, 0, 0, 64, 32,
                                 (const float *)P(4), 16, P(5), P(5)), DSC_ERR_ALIAS, "rope bwd alias");

    /* low-rank, both backward entry points */
    expect(dsc_lowrank_fwd(0, DSC_BF16, 1, 8, 64, 4, 0, P(1), P(2), P(3), NULL, 0, 0, P(4)), DSC_ERR_SHAPE, "lr R");
    expect(dsc_lowrank_fwd(0, DSC_BF16, 1, 8, 64, 4, 16, P(1), P(2), P(3), NULL, 0, 0, P(3)), DSC_ERR_ALIAS, "lr alias");
    const size_t need = dsc_lowrank_bwd_workspace_size(DSC_BF16, 8, 2048, 2304, 4, 32);
    const size_t dneed = dsc_lowrank_bwd_deterministic_workspace_size(DSC_BF16, 8, 2048, 2304, 4, 32);
    if (need == 0 || dneed <= need) { fprintf(stderr, "workspace sizes %zu %zu\n", need, dneed); ++failures; }
    expect((int)dsc_lowrank_bwd_workspace_size(DSC_BF16, big, big, 64, 4, 16), 0, "lr ws B*T");
    expect((int)dsc_lowrank_bwd_deterministic_workspace_size(DSC_BF16, 1, 1 << 30, 1 << 30, 4, 128), 0, "det ws");
    expect((int)dsc_lowrank_bwd_deterministic_workspace_size(DSC_BF16, huge, 1, 64, 4, 16), 0, "det ws B max");
    for (int det = 0; det < 2; ++det) {
        dsc_status (*f)(void *, int, int64_t, int64_t, int64_t, int32_t, int32_t, const void *, const void *,
                        const void *, const void *, const int32_t *, int32_t, int32_t, void *, void *, float *,
                        void *, size_t) = det ? dsc_lowrank_bwd_deterministic : dsc_lowrank_bwd;
        const size_t n = det ? dneed : need;
        expect(f(0, DSC_BF16, 8, 2048, 2304, 4, 32, P(1), P(2), P(3), P(4), NULL, 0, 0, P(5), P(6), (float *)P(7),
                 NULL, 0), DSC_ERR_WORKSPACE, "lr bwd no workspace");
        expect(f(0, DSC_BF16, 8, 2048, 2304, 4, 32, P(1), P(2), P(3), P(4), NULL, 0, 0, P(5), P(6), (float *)P(7),
                 P(8), n - 1), DSC_ERR_WORKSPACE, "lr bwd small workspace");
        expect(f(0, DSC_BF16, 8, 2048, 2304, 4, 32, P(1), P(2), P(3), P(4), NULL, 0, 0, P(5), P(6), (float *)P(7),
                 P(1), n), DSC_ERR_ALIAS, "lr bwd workspace alias");
        expect(f(0, DSC_BF16, 8, 2048, 2304, 4, 129, P(1), P(2), P(3), P(4), NULL, 0, 0, P(5), P(6), (float *)P(7),
                 P(8), n), DSC_ERR_SHAPE, "lr bwd R");
        expect(f(0, DSC_BF16, 0, 2048, 2304, 4, 32, NULL, NULL, NULL, NULL, NULL, 0, 0, NULL, NULL, NULL, NULL, 0),
               DSC_ERR_NULL, "lr bwd empty needs dU");
    }

    /* the allocation-free backward: its scratch limit and the usual checks, before any HIP call */
    expect(dsc_lowrank_bwd_noalloc(0, DSC_BF16, 4, 16385, 64, 4, 64, P(1), P(2), P(3), P(4), NULL, 0, 0, P(5), P(6),
                                   (float *)P(7)), DSC_ERR_WORKSPACE, "noalloc limit");
    expect(dsc_lowrank_bwd_noalloc(0, DSC_BF16, huge, 2, 64, 4, 64, P(1), P(2), P(3), P(4), NULL, 0, 0, P(5), P(6),
                                   (float *)P(7)), DSC_ERR_SHAPE, "noalloc B max");
    expect(dsc_lowrank_bwd_noalloc(0, DSC_BF16, 1, 8, 64, 4, 16, P(1), P(2), P(3), P(4), NULL, 0, 0, P(1), P(6),
                                   (float *)P(7)), DSC_ERR_ALIAS, "noalloc alias");

    /* static layer */
    expect(dsc_static_fwd(0, DSC_BF16, 1, 8, 64, 9, P(1), P(2), NULL, 0, 0, P(3)), DSC_ERR_SHAPE, "st W");
    expect(dsc_static_bwd(0, DSC_BF16, 1, 8, 64, 4, P(1), P(2), P(3), NULL, 0, 0, P(4), (float *)P(4)),
           DSC_ERR_ALIAS, "st alias");
    expect(dsc_static_bwd(0, DSC_BF16, 1, 0, 64, 4, NULL, NULL, NULL, NULL, 0, 0, NULL, NULL), DSC_ERR_NULL,
           "st empty needs dc");

    const size_t sneed = dsc_static_bwd_deterministic_workspace_size(DSC_BF16, 8, 2048, 2304, 4);
    if (sneed == 0) { fprintf(stderr, "static workspace size 0\n"); ++failures; }
    expect((int)dsc_static_bwd_deterministic_workspace_size(DSC_BF16, big, big, 2304, 4), 0, "st det ws B*T");
    expect(dsc_static_bwd_deterministic(0, DSC_BF16, 8, 2048, 2304, 4, P(1), P(2), P(3), NULL, 0, 0, P(4),
                                        (float *)P(5), P(6), sneed - 1), DSC_ERR_WORKSPACE, "st det small workspace");
    expect(dsc_static_bwd_deterministic(0, DSC_BF16, 8, 2048, 2304, 4, P(1), P(2), P(3), NULL, 0, 0, P(4),
                                        (float *)P(5), P(3), sneed), DSC_ERR_ALIAS, "st det workspace alias");

    /* decoding */
    expect(dsc_headwise_decode(0, DSC_BF16, 4, 64, 4, 8, P(1), P(2), P(3), 0, P(3)), DSC_ERR_ALIAS, "dec alias");
    expect(dsc_headwise_decode(0, DSC_BF16, 4, 64, 4, 8, P(1), P(2), NULL, 0, P(4)), DSC_ERR_NULL, "dec state");
    expect(dsc_headwise_rope_decode(0, DSC_BF16, 4, 64, 4, 8, P(1), P(2), P(3), 0, 64, 32, (const float *)P(5), 16,
                                    NULL, P(4)), DSC_ERR_NULL, "rope dec positions");
    expect(dsc_lowrank_decode(0, DSC_BF16, 4, 64, 4, 0, P(1), P(2), P(3), P(4), 0, P(5)), DSC_ERR_SHAPE, "lr dec R");
    expect(dsc_state_from_prefill(0, DSC_BF16, 1, 8, 64, 4, P(1), NULL, 0, P(1)), DSC_ERR_ALIAS, "prefill alias");
    expect(dsc_state_from_prefill(0, DSC_BF16, big, big, 64, 4, P(1), NULL, 0, P(2)), DSC_ERR_SHAPE, "prefill B*T");

    expect(dsc_headwise_decode(0, DSC_BF16, huge, 64, 4, 8, P(1), P(2), P(3), 0, P(4)), DSC_ERR_SHAPE, "dec B max");
    expect(dsc_lowrank_decode(0, DSC_BF16, huge, 64, 4, 16, P(1), P(2), P(3), P(4), 0, P(5)), DSC_ERR_SHAPE,
           "lr dec B max");
    expect(dsc_headwise_rope_decode(0, DSC_BF16, 4, 64, 4, 8, P(1), P(2), P(3), 0, 64, 32, (const float *)P(5), huge,
                                    (const int32_t *)P(6), P(4)), DSC_ERR_SHAPE, "rope dec max_pos");
    expect(dsc_state_from_prefill(0, DSC_BF16, 1, 8, 64, 4, P(1), cu_ok, INT32_MAX, P(2)), DSC_ERR_SHAPE,
           "prefill n_seqs");

    /* status strings, every code and out of range */
    for (int st = -3; st < 12; ++st)
        if (!dsc_status_string(st) || !dsc_status_string(st)[0]) { fprintf(stderr, "status %d\n", st); ++failures; }
    if (dsc_abi_version() != 1) ++failures;
    if (failures) return 1;
    printf("abi checks ok\n");
    return 0;
}
