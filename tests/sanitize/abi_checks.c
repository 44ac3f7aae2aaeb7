/*
 * Host-side argument validation of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Built by tests/test_sanitizers.py from the
 * ABI's source (api.hip, host code instrumented) with the kernel launchers
 * replaced by stubs that abort (launch_stubs.cpp); no GPU is needed: every
 * call below passes a NULL context or bad arguments, so it returns from
 * validation before any HIP call.  Buffers are ordinary host memory of
 * exactly the documented sizes, so any read or write past them, or any
 * overflow in the size arithmetic, stops the run.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "linrec.h"

static int failures = 0;

#define EXPECT(cond, what)                                             \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, what); \
            ++failures;                                                \
        }                                                              \
    } while (0)

static void* buf(size_t n)
{
    /* 256-byte aligned, rounded up so aligned_alloc accepts the size */
    void* p = aligned_alloc(256, (n + 255) / 256 * 256 + 256);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    memset(p, 0, (n + 255) / 256 * 256 + 256);
    return p;
}

static linrec_tensor act(void* p, int B, int H, int T, int d)
{
    (void)B;
    linrec_tensor t = {p, (int64_t)H * T * d, (int64_t)T * d, d};
    return t;
}

int main(void)
{
    const int B = 2, H = 3, T = 320, D = 64;
    linrec_desc d = {B, H, T, D, D, 64, LINREC_BF16, LINREC_DECAY_TOKEN, LINREC_BF16};
    const size_t na = (size_t)B * H * T * D, ns = (size_t)B * H * D * D;

    void* q = buf(na * 2);
    void* k = buf(na * 2);
    void* v = buf(na * 2);
    void* dO = buf(na * 2);
    void* o = buf(na * 2);
    void* dq = buf(na * 2);
    void* dk = buf(na * 2);
    void* dv = buf(na * 2);
    float* dec = (float*)buf((size_t)B * H * T * 4);
    float* beta = (float*)buf((size_t)B * H * T * 4);
    float* dbeta = (float*)buf((size_t)B * H * T * 4);
    float* da = (float*)buf((size_t)B * H * T * 4);
    float* S_in = (float*)buf(ns * 4);
    float* S_out = (float*)buf(ns * 4);
    float* carry = (float*)buf((size_t)B * H * 4);

    /* sizes: positive for a valid descriptor, 0 for invalid ones */
    const size_t st_b = linrec_states_bytes(&d);
    EXPECT(st_b > 0, "states bytes");
    EXPECT(linrec_bwd_workspace_bytes(&d) > 0, "bwd workspace bytes");
    EXPECT(linrec_bwd_recompute_workspace_bytes(&d) > 0, "recompute workspace bytes");
    EXPECT(linrec_bwd_da_workspace_bytes(&d) > 0, "da workspace bytes");
    EXPECT(linrec_delta_workspace_bytes(&d) > 0, "delta workspace bytes");
    EXPECT(linrec_delta_saved_bytes(&d) > 0, "delta saved bytes");
    EXPECT(linrec_delta_bwd_workspace_bytes(&d) > 0, "delta bwd workspace bytes");
    const int32_t lens[3] = {64, 192, 64};
    EXPECT(linrec_seq_states_bytes(&d, 3, lens) > 0, "seq states bytes");
    EXPECT(linrec_bwd_seq_workspace_bytes(&d, 3, lens) > 0, "seq workspace bytes");
    const int32_t bad_lens[3] = {64, -1, 64};
    EXPECT(linrec_seq_states_bytes(&d, 3, bad_lens) == 0, "negative piece");
    EXPECT(linrec_seq_states_bytes(&d, 0, lens) == 0, "no pieces");
    EXPECT(linrec_seq_states_bytes(&d, 3, NULL) == 0, "NULL lengths");
    EXPECT(linrec_seq_states_bytes(NULL, 3, lens) == 0, "NULL desc");
    {
        linrec_desc e = d;
        e.dk = 96;
        EXPECT(linrec_states_bytes(&e) == 0, "d_k 96");
        e = d;
        e.chunk = 32;
        EXPECT(linrec_states_bytes(&e) == 0, "chunk 32");
        e = d;
        e.T = -64;
        EXPECT(linrec_states_bytes(&e) == 0, "negative T");
        e = d;
        e.B = 1 << 30;
        e.H = 1 << 30;
        EXPECT(linrec_states_bytes(&e) == 0, "B*H overflow");
        e = d;
        e.dtype = 7;
        EXPECT(linrec_states_bytes(&e) == 0, "unknown dtype");
    }

    const size_t ws_b = linrec_bwd_da_workspace_bytes(&d) + linrec_bwd_recompute_workspace_bytes(&d) +
                        linrec_bwd_seq_workspace_bytes(&d, 3, lens) + linrec_delta_bwd_workspace_bytes(&d);
    void* states = buf(st_b + linrec_seq_states_bytes(&d, 3, lens) + linrec_delta_saved_bytes(&d));
    void* ws = buf(ws_b + linrec_delta_workspace_bytes(&d));

    linrec_tensor tq = act(q, B, H, T, D), tk = act(k, B, H, T, D), tv = act(v, B, H, T, D);
    linrec_tensor tdO = act(dO, B, H, T, D), to = act(o, B, H, T, D);
    linrec_tensor tdq = act(dq, B, H, T, D), tdk = act(dk, B, H, T, D), tdv = act(dv, B, H, T, D);
    linrec_tensor tdec = {dec, (int64_t)H * T, T, 1}, tbeta = {beta, (int64_t)H * T, T, 1};
    linrec_tensor tdbeta = {dbeta, (int64_t)H * T, T, 1}, tda = {da, (int64_t)H * T, T, 1};

    /* valid arguments, NULL context: validation runs to the end, then E_NULL */
    EXPECT(linrec_fwd(NULL, &d, tq, tk, tv, tdec, S_in, to, S_out, states, NULL) == LINREC_E_NULL, "fwd");
    EXPECT(linrec_bwd(NULL, &d, tq, tk, tv, tdec, states, tdO, S_in, tdq, tdk, tdv, S_out, ws, NULL) ==
               LINREC_E_NULL, "bwd");
    EXPECT(linrec_bwd_noalloc(NULL, &d, tq, tk, tv, tdec, states, tdO, S_in, tdq, tdk, tdv, S_out, NULL) ==
               LINREC_E_NULL, "bwd_noalloc");
    EXPECT(linrec_bwd_recompute(NULL, &d, tq, tk, tv, tdec, S_in, tdO, NULL, tdq, tdk, tdv, S_out, ws, NULL) ==
               LINREC_E_NULL, "bwd_recompute");
    EXPECT(linrec_bwd_da(NULL, &d, tq, tk, tv, tdec, states, tdO, S_in, tdq, tdk, tdv, S_out, tda, carry,
                         carry, ws, NULL) == LINREC_E_NULL, "bwd_da");
    EXPECT(linrec_fwd_seq(NULL, &d, 3, lens, tq, tk, tv, tdec, S_in, to, S_out, states, NULL) == LINREC_E_NULL,
           "fwd_seq");
    EXPECT(linrec_bwd_seq(NULL, &d, 3, lens, tq, tk, tv, tdec, states, tdO, NULL, tdq, tdk, tdv, S_out, ws,
                          NULL) == LINREC_E_NULL, "bwd_seq");
    {
        linrec_desc e = d;
        e.dk = e.dv = 128;
        e.T = 128;
        EXPECT(linrec_delta_fwd(NULL, &e, act(q, B, H, 128, 128), act(k, B, H, 128, 128),
                                act(v, B, H, 128, 128), tbeta, tdec, S_in, act(o, B, H, 128, 128), S_out,
                                states, ws, NULL) == LINREC_E_NULL, "delta_fwd");
        EXPECT(linrec_delta_bwd(NULL, &e, act(q, B, H, 128, 128), act(k, B, H, 128, 128),
                                act(v, B, H, 128, 128), tbeta, tdec, states, act(dO, B, H, 128, 128), NULL,
                                act(dq, B, H, 128, 128), act(dk, B, H, 128, 128), act(dv, B, H, 128, 128),
                                tdbeta, S_out, ws, NULL) == LINREC_E_NULL, "delta_bwd");
        const int32_t dl[3] = {64, 37, 27};
        EXPECT(linrec_delta_seq_saved_bytes(&e, 3, dl) > 0, "delta seq saved bytes");
        EXPECT(linrec_delta_fwd_seq_workspace_bytes(&e, 3, dl) <= linrec_delta_workspace_bytes(&e),
               "delta fwd seq workspace bytes");
        EXPECT(linrec_delta_bwd_seq_workspace_bytes(&e, 3, dl) > 0, "delta bwd seq workspace bytes");
        EXPECT(linrec_delta_fwd_seq(NULL, &e, 3, dl, act(q, B, H, 128, 128), act(k, B, H, 128, 128),
                                    act(v, B, H, 128, 128), tbeta, tdec, S_in, act(o, B, H, 128, 128),
                                    S_out, states, ws, NULL) == LINREC_E_NULL, "delta_fwd_seq");
        EXPECT(linrec_delta_bwd_seq(NULL, &e, 3, dl, act(q, B, H, 128, 128), act(k, B, H, 128, 128),
                                    act(v, B, H, 128, 128), tbeta, tdec, states, act(dO, B, H, 128, 128),
                                    NULL, act(dq, B, H, 128, 128), act(dk, B, H, 128, 128),
                                    act(dv, B, H, 128, 128), tdbeta, S_out, ws, NULL) == LINREC_E_NULL,
               "delta_bwd_seq");
        const int32_t bad_dl[2] = {64, 0};
        EXPECT(linrec_delta_fwd_seq(NULL, &e, 2, bad_dl, act(q, B, H, 128, 128), act(k, B, H, 128, 128),
                                    act(v, B, H, 128, 128), tbeta, tdec, S_in, act(o, B, H, 128, 128),
                                    S_out, states, ws, NULL) == LINREC_E_SHAPE, "delta_fwd_seq bad lengths");
    }

    /* bad arguments: rejected before the context is looked at */
    {
        linrec_tensor bad = tq;
        bad.st = D - 8;   /* rows overlap */
        EXPECT(linrec_fwd(NULL, &d, bad, tk, tv, tdec, S_in, to, S_out, states, NULL) != LINREC_E_NULL,
               "overlapping rows");
        bad = tq;
        bad.ptr = (char*)q + 2;   /* breaks 16-byte row alignment */
        EXPECT(linrec_fwd(NULL, &d, bad, tk, tv, tdec, S_in, to, S_out, states, NULL) == LINREC_E_ALIGN,
               "misaligned q");
        EXPECT(linrec_fwd(NULL, &d, tq, tk, tv, tdec, S_in, to, S_out, (char*)states + 8, NULL) ==
                   LINREC_E_WORKSPACE, "misaligned states");
        EXPECT(linrec_fwd(NULL, NULL, tq, tk, tv, tdec, S_in, to, S_out, states, NULL) == LINREC_E_NULL,
               "NULL desc");
        EXPECT(linrec_bwd(NULL, &d, tq, tk, tv, tdec, states, tdO, S_in, tdq, tdk, tdv, S_out, NULL, NULL) ==
                   LINREC_E_WORKSPACE, "NULL workspace");
        linrec_desc e = d;
        e.decay = LINREC_DECAY_NONE;
        EXPECT(linrec_bwd_da(NULL, &e, tq, tk, tv, tdec, states, tdO, S_in, tdq, tdk, tdv, S_out, tda, carry,
                             carry, ws, NULL) == LINREC_E_LAYOUT, "da without decay");
        e = d;
        e.out_dtype = 9;
        EXPECT(linrec_fwd(NULL, &e, tq, tk, tv, tdec, S_in, to, S_out, states, NULL) != LINREC_OK,
               "unknown out dtype");
        const int32_t ragged[2] = {100, 220};   /* ragged pieces are valid */
        EXPECT(linrec_fwd_seq(NULL, &d, 2, ragged, tq, tk, tv, tdec, S_in, to, S_out, states, NULL) ==
                   LINREC_E_NULL, "ragged pieces");
        const int32_t empty[2] = {0, 320};
        EXPECT(linrec_fwd_seq(NULL, &d, 2, empty, tq, tk, tv, tdec, S_in, to, S_out, states, NULL) ==
                   LINREC_E_SHAPE, "empty piece");
        /* an empty piece: only the carried pointers are checked */
        linrec_desc z = d;
        z.T = 0;
        linrec_tensor none = {NULL, 0, 0, 0};
        EXPECT(linrec_fwd(NULL, &z, none, none, none, none, NULL, none, S_out, NULL, NULL) == LINREC_E_NULL,
               "empty piece fwd");
        EXPECT(linrec_bwd_da(NULL, &z, none, none, none, none, NULL, none, NULL, none, none, none, S_out,
                             none, NULL, carry, NULL, NULL) == LINREC_E_NULL, "empty piece bwd_da");
        EXPECT(linrec_bwd_recompute_workspace_bytes(&z) == 0 && linrec_bwd_da_workspace_bytes(&z) == 0,
               "empty piece sizes");
        const int32_t short_sum[2] = {64, 64};
        EXPECT(linrec_fwd_seq(NULL, &d, 2, short_sum, tq, tk, tv, tdec, S_in, to, S_out, states, NULL) ==
                   LINREC_E_SHAPE, "pieces do not sum to T");
    }

    /* context-free helpers */
    for (int s = -3; s < 16; ++s)
        EXPECT(linrec_status_str((linrec_status)s) != NULL, "status string");
    EXPECT(linrec_ctx_set_timing(NULL, 1) == LINREC_E_NULL, "timing NULL ctx");
    {
        int64_t n = 0;
        double ms = 0;
        EXPECT(linrec_ctx_kernel_times(NULL, 0, &n, &ms) == LINREC_E_NULL, "kernel times NULL ctx");
    }
    EXPECT(linrec_ctx_destroy(NULL) == LINREC_OK || linrec_ctx_destroy(NULL) == LINREC_E_NULL,
           "destroy NULL");
    EXPECT(linrec_version() > 0, "version");
    (void)linrec_last_hip_error();

    free(q); free(k); free(v); free(dO); free(o); free(dq); free(dk); free(dv);
    free(dec); free(beta); free(dbeta); free(da); free(S_in); free(S_out); free(carry);
    free(states); free(ws);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi checks passed\n");
    return 0;
}
