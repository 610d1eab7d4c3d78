// Host-side sweep of the C ABI for an AddressSanitizer / UndefinedBehaviorSanitizer
// build (no GPU needed).  Every entry point is called with null, misaligned and
// out-of-range arguments and with argument sets that pass the checks; the latter
// reach a kernel launch, which fails with QSA_ERR_HIP on a machine without a GPU.
// Device pointers are fake, 16-byte-aligned addresses that the host code must never
// dereference.  Exits 1 on an unexpected status; the sanitizers abort on any memory
// error or undefined behaviour in the host code (argument checks, workspace layout,
// launch arithmetic).
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "qsa.h"

static int g_fail = 0;

#define EXPECT(expr, want)                                                                  \
    do {                                                                                    \
        const int got_ = (expr);                                                            \
        if (got_ != (want)) {                                                               \
            fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #expr, \
                    got_, (int)(want), qsa_last_error());                                   \
            g_fail = 1;                                                                     \
        }                                                                                   \
    } while (0)

// A status from a call whose arguments pass every check: the launch itself fails
// without a GPU (QSA_ERR_HIP); on a machine with one it may succeed.
#define EXPECT_LAUNCH(expr)                                                                   \
    do {                                                                                      \
        const int got_ = (expr);                                                              \
        if (got_ != QSA_ERR_HIP && got_ != QSA_OK) {                                          \
            fprintf(stderr, "line %d: %s returned %d before launching (%s)\n", __LINE__, #expr, \
                    got_, qsa_last_error());                                                  \
            g_fail = 1;                                                                       \
        }                                                                                     \
    } while (0)

static uint16_t *const D16 = (uint16_t *)(uintptr_t)0x7f0000100000ull;  // fake device address
static uint16_t *const MIS = (uint16_t *)(uintptr_t)0x7f0000100002ull;  // not 16-byte aligned
static float *const DF = (float *)(uintptr_t)0x7f0000200000ull;
static int32_t *const DI = (int32_t *)(uintptr_t)0x7f0000300000ull;
static void *const WS = (void *)(uintptr_t)0x7f0000400000ull;
static const size_t BIG = (size_t)1 << 40;

static qsa_config base_cfg(void)
{
    qsa_config c;
    c.h_idx = 16;
    c.d_idx = 128;
    c.block = 4;
    c.topk_blocks = 512;
    c.hq = 32;
    c.hkv = 4;
    c.d = 128;
    c.dv = 128;
    c.cap_tokens = 255244;
    c.rope_base = 1e4f;
    c.rms_eps = 1e-6f;
    c.attn_scale = 0.08838835f;
    return c;
}

static bool valid_status(int s)
{
    return s == QSA_OK || s == QSA_ERR_INVALID || s == QSA_ERR_CAPACITY ||
           s == QSA_ERR_UNSUPPORTED || s == QSA_ERR_HIP;
}

// Every integer field through extreme and boundary values: the check must classify
// each without overflow, and a valid shape must size its workspace for any n_q/n_ctx.
static void sweep_configs(void)
{
    const int32_t vals[] = {INT32_MIN, -1, 0, 1, 2, 3, 4, 7, 8, 16, 63, 64, 100, 128, 256,
                            512, 576, 1023, 1024, 1025, 4096, 65536, 1 << 21, (1 << 21) + 4,
                            INT32_MAX};
    const int nv = (int)(sizeof(vals) / sizeof(vals[0]));
    const int32_t nqs[] = {INT32_MIN, -1, 0, 1, 2, 3, 4, 5, 16, 1024, 65536, INT32_MAX};
    const int32_t nctx[] = {INT32_MIN, -1, 0, 1, 3, 4, 5, 4096, 255181, 1 << 21, INT32_MAX};
    for (int f = 0; f < 9; f++) {
        for (int i = 0; i < nv; i++) {
            qsa_config c = base_cfg();
            int32_t *fields[9] = {&c.h_idx, &c.d_idx, &c.block, &c.topk_blocks, &c.hq,
                                  &c.hkv, &c.d, &c.dv, &c.cap_tokens};
            *fields[f] = vals[i];
            const int s = qsa_config_check(&c);
            if (!valid_status(s) || s == QSA_ERR_HIP || s == QSA_ERR_CAPACITY) {
                fprintf(stderr, "config field %d = %d: status %d\n", f, vals[i], s);
                g_fail = 1;
            }
            for (int a = 0; a < (int)(sizeof(nqs) / sizeof(nqs[0])); a++)
                for (int b = 0; b < (int)(sizeof(nctx) / sizeof(nctx[0])); b++) {
                    const size_t w = qsa_workspace_size(&c, nqs[a], nctx[b]);
                    const bool ok = s == QSA_OK && nqs[a] >= 1 && nctx[b] >= 0 &&
                                    nctx[b] <= c.cap_tokens;
                    if (ok != (w != 0)) {
                        fprintf(stderr, "workspace field %d=%d n_q=%d n_ctx=%d: %zu bytes\n", f,
                                vals[i], nqs[a], nctx[b], w);
                        g_fail = 1;
                    }
                }
        }
    }
    // float fields
    const float fv[] = {-1.f, 0.f, 1e-30f, 1.f, 1e4f, 1e30f, __builtin_inff(), -__builtin_inff(),
                        __builtin_nanf("")};
    for (int f = 0; f < 3; f++)
        for (float v : fv) {
            qsa_config c = base_cfg();
            float *fields[3] = {&c.rope_base, &c.rms_eps, &c.attn_scale};
            *fields[f] = v;
            const int s = qsa_config_check(&c);
            if (s != QSA_OK && s != QSA_ERR_INVALID) {
                fprintf(stderr, "float field %d = %g: status %d\n", f, (double)v, s);
                g_fail = 1;
            }
        }
    EXPECT(qsa_config_check(NULL), QSA_ERR_INVALID);
    EXPECT((int)qsa_workspace_size(NULL, 1, 1), 0);
}

static void sweep_entry_points(void)
{
    qsa_config c = base_cfg();
    const qsa_config *cp = &c;
    qsa_layer_bufs L = {D16, D16, D16, D16, NULL};
    qsa_layer_bufs Lbad = {D16, MIS, D16, D16, NULL};
    qsa_layer_bufs Lnull = {D16, NULL, D16, D16, NULL};
    const int32_t n0 = 255180;

    // append / rebuild / kv append
    EXPECT(qsa_pool_append(cp, D16, -1, 0, D16, D16, NULL, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_pool_append(cp, D16, 1, -1, D16, D16, NULL, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_pool_append(cp, D16, 100, c.cap_tokens - 99, D16, D16, NULL, NULL),
           QSA_ERR_CAPACITY);
    EXPECT(qsa_pool_append(cp, D16, INT32_MAX, INT32_MAX, D16, D16, NULL, NULL),
           QSA_ERR_CAPACITY);
    EXPECT(qsa_pool_append(cp, NULL, 1, 0, D16, D16, NULL, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_pool_append(cp, D16, 1, 0, MIS, D16, NULL, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_pool_append(cp, D16, 0, 0, NULL, NULL, NULL, NULL), QSA_OK);
    EXPECT_LAUNCH(qsa_pool_append(cp, D16, 4096, 0, D16, D16, NULL, NULL));
    EXPECT_LAUNCH(qsa_pool_append(cp, D16, 1, n0, D16, D16, DF, NULL));
    EXPECT(qsa_pool_rebuild(cp, D16, D16, NULL, 0, c.cap_tokens + 1, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_pool_rebuild(cp, D16, D16, NULL, 5, 16, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_pool_rebuild(cp, D16, D16, NULL, 4, 16, NULL), QSA_OK);
    EXPECT_LAUNCH(qsa_pool_rebuild(cp, D16, D16, NULL, 0, n0, NULL));
    EXPECT(qsa_kv_append(cp, D16, D16, -3, 0, D16, D16, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_kv_append(cp, D16, NULL, 1, 0, D16, D16, NULL), QSA_ERR_INVALID);
    EXPECT_LAUNCH(qsa_kv_append(cp, D16, D16, 5, n0, D16, D16, NULL));

    // scores
    EXPECT(qsa_index_score(cp, D16, 0, 0, D16, DF, 1, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_index_score(cp, D16, 1, n0, D16, DF, 10, NULL), QSA_ERR_INVALID);  // ld small
    EXPECT(qsa_index_score(cp, D16, 2, c.cap_tokens, D16, DF, 1 << 20, NULL),
           QSA_ERR_CAPACITY);
    EXPECT(qsa_index_score(cp, D16, 8, 1000, D16, DF, 1003, NULL), QSA_ERR_INVALID);  // ld % 4
    EXPECT_LAUNCH(qsa_index_score(cp, D16, 1, n0, D16, DF, n0 / 4 + 1, NULL));
    EXPECT_LAUNCH(qsa_index_score(cp, D16, 1024, 126253, D16, DF, 31820, NULL));

    // top-k
    EXPECT(qsa_topk_blocks(cp, DF, 1, 100, 399, DI, DI, NULL, BIG, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_topk_blocks(cp, DF, 1, 100, 399, DI, DI, WS, 16, NULL), QSA_ERR_CAPACITY);
    EXPECT(qsa_topk_blocks(cp, DF, 1, 10, 399, DI, DI, WS, BIG, NULL), QSA_ERR_INVALID);
    EXPECT_LAUNCH(qsa_topk_blocks(cp, DF, 1, 100, 399, DI, DI, WS, BIG, NULL));
    EXPECT_LAUNCH(qsa_topk_blocks(cp, DF, 1024, 31820, 126253, DI, DI, WS, BIG, NULL));

    // gather / attention
    EXPECT(qsa_gather_kv(cp, DI, 511, n0 + 1, D16, D16, D16, D16, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_gather_kv(cp, DI, 512, -1, D16, D16, D16, D16, NULL), QSA_ERR_INVALID);
    EXPECT_LAUNCH(qsa_gather_kv(cp, DI, 512, n0 + 1, D16, D16, D16, D16, NULL));
    EXPECT_LAUNCH(qsa_gather_kv(cp, NULL, 0, 3, D16, D16, D16, D16, NULL));
    EXPECT(qsa_sparse_attn(cp, D16, D16, D16, 0, DF, WS, BIG, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_sparse_attn(cp, D16, D16, D16, 2052, DF, WS, BIG, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_sparse_attn(cp, D16, D16, D16, 2049, DF, WS, 64, NULL), QSA_ERR_CAPACITY);
    EXPECT_LAUNCH(qsa_sparse_attn(cp, D16, D16, D16, 2051, DF, WS, BIG, NULL));
    EXPECT(qsa_prefill_attn(cp, D16, 16, 1000, DI, 511, D16, D16, DF, 0, NULL, 0, NULL),
           QSA_ERR_INVALID);
    EXPECT(qsa_prefill_attn(cp, D16, 16, 1000, DI, 512, D16, D16, DF, 4, NULL, 0, NULL),
           QSA_ERR_INVALID);
    EXPECT(qsa_prefill_attn(cp, D16, 16, 1000, DI, 512, D16, D16, DF, 1, NULL, 0, NULL),
           QSA_ERR_INVALID);
    EXPECT_LAUNCH(qsa_prefill_attn(cp, D16, 1024, 126253, DI, 512, D16, D16, DF, 0, NULL, 0,
                                   NULL));
    EXPECT_LAUNCH(qsa_prefill_attn(cp, D16, 1024, 126253, DI, 512, D16, D16, DF, 1, WS, BIG,
                                   NULL));

    // decode steps
    EXPECT(qsa_decode_step(cp, NULL, n0, D16, D16, D16, D16, D16, DF, NULL, NULL, 0, WS, BIG,
                           NULL), QSA_ERR_INVALID);
    EXPECT(qsa_decode_step(cp, &Lbad, n0, D16, D16, D16, D16, D16, DF, NULL, NULL, 0, WS, BIG,
                           NULL), QSA_ERR_INVALID);
    EXPECT(qsa_decode_step(cp, &Lnull, n0, D16, D16, D16, D16, D16, DF, NULL, NULL, 0, WS, BIG,
                           NULL), QSA_ERR_INVALID);
    EXPECT(qsa_decode_step(cp, &L, c.cap_tokens, D16, D16, D16, D16, D16, DF, NULL, NULL, 0, WS,
                           BIG, NULL), QSA_ERR_CAPACITY);
    EXPECT(qsa_decode_step(cp, &L, n0, D16, D16, D16, D16, D16, DF, NULL, NULL, 7, WS, BIG,
                           NULL), QSA_ERR_INVALID);
    EXPECT(qsa_decode_step(cp, &L, n0, D16, D16, D16, D16, D16, DF, NULL, NULL, 0, WS, 1024,
                           NULL), QSA_ERR_CAPACITY);
    EXPECT(qsa_decode_step(cp, &L, n0, D16, D16, D16, D16, D16, DF, (float *)MIS, NULL, 0, WS,
                           BIG, NULL), QSA_ERR_INVALID);
    for (uint32_t flags = 0; flags < 2; flags++)
        for (int32_t n : {0, 1, 2, 3, 4, 2047, 2048, 2051, 4096, n0, c.cap_tokens - 1})
            EXPECT_LAUNCH(qsa_decode_step(cp, &L, n, D16, D16, D16, D16, D16, DF, DF, DI, flags,
                                          WS, BIG, NULL));
    EXPECT(qsa_decode_multi(cp, &L, n0, 5, D16, D16, D16, D16, D16, DF, NULL, 0, NULL, WS, BIG,
                            NULL), QSA_ERR_INVALID);
    EXPECT(qsa_decode_multi(cp, &L, n0, 3, D16, D16, D16, D16, D16, DF, DF, 10, NULL, WS, BIG,
                            NULL), QSA_ERR_INVALID);
    for (int32_t nq = 1; nq <= 4; nq++)
        EXPECT_LAUNCH(qsa_decode_multi(cp, &L, n0, nq, D16, D16, D16, D16, D16, DF, DF,
                                       n0 / 4 + 4, DI, WS, BIG, NULL));
    EXPECT(qsa_prefill_step(cp, &L, 126253, 0, D16, D16, D16, D16, D16, DF, NULL, 0, NULL, 0,
                            WS, BIG, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_prefill_step(cp, &L, 126253, 1024, D16, D16, D16, D16, D16, DF, DF, 100, NULL, 0,
                            WS, BIG, NULL), QSA_ERR_INVALID);
    EXPECT_LAUNCH(qsa_prefill_step(cp, &L, 126253, 1024, D16, D16, D16, D16, D16, DF, NULL, 0,
                                   NULL, 1, WS, BIG, NULL));

    // other shapes through the launch paths: k = 1024 with one KV head, 64-wide heads
    qsa_config c2 = base_cfg();
    c2.topk_blocks = 1024;
    c2.hq = 8;
    c2.hkv = 1;
    for (int32_t nq = 1; nq <= 4; nq++)
        EXPECT_LAUNCH(qsa_decode_multi(&c2, &L, 12001, nq, D16, D16, D16, D16, D16, DF, NULL, 0,
                                       NULL, WS, BIG, NULL));
    qsa_config c3 = base_cfg();
    c3.d = c3.dv = 64;
    c3.h_idx = 4;
    c3.d_idx = 64;
    EXPECT_LAUNCH(qsa_decode_step(&c3, &L, 4095, D16, D16, D16, D16, D16, DF, NULL, NULL, 1, WS,
                                  BIG, NULL));

    // MLA list attention
    EXPECT(qsa_mla_sparse_attn(D16, 16, D16, NULL, 576, 512, NULL, 262144, 2048, 0.04f, NULL, DI,
                               DF, WS, BIG, NULL), QSA_ERR_UNSUPPORTED);
    EXPECT(qsa_mla_sparse_attn(D16, 16, D16, NULL, 576, 512, D16, 4095, 1024, 0.04f, NULL, DI,
                               DF, WS, BIG, NULL), QSA_ERR_UNSUPPORTED);
    EXPECT(qsa_mla_sparse_attn(D16, 16, D16, NULL, 576, 512, D16, 262144, INT32_MAX, 0.04f, NULL,
                               DI, DF, WS, BIG, NULL), QSA_ERR_UNSUPPORTED);
    EXPECT(qsa_mla_sparse_attn(D16, 16, D16, NULL, 576, 512, D16, 262144, 2048,
                               __builtin_nanf(""), NULL, DI, DF, WS, BIG, NULL),
           QSA_ERR_INVALID);
    EXPECT(qsa_mla_sparse_attn(D16, 16, D16, NULL, 576, 512, D16, 262144, 2048, 0.04f, NULL, DI,
                               DF, WS, 100, NULL), QSA_ERR_CAPACITY);
    EXPECT_LAUNCH(qsa_mla_sparse_attn(D16, 16, D16, NULL, 576, 512, D16, 262144, 2048, 0.04f, DI,
                                      DI, DF, WS, BIG, NULL));
    EXPECT((int)qsa_mla_workspace_size(0, 512, 2048), 0);
    if (qsa_mla_workspace_size(16, 512, INT32_MAX) == 0)
        g_fail = 1;
    EXPECT(qsa_mla_list_status(NULL, 2048, NULL, NULL), QSA_ERR_INVALID);
    EXPECT_LAUNCH(qsa_mla_list_status(DI, 2048, NULL, NULL));

    // workspace init
    EXPECT(qsa_workspace_init(NULL, 64, NULL), QSA_ERR_INVALID);
    EXPECT(qsa_workspace_init(WS, 65, NULL), QSA_ERR_INVALID);
    EXPECT_LAUNCH(qsa_workspace_init(WS, 1 << 20, NULL));

    // status text for every code and a few others
    for (int s = -6; s <= 2; s++)
        if (!qsa_status_string(s) || !qsa_status_string(s)[0])
            g_fail = 1;
}

int main(void)
{
    sweep_configs();
    sweep_entry_points();
    if (g_fail)
        fprintf(stderr, "abi sweep: FAILED\n");
    else
        printf("abi sweep: ok\n");
    return g_fail;
}
