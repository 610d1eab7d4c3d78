/*
 * Drives every exported function of the CPU oracle (oracle/qsa_oracle.c and the
 * all-core timing form oracle/qsa_oracle_mt.c) on small and degenerate inputs for
 * an AddressSanitizer / UndefinedBehaviorSanitizer build: empty contexts, contexts
 * shorter than a block, every tail length, k = 0 and k >= nb, NaN and infinite
 * scores, empty cell and mask lists, absent optional arrays.  The sanitizers abort
 * on any memory error or undefined behaviour; a few consistency checks between
 * the oracle's own two forms of a result exit 1 when they disagree.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t h_idx, d_idx, topk;
    int32_t hq, hkv, d, dv;
    double rope_base, rms_eps, scale;
} orc_cfg;

double orc_h2d(uint16_t h);
uint16_t orc_d2h(double x);
void orc_h2d_array(const uint16_t *h, int64_t n, double *out);
void orc_d2h_array(const double *x, int64_t n, uint16_t *out);
int64_t orc_block_pos(int64_t b);
void orc_pool_block(int H, int d, const uint16_t *raw4, int64_t pos, double base, double eps,
                    const float *w, uint16_t *out);
void orc_pool_rebuild(int H, int d, const uint16_t *raw, int64_t n_tokens, double base,
                      double eps, const float *w, uint16_t *pooled);
void orc_pool_append(int H, int d, const uint16_t *k_new, int64_t n_new, int64_t n_before,
                     uint16_t *raw, uint16_t *pooled, double base, double eps, const float *w);
void orc_index_score(int H, int d, const uint16_t *q_idx, const uint16_t *pooled, int64_t nb,
                     double *s64, float *s32);
int64_t orc_topk_sort(const float *scores, int64_t nb, int64_t k, int32_t *blk);
int64_t orc_topk_rank(const float *scores, int64_t nb, int64_t k, int32_t *blk);
int64_t orc_cells(const int32_t *blk, int64_t n_sel, int64_t n_tokens, int64_t *cells);
void orc_attn_cells(int hq, int hkv, int d, int dv, const uint16_t *q, const uint16_t *kc,
                    const uint16_t *vc, const int64_t *cells, int64_t nc, double scale,
                    double *out);
void orc_attn_dense_masked(int hq, int hkv, int d, int dv, const uint16_t *q,
                           const uint16_t *kc, const uint16_t *vc, int64_t n_tokens,
                           const uint8_t *visible, double scale, double *out);
int64_t orc_decode_step(const orc_cfg *cf, uint16_t *raw, uint16_t *pooled, uint16_t *kc,
                        uint16_t *vc, int64_t n_before, const uint16_t *q_idx,
                        const uint16_t *k_idx_new, const uint16_t *q, const uint16_t *k_new,
                        const uint16_t *v_new, const float *rms_w, double *scores64,
                        float *scores32, int32_t *blk, double *out);
int64_t orc_decode_step_mt(const orc_cfg *cf, uint16_t *raw, uint16_t *pooled, uint16_t *kc,
                           uint16_t *vc, int64_t n_before, const uint16_t *q_idx,
                           const uint16_t *k_idx_new, const uint16_t *q, const uint16_t *k_new,
                           const uint16_t *v_new, const float *rms_w, double *scores64,
                           float *scores32, int32_t *blk, double *out, int n_threads);
int64_t orc_prefill_row(const orc_cfg *cf, const uint16_t *pooled, const uint16_t *kc,
                        const uint16_t *vc, int64_t pos, const uint16_t *q_idx_row,
                        const uint16_t *q_row, double *scores64, float *scores32, int32_t *blk,
                        double *out);
int64_t orc_mask_list(const uint16_t *mask, int64_t n, int32_t *list);
void orc_mla_attn(int hq, int dkq, int dv, const uint16_t *q, const uint16_t *kv,
                  const uint16_t *v, const uint16_t *mask, const int32_t *list, int64_t nl,
                  double scale, double *out);
void orc_mla_dense(int hq, int dkq, int dv, const uint16_t *q, const uint16_t *kv,
                   const uint16_t *v, const uint16_t *mask, int64_t n, double scale, double *out);

static int g_fail = 0;
static uint64_t g_state = 0x9e3779b97f4a7c15ull;

static double unif(void) /* splitmix64 -> [0, 1) */
{
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1.0p-53;
}

static uint16_t *rand_f16(int64_t n)
{
    uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; i++)
        a[i] = orc_d2h(4.0 * unif() - 2.0);
    return a;
}

static void check(int ok, const char *what)
{
    if (!ok) {
        fprintf(stderr, "oracle sweep: %s\n", what);
        g_fail = 1;
    }
}

static void sweep_codec(void)
{
    double *d = (double *)malloc(sizeof(double) * 65536);
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
    for (int i = 0; i < 65536; i++)
        h[i] = (uint16_t)i;
    orc_h2d_array(h, 65536, d);
    uint16_t *back = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
    orc_d2h_array(d, 65536, back);
    for (int i = 0; i < 65536; i++)
        if (!isnan(d[i]))
            check(back[i] == h[i], "binary16 round trip");
    const double edge[] = {0.0, -0.0, 1e-30, 5.96e-8, 2.98e-8, 6.1e-5, 65504.0, 65520.0, 1e30,
                           INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof(edge) / sizeof(edge[0]); i++)
        (void)orc_d2h(edge[i]);
    free(d);
    free(h);
    free(back);
}

static void sweep_pool(void)
{
    const int H = 2, d = 8;
    const int64_t row = H * d, cap = 24;
    float w[8];
    for (int i = 0; i < d; i++)
        w[i] = 0.5f + 0.1f * (float)i;
    for (int64_t n = 0; n <= 13; n++) {
        uint16_t *raw_all = rand_f16(cap * row);
        uint16_t *full = (uint16_t *)calloc((size_t)(cap / 4 * row), 2);
        uint16_t *inc = (uint16_t *)calloc((size_t)(cap / 4 * row), 2);
        uint16_t *raw = (uint16_t *)calloc((size_t)(cap * row), 2);
        const float *wt = (n & 1) ? w : NULL;
        orc_pool_rebuild(H, d, raw_all, n, 1e4, 1e-6, wt, full);
        for (int64_t t = 0; t < n; t++)
            orc_pool_append(H, d, raw_all + t * row, 1, t, raw, inc, 1e4, 1e-6, wt);
        check(memcmp(full, inc, sizeof(uint16_t) * (size_t)(n / 4 * row)) == 0,
              "append equals rebuild");
        free(raw_all);
        free(full);
        free(inc);
        free(raw);
    }
    /* all-zero block with eps = 0: 0 / 0 in the norm, no memory error */
    uint16_t zero4[4 * 16] = {0}, out[16];
    orc_pool_block(2, 8, zero4, orc_block_pos(3), 1e4, 0.0, NULL, out);
    orc_pool_block(2, 8, zero4, orc_block_pos(0), 1e4, 1e-6, NULL, out);
}

static void sweep_select(void)
{
    for (int64_t nb = 0; nb <= 40; nb += 3) {
        float *s = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
        for (int64_t b = 0; b < nb; b++) {
            double u = unif();
            s[b] = u < 0.1 ? NAN : (u < 0.15 ? INFINITY : (u < 0.2 ? -0.0f : (float)(u * 8.0)));
            if (u > 0.6)
                s[b] = 3.0f; /* ties */
        }
        int32_t *a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb + 1));
        int32_t *b2 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb + 1));
        const int64_t ks[] = {0, 1, 5, nb - 1, nb, nb + 7};
        for (size_t i = 0; i < sizeof(ks) / sizeof(ks[0]); i++) {
            if (ks[i] < 0)
                continue;
            const int64_t n1 = orc_topk_sort(s, nb, ks[i], a);
            const int64_t n2 = orc_topk_rank(s, nb, ks[i], b2);
            check(n1 == n2 && memcmp(a, b2, sizeof(int32_t) * (size_t)n1) == 0,
                  "sort form equals rank form");
            int64_t *cells = (int64_t *)malloc(sizeof(int64_t) * (size_t)(4 * n1 + 4));
            for (int64_t n = 4 * nb; n < 4 * nb + 4; n++)
                check(orc_cells(a, n1, n, cells) == 4 * n1 + n % 4, "cell count");
            free(cells);
        }
        free(s);
        free(a);
        free(b2);
    }
}

static void sweep_attention(void)
{
    const int hq = 4, hkv = 2, d = 8, dv = 8;
    const int64_t n = 23;
    uint16_t *q = rand_f16(hq * d), *kc = rand_f16(n * hkv * d), *vc = rand_f16(n * hkv * dv);
    double out[32], out2[32];
    int64_t cells[23];
    uint8_t vis[23];
    for (int64_t nc = 0; nc <= n; nc += 5) {
        for (int64_t c = 0; c < n; c++)
            vis[c] = 0;
        for (int64_t c = 0; c < nc; c++) {
            cells[c] = (c * 7) % n;
            vis[cells[c]] = 1;
        }
        /* distinct cells when nc <= n and 7 is prime to 23 */
        orc_attn_cells(hq, hkv, d, dv, q, kc, vc, cells, nc, 0.3, out);
        orc_attn_dense_masked(hq, hkv, d, dv, q, kc, vc, n, vis, 0.3, out2);
        if (nc > 0)
            for (int i = 0; i < hq * dv; i++)
                check(fabs(out[i] - out2[i]) <= 1e-12 * (1.0 + fabs(out2[i])), "gathered = dense");
    }
    free(q);
    free(kc);
    free(vc);
}

static void sweep_steps(void)
{
    orc_cfg cf = {2, 8, 3, 4, 2, 8, 8, 1e4, 1e-6, 0.35};
    const int64_t cap = 32, row = 16, kvr = 16;
    uint16_t *q_idx = rand_f16(row), *q = rand_f16(4 * 8), *news = rand_f16(cap * row);
    uint16_t *kn = rand_f16(cap * kvr), *vn = rand_f16(cap * kvr);
    for (int threads = 0; threads <= 5; threads++) {
        uint16_t *raw[2], *pooled[2], *kc[2], *vc[2];
        for (int s = 0; s < 2; s++) {
            raw[s] = (uint16_t *)calloc((size_t)(cap * row), 2);
            pooled[s] = (uint16_t *)calloc((size_t)(cap / 4 * row), 2);
            kc[s] = (uint16_t *)calloc((size_t)(cap * kvr), 2);
            vc[s] = (uint16_t *)calloc((size_t)(cap * kvr), 2);
        }
        for (int64_t nb = 0; nb < 20; nb++) {
            double s64[2][8], out[2][32];
            float s32[2][8];
            int32_t blk[2][8];
            const int64_t n1 = orc_decode_step(&cf, raw[0], pooled[0], kc[0], vc[0], nb, q_idx,
                                               news + nb * row, q, kn + nb * kvr, vn + nb * kvr,
                                               NULL, s64[0], s32[0], blk[0], out[0]);
            const int64_t n2 = orc_decode_step_mt(&cf, raw[1], pooled[1], kc[1], vc[1], nb,
                                                  q_idx, news + nb * row, q, kn + nb * kvr,
                                                  vn + nb * kvr, NULL, threads & 1 ? s64[1] : NULL,
                                                  s32[1], blk[1], out[1], threads);
            check(n1 == n2 && memcmp(blk[0], blk[1], sizeof(int32_t) * (size_t)n1) == 0 &&
                      memcmp(out[0], out[1], sizeof(double) * 32) == 0,
                  "threaded step equals step");
        }
        for (int s = 0; s < 2; s++) {
            free(raw[s]);
            free(pooled[s]);
            free(kc[s]);
            free(vc[s]);
        }
    }
    /* prefill rows over the caches of the last 20-token context */
    uint16_t *pooled = (uint16_t *)calloc((size_t)(cap / 4 * row), 2);
    orc_pool_rebuild(2, 8, news, 20, 1e4, 1e-6, NULL, pooled);
    for (int64_t pos = 0; pos < 20; pos++) {
        double s64[8], out[32];
        float s32[8];
        int32_t blk[8];
        orc_prefill_row(&cf, pooled, kn, vn, pos, q_idx, q, s64, s32, blk, out);
    }
    free(pooled);
    free(q_idx);
    free(q);
    free(news);
    free(kn);
    free(vn);
}

static void sweep_mla(void)
{
    const int hq = 2, dkq = 12, dv = 8;
    const int64_t n = 70;
    uint16_t *q = rand_f16(hq * dkq), *kv = rand_f16(n * dkq), *v = rand_f16(n * dv);
    uint16_t mask[70];
    int32_t list[70];
    double out[16], out2[16];
    for (int pattern = 0; pattern < 4; pattern++) {
        for (int64_t j = 0; j < n; j++) {
            const int vis = pattern == 0 ? 0 : (pattern == 1 ? 1 : (int)(j % (pattern + 1) == 0));
            mask[j] = vis ? orc_d2h(pattern == 3 ? -0.5 : 0.0) : orc_d2h(-INFINITY);
        }
        const int64_t nl = orc_mask_list(mask, n, list);
        for (int withv = 0; withv < 2; withv++) {
            orc_mla_attn(hq, dkq, dv, q, kv, withv ? v : NULL, mask, list, nl, 0.2, out);
            orc_mla_dense(hq, dkq, dv, q, kv, withv ? v : NULL, mask, n, 0.2, out2);
            if (nl > 0)
                for (int i = 0; i < hq * dv; i++)
                    check(fabs(out[i] - out2[i]) <= 1e-12 * (1.0 + fabs(out2[i])),
                          "list = dense");
        }
    }
    free(q);
    free(kv);
    free(v);
}

int main(void)
{
    sweep_codec();
    sweep_pool();
    sweep_select();
    sweep_attention();
    sweep_steps();
    sweep_mla();
    printf(g_fail ? "oracle sweep: FAILED\n" : "oracle sweep: ok\n");
    return g_fail;
}
