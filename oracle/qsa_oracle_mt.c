/*
 * QSA layer-step ORACLE, all-core timing form -- test infrastructure, not product
 * code.  Only the benchmark's CPU-baseline leg loads it.
 *
 * The decode step of qsa_oracle.c (orc_decode_step) with one change: the block
 * scan -- the score of every complete block against the query, the only O(N) part
 * of the step (ariera, Qiita part 10, "QSAとQSA indexerについて") -- is split into
 * contiguous block ranges, one per POSIX thread.  Each thread runs the unchanged
 * orc_index_score on its range, so every score is the same fp64 sum in the same
 * order as in the single-threaded oracle; the append, the top-k, the cell list and
 * the attention run on the calling thread through the same functions.  It is built
 * into its own library together with qsa_oracle.c; the parity library is not
 * changed by it.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BLOCK 4

/* The oracle's own functions (qsa_oracle.c). */
typedef struct {
    int32_t h_idx, d_idx, topk;
    int32_t hq, hkv, d, dv;
    double rope_base, rms_eps, scale;
} orc_cfg;

void orc_pool_append(int H, int d, const uint16_t *k_new, int64_t n_new, int64_t n_before,
                     uint16_t *raw, uint16_t *pooled, double base, double eps, const float *w);
void orc_index_score(int H, int d, const uint16_t *q_idx, const uint16_t *pooled, int64_t nb,
                     double *s64, float *s32);
int64_t orc_topk_sort(const float *scores, int64_t nb, int64_t k, int32_t *blk);
int64_t orc_cells(const int32_t *blk, int64_t n_sel, int64_t n_tokens, int64_t *cells);
void orc_attn_cells(int hq, int hkv, int d, int dv, const uint16_t *q, const uint16_t *kc,
                    const uint16_t *vc, const int64_t *cells, int64_t n_cells, double scale,
                    double *out);

typedef struct {
    int H, d;
    const uint16_t *q_idx, *pooled;
    int64_t b0, b1;
    double *s64;
    float *s32;
} scan_part;

static void *scan_range(void *arg)
{
    scan_part *p = (scan_part *)arg;
    const int64_t row = (int64_t)p->H * p->d;
    orc_index_score(p->H, p->d, p->q_idx, p->pooled + p->b0 * row, p->b1 - p->b0,
                    p->s64 ? p->s64 + p->b0 : NULL, p->s32 + p->b0);
    return NULL;
}

/* Scores of blocks [0, nb) on up to n_threads threads (contiguous ranges).  A
 * range whose thread cannot be created runs on the calling thread. */
static void scan_threaded(int H, int d, const uint16_t *q_idx, const uint16_t *pooled,
                          int64_t nb, double *s64, float *s32, int n_threads)
{
    if (n_threads < 1)
        n_threads = 1;
    if ((int64_t)n_threads > nb)
        n_threads = nb > 0 ? (int)nb : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    scan_part *part = (scan_part *)malloc(sizeof(scan_part) * (size_t)n_threads);
    char *running = (char *)calloc((size_t)n_threads, 1);
    for (int t = 0; t < n_threads; t++) {
        part[t].H = H;
        part[t].d = d;
        part[t].q_idx = q_idx;
        part[t].pooled = pooled;
        part[t].b0 = nb * t / n_threads;
        part[t].b1 = nb * (t + 1) / n_threads;
        part[t].s64 = s64;
        part[t].s32 = s32;
        if (t > 0 && pthread_create(&tid[t], NULL, scan_range, &part[t]) == 0)
            running[t] = 1;
    }
    for (int t = 0; t < n_threads; t++)
        if (!running[t])
            scan_range(&part[t]);
    for (int t = 1; t < n_threads; t++)
        if (running[t])
            pthread_join(tid[t], NULL);
    free(running);
    free(tid);
    free(part);
}

/* orc_decode_step with the block scan on n_threads threads; same arguments and
 * results (scores64 may be NULL). */
int64_t orc_decode_step_mt(const orc_cfg *cf, uint16_t *raw, uint16_t *pooled, uint16_t *kc,
                           uint16_t *vc, int64_t n_before, const uint16_t *q_idx,
                           const uint16_t *k_idx_new, const uint16_t *q, const uint16_t *k_new,
                           const uint16_t *v_new, const float *rms_w, double *scores64,
                           float *scores32, int32_t *blk, double *out, int n_threads)
{
    orc_pool_append(cf->h_idx, cf->d_idx, k_idx_new, 1, n_before, raw, pooled, cf->rope_base,
                    cf->rms_eps, rms_w);
    memcpy(kc + n_before * (int64_t)cf->hkv * cf->d, k_new,
           sizeof(uint16_t) * (size_t)cf->hkv * cf->d);
    memcpy(vc + n_before * (int64_t)cf->hkv * cf->dv, v_new,
           sizeof(uint16_t) * (size_t)cf->hkv * cf->dv);
    const int64_t n = n_before + 1;
    const int64_t nb = n / ORC_BLOCK;
    scan_threaded(cf->h_idx, cf->d_idx, q_idx, pooled, nb, scores64, scores32, n_threads);
    int64_t n_sel = orc_topk_sort(scores32, nb, cf->topk, blk);
    int64_t *cells = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ORC_BLOCK * n_sel + ORC_BLOCK));
    int64_t nc = orc_cells(blk, n_sel, n, cells);
    orc_attn_cells(cf->hq, cf->hkv, cf->d, cf->dv, q, kc, vc, cells, nc, cf->scale, out);
    free(cells);
    return n_sel;
}
