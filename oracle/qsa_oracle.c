/*
 * QSA layer-step ORACLE -- test infrastructure, not product code.
 *
 * A plain, slow, single-threaded CPU statement of what one QSA (Qwen Sparse
 * Attention) layer step computes, written in fp64 from the sources cited below.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or helper with the HIP
 * path, and the HIP path never calls it.
 *
 * Sources (cited by page and section only):
 *  [Q10]  ariera, Qiita, EVO-X2 + Qwen3.8-Flash-Next llama.cpp series, part 10
 *         (COMMON-004 / COMMON-005 write-up).
 *           "QSAとQSA indexerについて"            -- two-stage QSA, 4-token pooling,
 *                                                   RMS norm, RoPE, score, top-k,
 *                                                   2048 tokens / ratio 4, tail block
 *           "incremental pooled-key cache（COMMON-004）" -- cache completed blocks,
 *                                                   update only new ones
 *           "なぜFlash Attentionがcontext長に比例していたのか" -- 2048+4-1 = 2051 cells
 *           "selected QSA K/V gather（COMMON-005）" -- gather selected K/V, then
 *                                                   ordinary attention over them
 *           "block-domain top-k（COMMON-006）実装は見送り" -- top-k on pool scores,
 *                                                   expand picked pools, add tail
 *  [CDNA] devotd.net news, "llama.cpp opens the sparse-attention path on AMD CDNA",
 *           section 2 -- visible key positions collected from the mask into a list
 *           section 3 -- DKQ 576 variant; mask present, no bias, no softcap
 *
 * Readings where the sources are silent (each is listed with its reason in the
 * design notes): the score is the plain sum over indexer heads of dot products;
 * the RoPE position of block b is 4b (block_pos below); RoPE is the half-split
 * form over the full head dim with angle p * base^(-2i/d); RMS norm is per head
 * over d with eps added to the mean square; ties in top-k go to the lower block
 * id, -0 equals +0, NaN ranks lowest; the attention scale is given by the caller.
 *
 * Parity status: every function below is pinned by CPU tests against closed
 * forms, invariants, brute force or library routines (numpy / scipy).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* IEEE 754 binary16 <-> binary64, written from the format definition:        */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds   */
/* subnormals (fraction * 2^-24), exponent 31 holds inf / NaN.                 */
/* ------------------------------------------------------------------------- */
double orc_h2d(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);
    return sign ? -v : v;
}

/* Round to nearest, ties to even.  Scaling by a power of two is exact in    */
/* binary64, so rint() (default mode: nearest-even) rounds exactly once.     */
uint16_t orc_d2h(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    if (isinf(a))
        return (uint16_t)(sign | 0x7c00);
    if (a == 0.0)
        return sign;
    int E;
    frexp(a, &E);          /* a = m * 2^E with m in [0.5, 1) */
    int u = E - 1;         /* a = 1.f * 2^u                  */
    if (u < -14) {         /* subnormal spacing 2^-24        */
        double r = rint(ldexp(a, 24));
        if (r >= 1024.0)
            return (uint16_t)(sign | 0x0400);
        return (uint16_t)(sign | (uint16_t)r);
    }
    double r = rint(ldexp(a, 10 - u)); /* in [1024, 2048] */
    if (r >= 2048.0) {
        r = 1024.0;
        u += 1;
    }
    if (u > 15)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((u + 15) << 10) | (uint16_t)(r - 1024.0));
}

void orc_h2d_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_h2d(h[i]);
}

void orc_d2h_array(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_d2h(x[i]);
}

/* ------------------------------------------------------------------------- */
/* Indexer side: pooled summary of one 4-token micro-block.  [Q10] "QSAとQSA   */
/* indexerについて": the indexer keys of 4 tokens are average-pooled into one   */
/* summary, which is RMS-normalised and then given its position with RoPE.    */
/* ------------------------------------------------------------------------- */
#define ORC_BLOCK 4

/* Position given to the pooled summary of block b: its first token. */
int64_t orc_block_pos(int64_t b)
{
    return ORC_BLOCK * b;
}

/*
 * raw4: the 4 raw indexer keys of the block, [4][H][d] binary16.
 * w:    RMS-norm weight [d] (NULL means all ones).
 * out:  pooled row [H][d] binary16 (the pooled cache is stored in binary16).
 */
void orc_pool_block(int H, int d, const uint16_t *raw4, int64_t pos, double base,
                    double eps, const float *w, uint16_t *out)
{
    const int64_t row = (int64_t)H * d;
    double *m = (double *)malloc(sizeof(double) * d);
    double *n = (double *)malloc(sizeof(double) * d);
    const int half = d / 2;
    for (int h = 0; h < H; h++) {
        /* mean of the 4 token keys */
        for (int i = 0; i < d; i++) {
            double s = 0.0;
            for (int t = 0; t < ORC_BLOCK; t++)
                s += orc_h2d(raw4[t * row + (int64_t)h * d + i]);
            m[i] = s / ORC_BLOCK;
        }
        /* RMS norm over the head dimension */
        double ss = 0.0;
        for (int i = 0; i < d; i++)
            ss += m[i] * m[i];
        double rms = sqrt(ss / d + eps);
        for (int i = 0; i < d; i++)
            n[i] = m[i] / rms * (w ? (double)w[i] : 1.0);
        /* RoPE: rotate the pair (i, i + d/2) by pos * base^(-2i/d) */
        for (int i = 0; i < half; i++) {
            double theta = (double)pos * pow(base, -2.0 * (double)i / (double)d);
            double c = cos(theta), s = sin(theta);
            double a = n[i], b = n[i + half];
            out[(int64_t)h * d + i] = orc_d2h(a * c - b * s);
            out[(int64_t)h * d + i + half] = orc_d2h(a * s + b * c);
        }
    }
    free(m);
    free(n);
}

/* Old path: rebuild every complete block of the first n_tokens from scratch. */
void orc_pool_rebuild(int H, int d, const uint16_t *raw, int64_t n_tokens, double base,
                      double eps, const float *w, uint16_t *pooled)
{
    const int64_t row = (int64_t)H * d;
    const int64_t nb = n_tokens / ORC_BLOCK;
    for (int64_t b = 0; b < nb; b++)
        orc_pool_block(H, d, raw + b * ORC_BLOCK * row, orc_block_pos(b), base, eps, w,
                       pooled + b * row);
}

/*
 * COMMON-004 path ([Q10] "incremental pooled-key cache"): write the new raw
 * rows at [n_before, n_before + n_new) and compute the pooled row of each block
 * that becomes complete in that range; nothing else is touched.
 */
void orc_pool_append(int H, int d, const uint16_t *k_new, int64_t n_new, int64_t n_before,
                     uint16_t *raw, uint16_t *pooled, double base, double eps, const float *w)
{
    const int64_t row = (int64_t)H * d;
    memcpy(raw + n_before * row, k_new, sizeof(uint16_t) * (size_t)(n_new * row));
    int64_t b_lo = n_before / ORC_BLOCK;
    int64_t b_hi = (n_before + n_new) / ORC_BLOCK;
    for (int64_t b = b_lo; b < b_hi; b++)
        orc_pool_block(H, d, raw + b * ORC_BLOCK * row, orc_block_pos(b), base, eps, w,
                       pooled + b * row);
}

/* Score of every complete block: sum over indexer heads of <q_h, P[b,h]>.  */
void orc_index_score(int H, int d, const uint16_t *q_idx, const uint16_t *pooled, int64_t nb,
                     double *s64, float *s32)
{
    const int64_t row = (int64_t)H * d;
    double *q = (double *)malloc(sizeof(double) * (size_t)row);
    for (int64_t i = 0; i < row; i++)
        q[i] = orc_h2d(q_idx[i]);
    for (int64_t b = 0; b < nb; b++) {
        double s = 0.0;
        for (int64_t i = 0; i < row; i++)
            s += q[i] * orc_h2d(pooled[b * row + i]);
        if (s64)
            s64[b] = s;
        if (s32)
            s32[b] = (float)s;
    }
    free(q);
}

/* ------------------------------------------------------------------------- */
/* Top-k over pool scores, in the block domain ([Q10] COMMON-006 section).    */
/* Order: higher score first; equal scores -> lower block id first; -0 == +0; */
/* NaN below everything.  Output: the chosen block ids in ascending order.    */
/* ------------------------------------------------------------------------- */
typedef struct {
    float s;
    int32_t b;
} orc_sb;

/* <0 when x ranks before y */
static int orc_rank_cmp(float xs, int32_t xb, float ys, int32_t yb)
{
    int xn = isnan(xs), yn = isnan(ys);
    if (xn != yn)
        return xn ? 1 : -1;
    if (!xn) {
        if (xs > ys)
            return -1;
        if (xs < ys)
            return 1;
    }
    return (xb < yb) ? -1 : (xb > yb ? 1 : 0);
}

static int orc_sb_cmp(const void *x, const void *y)
{
    const orc_sb *a = (const orc_sb *)x, *b = (const orc_sb *)y;
    return orc_rank_cmp(a->s, a->b, b->s, b->b);
}

static int orc_i32_cmp(const void *x, const void *y)
{
    int32_t a = *(const int32_t *)x, b = *(const int32_t *)y;
    return (a > b) - (a < b);
}

/* Sort-based selection.  Returns the number selected, min(k, nb). */
int64_t orc_topk_sort(const float *scores, int64_t nb, int64_t k, int32_t *blk)
{
    if (nb <= k) {
        for (int64_t b = 0; b < nb; b++)
            blk[b] = (int32_t)b;
        return nb;
    }
    orc_sb *v = (orc_sb *)malloc(sizeof(orc_sb) * (size_t)nb);
    for (int64_t b = 0; b < nb; b++) {
        v[b].s = scores[b];
        v[b].b = (int32_t)b;
    }
    qsort(v, (size_t)nb, sizeof(orc_sb), orc_sb_cmp);
    for (int64_t j = 0; j < k; j++)
        blk[j] = v[j].b;
    qsort(blk, (size_t)k, sizeof(int32_t), orc_i32_cmp);
    free(v);
    return k;
}

/* Rank-count rule, O(nb^2), for tiny inputs: b is chosen iff fewer than k
 * blocks rank before it. */
int64_t orc_topk_rank(const float *scores, int64_t nb, int64_t k, int32_t *blk)
{
    int64_t c = 0;
    for (int64_t b = 0; b < nb; b++) {
        int64_t before = 0;
        for (int64_t o = 0; o < nb; o++)
            if (o != b && orc_rank_cmp(scores[o], (int32_t)o, scores[b], (int32_t)b) < 0)
                before++;
        if (before < k)
            blk[c++] = (int32_t)b;
    }
    return c;
}

/* Cells attended: the 4 cells of each chosen block, then the incomplete tail
 * block [4*floor(N/4), N) ([Q10] "QSAとQSA indexerについて", COMMON-006 section). */
int64_t orc_cells(const int32_t *blk, int64_t n_sel, int64_t n_tokens, int64_t *cells)
{
    int64_t c = 0;
    for (int64_t j = 0; j < n_sel; j++)
        for (int t = 0; t < ORC_BLOCK; t++)
            cells[c++] = (int64_t)ORC_BLOCK * blk[j] + t;
    for (int64_t t = (n_tokens / ORC_BLOCK) * ORC_BLOCK; t < n_tokens; t++)
        cells[c++] = t;
    return c;
}

/* ------------------------------------------------------------------------- */
/* Attention ([Q10] COMMON-005: ordinary attention over the gathered cells).  */
/* q [hq][d]; caches are token-major [*, hkv, d] and [*, hkv, dv]; query head */
/* h reads kv head h / (hq / hkv).  Output [hq][dv] in fp64.                  */
/* ------------------------------------------------------------------------- */
void orc_attn_cells(int hq, int hkv, int d, int dv, const uint16_t *q, const uint16_t *kc,
                    const uint16_t *vc, const int64_t *cells, int64_t nc, double scale,
                    double *out)
{
    const int G = hq / hkv;
    double *lg = (double *)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
    for (int h = 0; h < hq; h++) {
        const int g = h / G;
        double mx = -INFINITY;
        for (int64_t c = 0; c < nc; c++) {
            const uint16_t *kr = kc + (cells[c] * hkv + g) * (int64_t)d;
            double s = 0.0;
            for (int j = 0; j < d; j++)
                s += orc_h2d(q[(int64_t)h * d + j]) * orc_h2d(kr[j]);
            lg[c] = scale * s;
            if (lg[c] > mx)
                mx = lg[c];
        }
        double den = 0.0;
        for (int64_t c = 0; c < nc; c++) {
            lg[c] = exp(lg[c] - mx);
            den += lg[c];
        }
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int64_t c = 0; c < nc; c++)
                acc += lg[c] * orc_h2d(vc[(cells[c] * hkv + g) * (int64_t)dv + j]);
            out[(int64_t)h * dv + j] = acc / den;
        }
    }
    free(lg);
}

/* The same attention written as the dense masked form: every t < n_tokens,
 * with logit -inf where visible[t] == 0 (the pre-gather path of [Q10]). */
void orc_attn_dense_masked(int hq, int hkv, int d, int dv, const uint16_t *q,
                           const uint16_t *kc, const uint16_t *vc, int64_t n_tokens,
                           const uint8_t *visible, double scale, double *out)
{
    const int G = hq / hkv;
    double *lg = (double *)malloc(sizeof(double) * (size_t)(n_tokens > 0 ? n_tokens : 1));
    for (int h = 0; h < hq; h++) {
        const int g = h / G;
        double mx = -INFINITY;
        for (int64_t t = 0; t < n_tokens; t++) {
            double s = 0.0;
            for (int j = 0; j < d; j++)
                s += orc_h2d(q[(int64_t)h * d + j]) * orc_h2d(kc[(t * hkv + g) * (int64_t)d + j]);
            lg[t] = visible[t] ? scale * s : -INFINITY;
            if (lg[t] > mx)
                mx = lg[t];
        }
        double den = 0.0;
        for (int64_t t = 0; t < n_tokens; t++) {
            lg[t] = exp(lg[t] - mx);
            den += lg[t];
        }
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int64_t t = 0; t < n_tokens; t++)
                acc += lg[t] * orc_h2d(vc[(t * hkv + g) * (int64_t)dv + j]);
            out[(int64_t)h * dv + j] = acc / den;
        }
    }
    free(lg);
}

/* ------------------------------------------------------------------------- */
/* One decode step of one layer, composed from the pieces above:             */
/* append the new token (indexer key, K, V), score the complete blocks,      */
/* pick the top-k on the scores rounded to fp32, add the tail, attend.       */
/* ------------------------------------------------------------------------- */
typedef struct {
    int32_t h_idx, d_idx, topk;
    int32_t hq, hkv, d, dv;
    double rope_base, rms_eps, scale;
} orc_cfg;

int64_t orc_decode_step(const orc_cfg *cf, uint16_t *raw, uint16_t *pooled, uint16_t *kc,
                        uint16_t *vc, int64_t n_before, const uint16_t *q_idx,
                        const uint16_t *k_idx_new, const uint16_t *q, const uint16_t *k_new,
                        const uint16_t *v_new, const float *rms_w, double *scores64,
                        float *scores32, int32_t *blk, double *out)
{
    orc_pool_append(cf->h_idx, cf->d_idx, k_idx_new, 1, n_before, raw, pooled, cf->rope_base,
                    cf->rms_eps, rms_w);
    memcpy(kc + n_before * (int64_t)cf->hkv * cf->d, k_new,
           sizeof(uint16_t) * (size_t)cf->hkv * cf->d);
    memcpy(vc + n_before * (int64_t)cf->hkv * cf->dv, v_new,
           sizeof(uint16_t) * (size_t)cf->hkv * cf->dv);
    const int64_t n = n_before + 1;
    const int64_t nb = n / ORC_BLOCK;
    orc_index_score(cf->h_idx, cf->d_idx, q_idx, pooled, nb, scores64, scores32);
    int64_t n_sel = orc_topk_sort(scores32, nb, cf->topk, blk);
    int64_t *cells = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ORC_BLOCK * n_sel + ORC_BLOCK));
    int64_t nc = orc_cells(blk, n_sel, n, cells);
    orc_attn_cells(cf->hq, cf->hkv, cf->d, cf->dv, q, kc, vc, cells, nc, cf->scale, out);
    free(cells);
    return n_sel;
}

/*
 * One query row of a prefill chunk: the caches already hold every token up to
 * and including position pos; the row sees N = pos + 1 tokens and runs the
 * decode selection and attention on them.
 */
int64_t orc_prefill_row(const orc_cfg *cf, const uint16_t *pooled, const uint16_t *kc,
                        const uint16_t *vc, int64_t pos, const uint16_t *q_idx_row,
                        const uint16_t *q_row, double *scores64, float *scores32, int32_t *blk,
                        double *out)
{
    const int64_t n = pos + 1;
    const int64_t nb = n / ORC_BLOCK;
    orc_index_score(cf->h_idx, cf->d_idx, q_idx_row, pooled, nb, scores64, scores32);
    int64_t n_sel = orc_topk_sort(scores32, nb, cf->topk, blk);
    int64_t *cells = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ORC_BLOCK * n_sel + ORC_BLOCK));
    int64_t nc = orc_cells(blk, n_sel, n, cells);
    orc_attn_cells(cf->hq, cf->hkv, cf->d, cf->dv, q_row, kc, vc, cells, nc, cf->scale, out);
    free(cells);
    return n_sel;
}

/* ------------------------------------------------------------------------- */
/* MLA-style list attention ([CDNA] sections 2-3): the visible positions of  */
/* an additive mask (0 or -inf) are listed in ascending order, then every     */
/* query head attends over those positions of a single shared KV head.       */
/* kv [n][dkq]; the value of position j is v[j][0:dv] if v is given, else     */
/* the first dv entries of kv[j] (the latent part).                          */
/* ------------------------------------------------------------------------- */
int64_t orc_mask_list(const uint16_t *mask, int64_t n, int32_t *list)
{
    int64_t c = 0;
    for (int64_t j = 0; j < n; j++)
        if (orc_h2d(mask[j]) != -INFINITY)
            list[c++] = (int32_t)j;
    return c;
}

static double orc_mla_logit(int dkq, const uint16_t *qh, const uint16_t *kvj, double scale,
                            uint16_t mj)
{
    double s = 0.0;
    for (int i = 0; i < dkq; i++)
        s += orc_h2d(qh[i]) * orc_h2d(kvj[i]);
    return scale * s + orc_h2d(mj);
}

void orc_mla_attn(int hq, int dkq, int dv, const uint16_t *q, const uint16_t *kv,
                  const uint16_t *v, const uint16_t *mask, const int32_t *list, int64_t nl,
                  double scale, double *out)
{
    double *lg = (double *)malloc(sizeof(double) * (size_t)(nl > 0 ? nl : 1));
    for (int h = 0; h < hq; h++) {
        double mx = -INFINITY;
        for (int64_t c = 0; c < nl; c++) {
            int64_t j = list[c];
            lg[c] = orc_mla_logit(dkq, q + (int64_t)h * dkq, kv + j * dkq, scale, mask[j]);
            if (lg[c] > mx)
                mx = lg[c];
        }
        double den = 0.0;
        for (int64_t c = 0; c < nl; c++) {
            lg[c] = exp(lg[c] - mx);
            den += lg[c];
        }
        for (int i = 0; i < dv; i++) {
            double acc = 0.0;
            for (int64_t c = 0; c < nl; c++) {
                int64_t j = list[c];
                double vv = v ? orc_h2d(v[j * dv + i]) : orc_h2d(kv[j * dkq + i]);
                acc += lg[c] * vv;
            }
            out[(int64_t)h * dv + i] = acc / den;
        }
    }
    free(lg);
}

/* Dense form of the same: all n positions, mask added to every logit. */
void orc_mla_dense(int hq, int dkq, int dv, const uint16_t *q, const uint16_t *kv,
                   const uint16_t *v, const uint16_t *mask, int64_t n, double scale, double *out)
{
    double *lg = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int h = 0; h < hq; h++) {
        double mx = -INFINITY;
        for (int64_t j = 0; j < n; j++) {
            lg[j] = orc_mla_logit(dkq, q + (int64_t)h * dkq, kv + j * dkq, scale, mask[j]);
            if (lg[j] > mx)
                mx = lg[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j < n; j++) {
            lg[j] = exp(lg[j] - mx);
            den += lg[j];
        }
        for (int i = 0; i < dv; i++) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; j++) {
                double vv = v ? orc_h2d(v[j * dv + i]) : orc_h2d(kv[j * dkq + i]);
                acc += lg[j] * vv;
            }
            out[(int64_t)h * dv + i] = acc / den;
        }
    }
    free(lg);
}
