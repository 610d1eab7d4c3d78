// C ABI entry points of libqsa: argument checks on the host, workspace layout,
// and the kernel sequences of each call.  Declarations and contracts: qsa.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "qsa.h"
#include "qsa_internal.h"

using namespace qsa;

namespace {

thread_local char g_err[512] = "";
// Events for the calling thread's next decode-step scoring launch (qsa_trace_scan).
thread_local KernelEvents g_scan_events;

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char *where)
{
    return fail(QSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

#define NEED_PTR(p)                                                                  \
    do {                                                                             \
        if (!(p))                                                                    \
            return fail(QSA_ERR_INVALID, "%s: " #p " is NULL", __func__);            \
        if (!aligned16(p))                                                           \
            return fail(QSA_ERR_INVALID, "%s: " #p " is not 16-byte aligned", __func__); \
    } while (0)

#define OPT_PTR(p)                                                                   \
    do {                                                                             \
        if ((p) && !aligned16(p))                                                    \
            return fail(QSA_ERR_INVALID, "%s: " #p " is not 16-byte aligned", __func__); \
    } while (0)

#define HIP_CHECK(expr)                        \
    do {                                       \
        hipError_t e_ = (expr);                \
        if (e_ != hipSuccess)                  \
            return hip_fail(e_, #expr);        \
    } while (0)

int check_cfg(const qsa_config *c)
{
    if (!c)
        return fail(QSA_ERR_INVALID, "config is NULL");
    if (c->block != kBlockTokens)
        return fail(QSA_ERR_UNSUPPORTED, "block must be 4 (got %d)", c->block);
    if (c->h_idx < 1 || c->d_idx < 8 || c->d_idx % 8)
        return fail(QSA_ERR_INVALID, "indexer shape %d x %d", c->h_idx, c->d_idx);
    if (!pow2(c->d_idx / 8) || c->d_idx / 8 > 64)
        return fail(QSA_ERR_UNSUPPORTED, "d_idx/8 must be a power of two <= 64 (d_idx=%d)",
                    c->d_idx);
    const int64_t rowc = (int64_t)c->h_idx * c->d_idx / 8;
    if (!pow2(rowc) || rowc < 16 || rowc > 512)
        return fail(QSA_ERR_UNSUPPORTED, "h_idx*d_idx/8 must be a power of two in [16, 512] (%lld)",
                    (long long)rowc);
    if (c->topk_blocks < 1 || c->topk_blocks > 1024)
        return fail(QSA_ERR_UNSUPPORTED, "topk_blocks must be in [1, 1024] (%d)", c->topk_blocks);
    if (c->hq < 1 || c->hkv < 1 || c->hq % c->hkv)
        return fail(QSA_ERR_INVALID, "heads hq=%d hkv=%d", c->hq, c->hkv);
    const int G = c->hq / c->hkv;
    if (!pow2(G) || G > 16)
        return fail(QSA_ERR_UNSUPPORTED, "hq/hkv must be 1, 2, 4, 8 or 16 (%d)", G);
    if (c->d != c->dv || (c->d != 64 && c->d != 128))
        return fail(QSA_ERR_UNSUPPORTED, "attention head dims d=%d dv=%d (need d == dv in {64,128})",
                    c->d, c->dv);
    if (c->cap_tokens < kBlockTokens || c->cap_tokens % kBlockTokens ||
        c->cap_tokens > kBlockTokens * topk_max_blocks())
        return fail(QSA_ERR_UNSUPPORTED, "cap_tokens must be a multiple of 4 in [4, %d] (%d)",
                    kBlockTokens * topk_max_blocks(), c->cap_tokens);
    if (!(c->rope_base > 0.f) || !(c->rms_eps >= 0.f) || !isfinite(c->attn_scale))
        return fail(QSA_ERR_INVALID, "rope_base/rms_eps/attn_scale out of range");
    return QSA_OK;
}

// Workspace layout: data regions whose sizes depend on (cfg, n_q, n_ctx).  No
// call relies on what a previous call left there.
struct Layout {
    size_t lists, lrows, scores, blk, nsel, part, ksel, vsel, uid, umask, nu, upart, total;
    int64_t ld;  // score row stride
};

int32_t max_cells(const qsa_config *c) { return kBlockTokens * c->topk_blocks + kBlockTokens - 1; }
int32_t max_splits(const qsa_config *c) { return (max_cells(c) + kAttnChunk - 1) / kAttnChunk; }

Layout layout(const qsa_config *c, int32_t n_q, int32_t n_ctx)
{
    Layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    const int64_t nb = (int64_t)n_ctx / kBlockTokens + 1;
    const size_t nd = (size_t)(n_q < kMaxDecodeRows ? n_q : kMaxDecodeRows);  // decode rows
    L.ld = (int64_t)round_up((size_t)nb, 64);
    L.lists = take(sizeof(uint64_t) * nd * kListWgs * kListLen);
    L.lrows = take(sizeof(uint32_t) * nd * kListWgs);
    L.scores = take(sizeof(float) * (size_t)n_q * (size_t)L.ld);
    L.blk = take(sizeof(int32_t) * (size_t)n_q * (size_t)c->topk_blocks);
    L.nsel = take(sizeof(int32_t) * (size_t)n_q);
    L.part = take(sizeof(float) * nd * c->hq * (size_t)max_splits(c) * (size_t)(c->dv + 2));
    L.ksel = take(sizeof(uint16_t) * (size_t)max_cells(c) * c->hkv * c->d);
    L.vsel = take(sizeof(uint16_t) * (size_t)max_cells(c) * c->hkv * c->dv);
    // grouped-union prefill attention: union lists, row masks, partials
    size_t groups = 0, cap_u = 0, usplits = 0;
    if (union_supported(c->hq, c->hkv, c->d, c->dv, c->topk_blocks)) {
        const int32_t G = union_group_rows(c->hq, c->hkv);
        groups = (size_t)(((int64_t)n_q + G - 1) / G);
        cap_u = (size_t)G * c->topk_blocks;
        const int32_t sp = union_splits(n_q, c->hq, c->hkv);
        usplits = sp > 1 ? (size_t)sp : 0;
    }
    L.uid = take(sizeof(int32_t) * groups * cap_u);
    L.umask = take(sizeof(uint32_t) * groups * cap_u);
    L.nu = take(sizeof(int32_t) * groups);
    L.upart = take(sizeof(float) * (size_t)n_q * c->hq * usplits * (size_t)kUnionPartStride);
    L.total = off;
    return L;
}

template <class T>
T *at(void *ws, size_t off)
{
    return (T *)((char *)ws + off);
}

CandLists cand_lists(void *ws, const Layout &L)
{
    return CandLists{at<uint64_t>(ws, L.lists), at<uint32_t>(ws, L.lrows)};
}

int check_ws(const qsa_config *c, void *ws, size_t ws_bytes, int32_t n_q, int32_t n_ctx,
             const char *fn)
{
    if (!ws)
        return fail(QSA_ERR_INVALID, "%s: workspace is NULL", fn);
    if (!aligned16(ws))
        return fail(QSA_ERR_INVALID, "%s: workspace is not 16-byte aligned", fn);
    const size_t need = layout(c, n_q, n_ctx).total;
    if (ws_bytes < need)
        return fail(QSA_ERR_CAPACITY, "%s: workspace has %zu bytes, needs %zu", fn, ws_bytes, need);
    return QSA_OK;
}

const h16 *H(const uint16_t *p) { return (const h16 *)p; }
h16 *H(uint16_t *p) { return (h16 *)p; }

AttnArgs attn_base(const qsa_config *c)
{
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.hq = c->hq;
    a.hkv = c->hkv;
    a.k_tok = (int64_t)c->hkv * c->d;
    a.v_tok = (int64_t)c->hkv * c->dv;
    a.topk = c->topk_blocks;
    a.scale = c->attn_scale;
    a.rows = 1;
    return a;
}

// Splits of a cell range for split-K attention: each work group walks
// kAttnChunksPerSplit 64-cell chunks (the next chunk's loads overlap the current
// chunk's math), more if that would exceed kAttnMaxSplits work groups per
// (row, KV head).  Fewer splits keep the final merge small.
void split_plan(int32_t cells, int32_t *splits, int32_t *chunks)
{
    const int32_t nch = cells > 0 ? (cells + kAttnChunk - 1) / kAttnChunk : 1;
    int32_t c = kAttnChunksPerSplit;
    const int32_t cmin = (nch + kAttnMaxSplits - 1) / kAttnMaxSplits;
    if (c < cmin)
        c = cmin;
    if (c > nch)
        c = nch;
    *chunks = c;
    *splits = (nch + c - 1) / c;
}

int attn_decode_launch(const qsa_config *c, AttnArgs a, int32_t cells, void *ws, const Layout &L,
                       hipStream_t s)
{
    split_plan(cells, &a.splits, &a.chunks);
    a.part = at<float>(ws, L.part);
    HIP_CHECK(launch_attn(a, c->d, c->dv, s));
    return QSA_OK;
}

// One or more decode query rows (the tokens at n_before .. n_before + n_q - 1).
int decode_impl(const char *fn, const qsa_config *cfg, const qsa_layer_bufs *Lb, int32_t n_before,
                int32_t n_q, const uint16_t *q_idx, const uint16_t *k_idx_new, const uint16_t *q,
                const uint16_t *k_new, const uint16_t *v_new, float *out, float *scores_out,
                int32_t ld_scores, int32_t *blk_out, uint32_t flags, void *ws, size_t ws_bytes,
                qsa_stream_t stream)
{
    // the events set by qsa_trace_scan are for this call only, whatever it returns
    const KernelEvents ev = g_scan_events;
    g_scan_events = KernelEvents{};
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (!Lb)
        return fail(QSA_ERR_INVALID, "%s: layer buffers are NULL", fn);
    if (n_before < 0)
        return fail(QSA_ERR_INVALID, "%s: n_before=%d", fn, n_before);
    if (n_q < 1 || n_q > kMaxDecodeRows)
        return fail(QSA_ERR_INVALID, "%s: n_q=%d outside [1, %d]", fn, n_q, kMaxDecodeRows);
    if ((int64_t)n_before + n_q > cfg->cap_tokens)
        return fail(QSA_ERR_CAPACITY, "%s: position %d beyond cap_tokens %d", fn,
                    n_before + n_q - 1, cfg->cap_tokens);
    if (flags > QSA_STEP_COMPACT_GATHER)
        return fail(QSA_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
    if (flags == QSA_STEP_COMPACT_GATHER && n_q != 1)
        return fail(QSA_ERR_UNSUPPORTED, "%s: the compact gather takes one query row", fn);
    NEED_PTR(Lb->k_raw);
    NEED_PTR(Lb->k_pool);
    NEED_PTR(Lb->k_cache);
    NEED_PTR(Lb->v_cache);
    OPT_PTR(Lb->rms_w);
    NEED_PTR(q_idx);
    NEED_PTR(k_idx_new);
    NEED_PTR(q);
    NEED_PTR(k_new);
    NEED_PTR(v_new);
    NEED_PTR(out);
    OPT_PTR(scores_out);
    OPT_PTR(blk_out);
    const int32_t N = n_before + n_q;  // tokens seen by the last row
    const int32_t nb = N / kBlockTokens;
    if (scores_out && n_q > 1 && ld_scores < nb)
        return fail(QSA_ERR_INVALID, "%s: ld_scores %d < %d blocks", fn, ld_scores, nb);
    if ((r = check_ws(cfg, ws, ws_bytes, n_q, N, fn)))
        return r;
    const Layout L = layout(cfg, n_q, N);
    hipStream_t s = (hipStream_t)stream;

    const int64_t row = (int64_t)cfg->h_idx * cfg->d_idx;
    const int64_t kr = (int64_t)cfg->hkv * cfg->d, vr = (int64_t)cfg->hkv * cfg->dv;
    const int32_t k = cfg->topk_blocks;

    // 1. append: raw indexer rows, K rows, V rows, pooled row of the block completed
    // (at most one for up to 4 new tokens)
    AppendArgs ap;
    memset(&ap, 0, sizeof(ap));
    ap.seg[0] = CopySeg{k_idx_new, Lb->k_raw + n_before * row, n_q * row / 8};
    ap.seg[1] = CopySeg{k_new, Lb->k_cache + n_before * kr, n_q * kr / 8};
    ap.seg[2] = CopySeg{v_new, Lb->v_cache + n_before * vr, n_q * vr / 8};
    ap.k_new = H(k_idx_new);
    ap.n_before = n_before;
    ap.k_raw = H(Lb->k_raw);
    ap.k_pool = H(Lb->k_pool);
    ap.rms_w = Lb->rms_w;
    ap.H = cfg->h_idx;
    ap.d = cfg->d_idx;
    ap.b_lo = n_before / kBlockTokens;
    ap.n_blocks = nb - ap.b_lo;
    ap.eps = cfg->rms_eps;
    ap.base = cfg->rope_base;

    // 2. scores of every query row over the blocks complete before the call; the
    // append runs in the same launch and scores the block it completes.  Every
    // scan work group leaves its best kListLen candidates per query row
    float *scores = scores_out ? scores_out : at<float>(ws, L.scores);
    const int32_t ld = scores_out ? (n_q > 1 ? ld_scores : 0) : (int32_t)L.ld;
    const CandLists cl = cand_lists(ws, L);
    int32_t n_lists = 0;
    HIP_CHECK(launch_score_decode(H(q_idx), n_q, H(Lb->k_pool), ap.b_lo, (int32_t)row, scores, ld,
                                  &ap, &cl, &n_lists, s, ev));

    if (flags == QSA_STEP_FUSED_GATHER) {
        // 3-5. top-k from the candidate lists and attention over the chosen
        // cells (read straight from the caches) in one launch, then the combine
        StepTail st;
        st.cl = cl;
        st.n_lists = n_lists;
        st.scores = scores;
        st.ld = ld;
        st.pos0 = n_before;
        st.rows = n_q;
        st.k = k;
        st.q = H(q);
        st.k_cache = H(Lb->k_cache);
        st.v_cache = H(Lb->v_cache);
        st.hq = cfg->hq;
        st.hkv = cfg->hkv;
        st.d = cfg->d;
        st.dv = cfg->dv;
        st.scale = cfg->attn_scale;
        st.part = at<float>(ws, L.part);
        st.out = out;
        st.blk_out = blk_out;
        st.scan_rpw = scan_rows_per_group((int32_t)row);
        HIP_CHECK(launch_step_tail(st, s));
        return QSA_OK;
    }

    // 3. top-k blocks (ascending ids) from the candidate lists
    const int32_t nsel = nb < k ? nb : k;
    const int32_t cells = kBlockTokens * nsel + N % kBlockTokens;
    int32_t *blk = blk_out ? blk_out : at<int32_t>(ws, L.blk);
    HIP_CHECK(launch_topk_lists(scores, nb, k, cl, n_lists, blk, at<int32_t>(ws, L.nsel), s,
                                scan_rows_per_group((int32_t)row), ap.b_lo));

    // 4-5. compact gather, then attention over the compact rows
    AttnArgs a = attn_base(cfg);
    a.q = H(q);
    a.out = out;
    h16 *ks = at<h16>(ws, L.ksel), *vs = at<h16>(ws, L.vsel);
    HIP_CHECK(launch_gather(blk, nsel, N, H(Lb->k_cache), H(Lb->v_cache), (int32_t)(kr / 8),
                            (int32_t)(vr / 8), ks, vs, s));
    a.kbase = ks;
    a.vbase = vs;
    a.mode = kCellsCompact;
    a.n_cells = cells;
    return attn_decode_launch(cfg, a, cells, ws, L, s);
}

// Scratch of qsa_decode_step_noalloc: one array per GPU, in the library's code
// object, kept until the process ends.  Host code never uses the array's name as
// an address (on the host it stands in for the symbol only); the device address
// comes from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = QSA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`; the stream must belong to that device.
int static_scratch(hipStream_t stream, void **out, const char *fn)
{
    int dev = -1;
    HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(QSA_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn,
                    dev, kMaxDevices);
    if (stream) {
        hipDevice_t sd = -1;
        HIP_CHECK(hipStreamGetDevice(stream, &sd));
        if (sd != dev)
            return fail(QSA_ERR_INVALID, "%s: the stream belongs to device %d, device %d is current",
                        fn, (int)sd, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || !aligned16(p))
            return fail(QSA_ERR_HIP, "%s: no usable address for the scratch array", fn);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QSA_OK;
}

}  // namespace

extern "C" {

const char *qsa_status_string(int status)
{
    switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_INVALID: return "invalid argument";
    case QSA_ERR_CAPACITY: return "capacity exceeded";
    case QSA_ERR_UNSUPPORTED: return "unsupported shape or precondition";
    case QSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *qsa_last_error(void) { return g_err; }

int qsa_config_check(const qsa_config *cfg)
{
    const int r = check_cfg(cfg);
    if (r == QSA_OK)
        g_err[0] = 0;
    return r;
}

size_t qsa_workspace_size(const qsa_config *cfg, int32_t n_q, int32_t n_ctx)
{
    if (check_cfg(cfg) != QSA_OK || n_q < 1 || n_ctx < 0 || n_ctx > cfg->cap_tokens)
        return 0;
    return layout(cfg, n_q, n_ctx).total;
}

int qsa_workspace_init(void *ws, size_t ws_bytes, qsa_stream_t stream)
{
    NEED_PTR(ws);
    if (ws_bytes % 16)
        return fail(QSA_ERR_INVALID, "workspace size must be a multiple of 16");
    HIP_CHECK(launch_fill_zero(ws, ws_bytes, (hipStream_t)stream));
    return QSA_OK;
}

int qsa_pool_append(const qsa_config *cfg, const uint16_t *k_new, int32_t n_new, int32_t n_before,
                    uint16_t *k_raw, uint16_t *k_pool, const float *rms_w, qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_new < 0 || n_before < 0)
        return fail(QSA_ERR_INVALID, "qsa_pool_append: n_new=%d n_before=%d", n_new, n_before);
    if ((int64_t)n_before + n_new > cfg->cap_tokens)
        return fail(QSA_ERR_CAPACITY, "qsa_pool_append: %d + %d tokens exceed cap_tokens %d",
                    n_before, n_new, cfg->cap_tokens);
    if (n_new == 0)
        return QSA_OK;
    NEED_PTR(k_new);
    NEED_PTR(k_raw);
    NEED_PTR(k_pool);
    OPT_PTR(rms_w);
    const int64_t row = (int64_t)cfg->h_idx * cfg->d_idx;
    AppendArgs a;
    memset(&a, 0, sizeof(a));
    a.seg[0] = CopySeg{k_new, k_raw + n_before * row, (int64_t)n_new * row / 8};
    a.k_new = H(k_new);
    a.n_before = n_before;
    a.k_raw = H(k_raw);
    a.k_pool = H(k_pool);
    a.rms_w = rms_w;
    a.H = cfg->h_idx;
    a.d = cfg->d_idx;
    a.b_lo = n_before / kBlockTokens;
    a.n_blocks = (n_before + n_new) / kBlockTokens - a.b_lo;
    a.eps = cfg->rms_eps;
    a.base = cfg->rope_base;
    HIP_CHECK(launch_append(a, (hipStream_t)stream));
    return QSA_OK;
}

int qsa_pool_rebuild(const qsa_config *cfg, const uint16_t *k_raw, uint16_t *k_pool,
                     const float *rms_w, int32_t b_from, int32_t n_tokens, qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_tokens < 0 || n_tokens > cfg->cap_tokens)
        return fail(QSA_ERR_INVALID, "qsa_pool_rebuild: n_tokens=%d outside [0, %d]", n_tokens,
                    cfg->cap_tokens);
    const int32_t nb = n_tokens / kBlockTokens;
    if (b_from < 0 || b_from > nb)
        return fail(QSA_ERR_INVALID, "qsa_pool_rebuild: b_from=%d outside [0, %d]", b_from, nb);
    if (b_from == nb)
        return QSA_OK;
    NEED_PTR(k_raw);
    NEED_PTR(k_pool);
    OPT_PTR(rms_w);
    // the append's pooling with every token taken from k_raw and nothing copied
    AppendArgs a;
    memset(&a, 0, sizeof(a));
    a.k_new = H(k_raw);
    a.n_before = n_tokens;
    a.k_raw = H(const_cast<uint16_t *>(k_raw));
    a.k_pool = H(k_pool);
    a.rms_w = rms_w;
    a.H = cfg->h_idx;
    a.d = cfg->d_idx;
    a.b_lo = b_from;
    a.n_blocks = nb - b_from;
    a.eps = cfg->rms_eps;
    a.base = cfg->rope_base;
    HIP_CHECK(launch_append(a, (hipStream_t)stream));
    return QSA_OK;
}

int qsa_kv_append(const qsa_config *cfg, const uint16_t *k_new, const uint16_t *v_new,
                  int32_t n_new, int32_t n_before, uint16_t *k_cache, uint16_t *v_cache,
                  qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_new < 0 || n_before < 0)
        return fail(QSA_ERR_INVALID, "qsa_kv_append: n_new=%d n_before=%d", n_new, n_before);
    if ((int64_t)n_before + n_new > cfg->cap_tokens)
        return fail(QSA_ERR_CAPACITY, "qsa_kv_append: %d + %d tokens exceed cap_tokens %d",
                    n_before, n_new, cfg->cap_tokens);
    if (n_new == 0)
        return QSA_OK;
    NEED_PTR(k_new);
    NEED_PTR(v_new);
    NEED_PTR(k_cache);
    NEED_PTR(v_cache);
    const int64_t kr = (int64_t)cfg->hkv * cfg->d, vr = (int64_t)cfg->hkv * cfg->dv;
    AppendArgs a;
    memset(&a, 0, sizeof(a));
    a.seg[1] = CopySeg{k_new, k_cache + n_before * kr, (int64_t)n_new * kr / 8};
    a.seg[2] = CopySeg{v_new, v_cache + n_before * vr, (int64_t)n_new * vr / 8};
    a.H = cfg->h_idx;
    a.d = cfg->d_idx;
    HIP_CHECK(launch_append(a, (hipStream_t)stream));
    return QSA_OK;
}

int qsa_index_score(const qsa_config *cfg, const uint16_t *q_idx, int32_t n_q, int32_t pos0,
                    const uint16_t *k_pool, float *scores, int32_t ld, qsa_stream_t stream)
{
    // the events set by qsa_trace_scan are for this call only, whatever it returns
    const KernelEvents ev = g_scan_events;
    g_scan_events = KernelEvents{};
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_q < 1 || pos0 < 0)
        return fail(QSA_ERR_INVALID, "qsa_index_score: n_q=%d pos0=%d", n_q, pos0);
    if ((int64_t)pos0 + n_q > cfg->cap_tokens)
        return fail(QSA_ERR_CAPACITY, "qsa_index_score: rows reach past cap_tokens");
    const int32_t nb_last = (pos0 + n_q) / kBlockTokens;
    if (ld < nb_last)
        return fail(QSA_ERR_INVALID, "qsa_index_score: ld %d < %d blocks", ld, nb_last);
    NEED_PTR(q_idx);
    NEED_PTR(k_pool);
    NEED_PTR(scores);
    const int32_t row = cfg->h_idx * cfg->d_idx;
    if (n_q == 1) {
        HIP_CHECK(launch_score_decode(H(q_idx), 1, H(k_pool), (pos0 + 1) / kBlockTokens, row,
                                      scores, 0, nullptr, nullptr, nullptr, (hipStream_t)stream,
                                      ev));
        return QSA_OK;
    }
    if (ld % 4)
        return fail(QSA_ERR_INVALID, "qsa_index_score: ld must be a multiple of 4 for n_q > 1");
    HIP_CHECK(launch_score_prefill(H(q_idx), n_q, pos0, H(k_pool), row, scores, ld,
                                   (hipStream_t)stream, ev));
    return QSA_OK;
}

int qsa_topk_blocks(const qsa_config *cfg, const float *scores, int32_t n_q, int32_t ld,
                    int32_t pos0, int32_t *blk, int32_t *n_sel, void *ws, size_t ws_bytes,
                    qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_q < 1 || pos0 < 0)
        return fail(QSA_ERR_INVALID, "qsa_topk_blocks: n_q=%d pos0=%d", n_q, pos0);
    if ((int64_t)pos0 + n_q > cfg->cap_tokens)
        return fail(QSA_ERR_CAPACITY, "qsa_topk_blocks: rows reach past cap_tokens");
    if (ld < (pos0 + n_q) / kBlockTokens)
        return fail(QSA_ERR_INVALID, "qsa_topk_blocks: ld %d too small", ld);
    NEED_PTR(scores);
    NEED_PTR(blk);
    NEED_PTR(n_sel);
    hipStream_t s = (hipStream_t)stream;
    if (n_q == 1) {
        if ((r = check_ws(cfg, ws, ws_bytes, 1, pos0 + 1, __func__)))
            return r;
        const Layout L = layout(cfg, 1, pos0 + 1);
        HIP_CHECK(launch_topk_decode(scores, (pos0 + 1) / kBlockTokens, cfg->topk_blocks, blk,
                                     n_sel, cand_lists(ws, L), s));
        return QSA_OK;
    }
    HIP_CHECK(launch_topk_rows(scores, n_q, ld, pos0, cfg->topk_blocks, blk, n_sel, s));
    return QSA_OK;
}

int qsa_gather_kv(const qsa_config *cfg, const int32_t *blk, int32_t n_blk, int32_t n_tokens,
                  const uint16_t *k_cache, const uint16_t *v_cache, uint16_t *k_sel,
                  uint16_t *v_sel, qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_tokens < 0 || n_tokens > cfg->cap_tokens)
        return fail(QSA_ERR_INVALID, "qsa_gather_kv: n_tokens=%d", n_tokens);
    const int32_t nb = n_tokens / kBlockTokens;
    const int32_t want = nb < cfg->topk_blocks ? nb : cfg->topk_blocks;
    if (n_blk != want)
        return fail(QSA_ERR_INVALID, "qsa_gather_kv: n_blk=%d, expected min(k, nb)=%d", n_blk, want);
    if (n_blk > 0)
        NEED_PTR(blk);
    NEED_PTR(k_cache);
    NEED_PTR(v_cache);
    NEED_PTR(k_sel);
    NEED_PTR(v_sel);
    HIP_CHECK(launch_gather(blk, n_blk, n_tokens, H(k_cache), H(v_cache),
                            cfg->hkv * cfg->d / 8, cfg->hkv * cfg->dv / 8, H(k_sel), H(v_sel),
                            (hipStream_t)stream));
    return QSA_OK;
}

int qsa_sparse_attn(const qsa_config *cfg, const uint16_t *q, const uint16_t *k_sel,
                    const uint16_t *v_sel, int32_t n_cells, float *out, void *ws, size_t ws_bytes,
                    qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_cells < 1 || n_cells > max_cells(cfg))
        return fail(QSA_ERR_INVALID, "qsa_sparse_attn: n_cells=%d outside [1, %d]", n_cells,
                    max_cells(cfg));
    NEED_PTR(q);
    NEED_PTR(k_sel);
    NEED_PTR(v_sel);
    NEED_PTR(out);
    if ((r = check_ws(cfg, ws, ws_bytes, 1, 0, __func__)))
        return r;
    const Layout L = layout(cfg, 1, 0);
    AttnArgs a = attn_base(cfg);
    a.q = H(q);
    a.kbase = H(k_sel);
    a.vbase = H(v_sel);
    a.mode = kCellsCompact;
    a.n_cells = n_cells;
    a.out = out;
    return attn_decode_launch(cfg, a, n_cells, ws, L, (hipStream_t)stream);
}

// Attention of a prefill chunk over each row's chosen blocks and tail: per row, or
// (QSA_PREFILL_GROUPED_UNION) per group of rows over the union of their blocks.
static hipError_t prefill_attn_launch(const qsa_config *cfg, const h16 *q, int32_t n_q, int32_t pos0,
                               const int32_t *blk, int32_t ldb, const h16 *kc, const h16 *vc,
                               float *out, uint32_t flags, void *ws, const Layout &L,
                               hipStream_t s)
{
    if (flags & QSA_PREFILL_GROUPED_UNION) {
        UnionArgs u;
        u.q = q;
        u.blk = blk;
        u.ldb = ldb;
        u.k_cache = kc;
        u.v_cache = vc;
        u.n_q = n_q;
        u.pos0 = pos0;
        u.k = cfg->topk_blocks;
        u.hq = cfg->hq;
        u.hkv = cfg->hkv;
        u.scale = cfg->attn_scale;
        u.splits = union_splits(n_q, cfg->hq, cfg->hkv);
        // the union for every group when asked, or when the per-row kernel cannot
        // take this shape
        const bool rows_ok = rows_supported(cfg->hq, cfg->hkv, cfg->d, cfg->dv,
                                            cfg->topk_blocks, (int64_t)pos0 + n_q);
        u.u_limit = ((flags & QSA_PREFILL_UNION_ALL) || !rows_ok)
                        ? INT32_MAX
                        : union_limit(cfg->hq, cfg->hkv, cfg->topk_blocks);
        u.uid = at<int32_t>(ws, L.uid);
        u.umask = at<uint32_t>(ws, L.umask);
        u.n_u = at<int32_t>(ws, L.nu);
        u.part = at<float>(ws, L.upart);
        u.out = out;
        return launch_union_attn(u, s);
    }
    if (rows_supported(cfg->hq, cfg->hkv, cfg->d, cfg->dv, cfg->topk_blocks,
                       (int64_t)pos0 + n_q)) {
        RowsArgs ra;
        ra.q = q;
        ra.blk = blk;
        ra.ldb = ldb;
        ra.k_cache = kc;
        ra.v_cache = vc;
        ra.n_q = n_q;
        ra.pos0 = pos0;
        ra.k = cfg->topk_blocks;
        ra.hq = cfg->hq;
        ra.hkv = cfg->hkv;
        ra.scale = cfg->attn_scale;
        ra.out = out;
        ra.n_u = nullptr;
        ra.group_rows = 1;
        ra.u_limit = 0;
        ra.part = nullptr;
        ra.splits = 0;
        return launch_rows_attn(ra, s);
    }
    AttnArgs a = attn_base(cfg);
    a.q = q;
    a.kbase = kc;
    a.vbase = vc;
    a.mode = kCellsBlocks;
    a.blk = blk;
    a.ldb = ldb;
    a.pos0 = pos0;
    a.rows = n_q;
    a.splits = 1;
    a.chunks = max_splits(cfg);
    a.out = out;
    return launch_attn(a, cfg->d, cfg->dv, s);
}

static int check_prefill_flags(const qsa_config *cfg, uint32_t flags, const char *fn)
{
    if (flags & ~(QSA_PREFILL_GROUPED_UNION | QSA_PREFILL_UNION_ALL))
        return fail(QSA_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
    if ((flags & QSA_PREFILL_UNION_ALL) && !(flags & QSA_PREFILL_GROUPED_UNION))
        return fail(QSA_ERR_INVALID, "%s: QSA_PREFILL_UNION_ALL needs QSA_PREFILL_GROUPED_UNION",
                    fn);
    if ((flags & QSA_PREFILL_GROUPED_UNION) &&
        !union_supported(cfg->hq, cfg->hkv, cfg->d, cfg->dv, cfg->topk_blocks))
        return fail(QSA_ERR_UNSUPPORTED,
                    "%s: grouped union needs hq/hkv in {4, 8, 16}, d = dv = 128 and "
                    "(128 / (hq/hkv)) * topk_blocks <= %d", fn, kUnionCap);
    return QSA_OK;
}

int qsa_prefill_attn(const qsa_config *cfg, const uint16_t *q, int32_t n_q, int32_t pos0,
                     const int32_t *blk, int32_t ldb, const uint16_t *k_cache,
                     const uint16_t *v_cache, float *out, uint32_t flags, void *ws,
                     size_t ws_bytes, qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_q < 1 || pos0 < 0 || ldb < cfg->topk_blocks)
        return fail(QSA_ERR_INVALID, "qsa_prefill_attn: n_q=%d pos0=%d ldb=%d", n_q, pos0, ldb);
    if ((int64_t)pos0 + n_q > cfg->cap_tokens)
        return fail(QSA_ERR_CAPACITY, "qsa_prefill_attn: rows reach past cap_tokens");
    NEED_PTR(q);
    NEED_PTR(blk);
    NEED_PTR(k_cache);
    NEED_PTR(v_cache);
    NEED_PTR(out);
    if ((r = check_prefill_flags(cfg, flags, __func__)))
        return r;
    // the per-row form needs no workspace
    const bool uni = (flags & QSA_PREFILL_GROUPED_UNION) != 0;
    if (uni && (r = check_ws(cfg, ws, ws_bytes, n_q, pos0 + n_q, __func__)))
        return r;
    const Layout L = layout(cfg, n_q, pos0 + n_q);
    HIP_CHECK(prefill_attn_launch(cfg, H(q), n_q, pos0, blk, ldb, H(k_cache), H(v_cache), out,
                                  flags, ws, L, (hipStream_t)stream));
    return QSA_OK;
}

int qsa_decode_step(const qsa_config *cfg, const qsa_layer_bufs *Lb, int32_t n_before,
                    const uint16_t *q_idx, const uint16_t *k_idx_new, const uint16_t *q,
                    const uint16_t *k_new, const uint16_t *v_new, float *out, float *scores_out,
                    int32_t *blk_out, uint32_t flags, void *ws, size_t ws_bytes,
                    qsa_stream_t stream)
{
    return decode_impl(__func__, cfg, Lb, n_before, 1, q_idx, k_idx_new, q, k_new, v_new, out,
                       scores_out, 0, blk_out, flags, ws, ws_bytes, stream);
}

int qsa_decode_step_noalloc(const qsa_config *cfg, const qsa_layer_bufs *Lb, int32_t n_before,
                            const uint16_t *q_idx, const uint16_t *k_idx_new, const uint16_t *q,
                            const uint16_t *k_new, const uint16_t *v_new, float *out,
                            float *scores_out, int32_t *blk_out, uint32_t flags,
                            qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (n_before < 0 || n_before >= cfg->cap_tokens)
        return fail(n_before < 0 ? QSA_ERR_INVALID : QSA_ERR_CAPACITY,
                    "qsa_decode_step_noalloc: n_before=%d outside [0, %d)", n_before,
                    cfg->cap_tokens);
    const size_t need = layout(cfg, 1, n_before + 1).total;
    if (need > kStaticScratchBytes)
        return fail(QSA_ERR_CAPACITY,
                    "qsa_decode_step_noalloc: this shape needs %zu bytes of scratch, the "
                    "library's static scratch holds %zu (use qsa_decode_step)",
                    need, kStaticScratchBytes);
    void *ws = nullptr;
    if ((r = static_scratch((hipStream_t)stream, &ws, __func__)))
        return r;
    return decode_impl(__func__, cfg, Lb, n_before, 1, q_idx, k_idx_new, q, k_new, v_new, out,
                       scores_out, 0, blk_out, flags, ws, kStaticScratchBytes, stream);
}

int qsa_decode_multi(const qsa_config *cfg, const qsa_layer_bufs *Lb, int32_t n_before,
                     int32_t n_q, const uint16_t *q_idx, const uint16_t *k_idx_new,
                     const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, float *out,
                     float *scores_out, int32_t ld_scores, int32_t *blk_out, void *ws,
                     size_t ws_bytes, qsa_stream_t stream)
{
    return decode_impl(__func__, cfg, Lb, n_before, n_q, q_idx, k_idx_new, q, k_new, v_new, out,
                       scores_out, ld_scores, blk_out, QSA_STEP_FUSED_GATHER, ws, ws_bytes,
                       stream);
}

int qsa_prefill_step(const qsa_config *cfg, const qsa_layer_bufs *Lb, int32_t n_before,
                     int32_t n_new, const uint16_t *q_idx, const uint16_t *k_idx_new,
                     const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, float *out,
                     float *scores_out, int32_t ld_scores, int32_t *blk_out, uint32_t flags,
                     void *ws, size_t ws_bytes, qsa_stream_t stream)
{
    int r = check_cfg(cfg);
    if (r)
        return r;
    if (!Lb)
        return fail(QSA_ERR_INVALID, "qsa_prefill_step: layer buffers are NULL");
    if ((r = check_prefill_flags(cfg, flags, __func__)))
        return r;
    if (n_before < 0 || n_new < 1)
        return fail(QSA_ERR_INVALID, "qsa_prefill_step: n_before=%d n_new=%d", n_before, n_new);
    if ((int64_t)n_before + n_new > cfg->cap_tokens)
        return fail(QSA_ERR_CAPACITY, "qsa_prefill_step: %d + %d tokens exceed cap_tokens %d",
                    n_before, n_new, cfg->cap_tokens);
    NEED_PTR(Lb->k_raw);
    NEED_PTR(Lb->k_pool);
    NEED_PTR(Lb->k_cache);
    NEED_PTR(Lb->v_cache);
    OPT_PTR(Lb->rms_w);
    NEED_PTR(q_idx);
    NEED_PTR(k_idx_new);
    NEED_PTR(q);
    NEED_PTR(k_new);
    NEED_PTR(v_new);
    NEED_PTR(out);
    OPT_PTR(scores_out);
    OPT_PTR(blk_out);
    const int32_t n_end = n_before + n_new;
    if ((r = check_ws(cfg, ws, ws_bytes, n_new, n_end, __func__)))
        return r;
    const Layout L = layout(cfg, n_new, n_end);
    if (scores_out && ld_scores < (int32_t)L.ld)
        return fail(QSA_ERR_INVALID, "qsa_prefill_step: ld_scores %d < %lld", ld_scores,
                    (long long)L.ld);
    hipStream_t s = (hipStream_t)stream;
    const int64_t row = (int64_t)cfg->h_idx * cfg->d_idx;
    const int64_t kr = (int64_t)cfg->hkv * cfg->d, vr = (int64_t)cfg->hkv * cfg->dv;

    AppendArgs ap;
    memset(&ap, 0, sizeof(ap));
    ap.seg[0] = CopySeg{k_idx_new, Lb->k_raw + n_before * row, (int64_t)n_new * row / 8};
    ap.seg[1] = CopySeg{k_new, Lb->k_cache + n_before * kr, (int64_t)n_new * kr / 8};
    ap.seg[2] = CopySeg{v_new, Lb->v_cache + n_before * vr, (int64_t)n_new * vr / 8};
    ap.k_new = H(k_idx_new);
    ap.n_before = n_before;
    ap.k_raw = H(Lb->k_raw);
    ap.k_pool = H(Lb->k_pool);
    ap.rms_w = Lb->rms_w;
    ap.H = cfg->h_idx;
    ap.d = cfg->d_idx;
    ap.b_lo = n_before / kBlockTokens;
    ap.n_blocks = n_end / kBlockTokens - ap.b_lo;
    ap.eps = cfg->rms_eps;
    ap.base = cfg->rope_base;
    HIP_CHECK(launch_append(ap, s));

    float *scores = scores_out ? scores_out : at<float>(ws, L.scores);
    const int32_t ld = scores_out ? ld_scores : (int32_t)L.ld;
    HIP_CHECK(launch_score_prefill(H(q_idx), n_new, n_before, H(Lb->k_pool), (int32_t)row, scores,
                                   ld, s));
    int32_t *blk = blk_out ? blk_out : at<int32_t>(ws, L.blk);
    HIP_CHECK(launch_topk_rows(scores, n_new, ld, n_before, cfg->topk_blocks, blk,
                               at<int32_t>(ws, L.nsel), s));
    HIP_CHECK(prefill_attn_launch(cfg, H(q), n_new, n_before, blk, cfg->topk_blocks,
                                  H(Lb->k_cache), H(Lb->v_cache), out, flags, ws, L, s));
    return QSA_OK;
}

size_t qsa_mla_workspace_size(int32_t hq, int32_t dv, int32_t list_cap)
{
    if (hq < 1 || dv < 1 || list_cap < 1)
        return 0;
    const size_t splits = ((size_t)list_cap + kAttnChunk - 1) / kAttnChunk;
    size_t off = round_up(sizeof(uint32_t) * kListSegMax, 256);  // segment counts
    off += round_up(sizeof(int32_t) * (size_t)list_cap, 256);  // list
    off += round_up(sizeof(float) * (size_t)hq * splits * (size_t)(dv + 2), 256);
    return off;
}

int qsa_mla_sparse_attn(const uint16_t *q, int32_t hq, const uint16_t *kv, const uint16_t *v,
                        int32_t dkq, int32_t dv, const uint16_t *mask, int32_t n, int32_t list_cap,
                        float scale, int32_t *list_out, int32_t *n_list, float *out, void *ws,
                        size_t ws_bytes, qsa_stream_t stream)
{
    if (!mask)
        return fail(QSA_ERR_UNSUPPORTED, "qsa_mla_sparse_attn: no mask (use dense attention)");
    if (n < 4096 || list_cap < 1 || (int64_t)n < 2 * (int64_t)list_cap)
        return fail(QSA_ERR_UNSUPPORTED,
                    "qsa_mla_sparse_attn: needs n >= 4096 and n >= 2*list_cap (n=%d cap=%d)", n,
                    list_cap);
    if (dkq != 576 || dv != 512)
        return fail(QSA_ERR_UNSUPPORTED, "qsa_mla_sparse_attn: implemented for dkq=576, dv=512");
    if (!pow2(hq) || hq > 16)
        return fail(QSA_ERR_UNSUPPORTED, "qsa_mla_sparse_attn: hq must be 1, 2, 4, 8 or 16");
    if ((int64_t)n > (int64_t)kListSeg * kListSegMax)
        return fail(QSA_ERR_UNSUPPORTED, "qsa_mla_sparse_attn: n too large");
    if (!isfinite(scale))
        return fail(QSA_ERR_INVALID, "qsa_mla_sparse_attn: scale is not finite");
    NEED_PTR(q);
    NEED_PTR(kv);
    OPT_PTR(v);
    NEED_PTR(mask);
    OPT_PTR(list_out);
    NEED_PTR(n_list);
    NEED_PTR(out);
    NEED_PTR(ws);
    const size_t need = qsa_mla_workspace_size(hq, dv, list_cap);
    if (ws_bytes < need)
        return fail(QSA_ERR_CAPACITY, "qsa_mla_sparse_attn: workspace has %zu bytes, needs %zu",
                    ws_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    uint32_t *seg_cnt = (uint32_t *)w;
    int32_t *list = (int32_t *)(w + round_up(sizeof(uint32_t) * kListSegMax, 256));
    float *part = (float *)((char *)list + round_up(sizeof(int32_t) * (size_t)list_cap, 256));
    if (list_out)
        list = list_out;
    HIP_CHECK(launch_mask_list(H(mask), n, list_cap, seg_cnt, list, n_list, s));
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = H(q);
    a.kbase = H(kv);
    a.vbase = v ? H(v) : H(kv);
    a.k_tok = dkq;
    a.v_tok = v ? dv : dkq;
    // one latent KV head: its query heads go in pairs to separate work groups,
    // which read the same rows (more work groups for a latency-bound call: 256 at
    // 16 heads and 2,048 listed rows, against 128 with groups of 4)
    a.hq = hq;
    a.hkv = hq > 2 ? hq / 2 : 1;
    a.kv_shared = 1;
    a.v_in_k = v ? 0 : 1;  // the latent view: V rows are KV[:, :dv]
    a.mode = kCellsList;
    a.list = list;
    a.n_list = n_list;
    a.list_cap = list_cap;
    a.bias = H(mask);
    a.scale = scale;
    split_plan(list_cap, &a.splits, &a.chunks);
    a.part = part;
    a.out = out;
    a.rows = 1;
    a.tok_bound = n;
    HIP_CHECK(launch_attn(a, dkq, dv, s));
    return QSA_OK;
}

int qsa_mla_list_status(const int32_t *n_list, int32_t list_cap, int32_t *n_list_host,
                        qsa_stream_t stream)
{
    if (!n_list)
        return fail(QSA_ERR_INVALID, "qsa_mla_list_status: n_list is NULL");
    if (list_cap < 1)
        return fail(QSA_ERR_INVALID, "qsa_mla_list_status: list_cap=%d", list_cap);
    int32_t n = 0;
    HIP_CHECK(hipMemcpyAsync(&n, n_list, sizeof(n), hipMemcpyDeviceToHost, (hipStream_t)stream));
    HIP_CHECK(hipStreamSynchronize((hipStream_t)stream));
    if (n_list_host)
        *n_list_host = n;
    if (n > list_cap)
        return fail(QSA_ERR_CAPACITY,
                    "qsa_mla_sparse_attn: %d positions visible, list_cap is %d (out is NaN)", n,
                    list_cap);
    return QSA_OK;
}

int qsa_trace_scan(void *start_event, void *stop_event)
{
    if (!start_event != !stop_event)
        return fail(QSA_ERR_INVALID, "qsa_trace_scan: give both events or neither");
    g_scan_events.start = (hipEvent_t)start_event;
    g_scan_events.stop = (hipEvent_t)stop_event;
    return QSA_OK;
}

}  // extern "C"
