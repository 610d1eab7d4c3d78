/*
 * qsa.h -- C ABI of libqsa, a QSA (Qwen Sparse Attention) layer step on AMD
 * Instinct MI355X (gfx950).
 *
 * One QSA layer step (sources: ariera, Qiita series part 10, sections
 * "QSAとQSA indexerについて", "incremental pooled-key cache（COMMON-004）",
 * "selected QSA K/V gather（COMMON-005）" and "block-domain top-k（COMMON-006）
 * 実装は見送り"; devotd.net news on the llama.cpp CDNA sparse path, sections 2-3):
 *   1. append the new token's indexer key; every completed 4-token block gets a
 *      pooled summary: mean of its 4 keys -> RMS norm per head -> RoPE at the
 *      block position -> binary16 row of the pooled-key cache;
 *   2. score the query against every complete block;
 *   3. keep the top-k blocks (ties to the lower block id) plus the incomplete
 *      tail block;
 *   4. gather the K/V of those cells;
 *   5. attention over those cells only.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers owned by the caller unless the name ends in
 *    _host.  binary16 data are passed as uint16_t (IEEE 754 binary16 bits).
 *  - Layouts are dense, row-major, token-major:
 *      k_raw   [cap_tokens][h_idx][d_idx]        raw indexer keys
 *      k_pool  [cap_tokens/4][h_idx][d_idx]      pooled-key cache
 *      k_cache [cap_tokens][hkv][d]              attention keys
 *      v_cache [cap_tokens][hkv][dv]             attention values
 *      q_idx   [n_q][h_idx][d_idx], q [n_q][hq][d], out [n_q][hq][dv] (fp32)
 *    Every pointer must be 16-byte aligned.
 *  - Token positions: a context of N tokens holds positions 0..N-1; block b
 *    holds tokens 4b..4b+3 and is complete once 4b+3 < N.  nb = floor(N/4)
 *    complete blocks; the tail is N mod 4 tokens; a decode step attends over
 *    4*min(k, nb) + (N mod 4) cells, a number the host can compute.
 *  - No entry point allocates device memory.  Scratch memory comes from a
 *    caller workspace of qsa_workspace_size() bytes; no call depends on what an
 *    earlier call left in it.  Calls that share one workspace must not overlap
 *    in time (same stream, or synchronised).
 *  - Every call enqueues its kernels on `stream` and returns without waiting.
 *    Arguments are checked on the host first; on a bad argument nothing is
 *    enqueued and a negative status is returned.  After QSA_ERR_HIP the
 *    workspace content is undefined: call qsa_workspace_init() again.
 *  - qsa_last_error() returns a message for the calling thread's last failure.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

/* Every entry point below is exported from the shared library; nothing else is. */
#if defined(__GNUC__) || defined(__clang__)
#define QSA_API __attribute__((visibility("default")))
#else
#define QSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_OK 0
#define QSA_ERR_INVALID -1      /* bad shape, size, null or misaligned pointer */
#define QSA_ERR_CAPACITY -2     /* position beyond cap_tokens, workspace too small */
#define QSA_ERR_UNSUPPORTED -3  /* shape outside what the kernels implement, or the
                                   list-attention preconditions fail */
#define QSA_ERR_HIP -4          /* the HIP runtime reported an error */

/* Decode-step flags. */
#define QSA_STEP_FUSED_GATHER 0u    /* attention reads the chosen cells from the caches */
#define QSA_STEP_COMPACT_GATHER 1u  /* copy chosen K/V to a compact buffer first, then
                                       attend over it (the COMMON-005 arrangement) */

/* Prefill flags. */
#define QSA_PREFILL_PER_ROW 0u        /* each row's attention reads its own cells */
#define QSA_PREFILL_GROUPED_UNION 1u  /* groups of 128 / (hq/hkv) consecutive rows read the
                                         union of their chosen blocks once (see
                                         qsa_prefill_attn) */
#define QSA_PREFILL_UNION_ALL 2u      /* with QSA_PREFILL_GROUPED_UNION: every group takes
                                         the union form, however large its union */

/* A hipStream_t; NULL is the null stream. */
typedef void *qsa_stream_t;

/* Shape and constants of one QSA layer. */
typedef struct qsa_config {
    int32_t h_idx;       /* indexer heads (16)                                   */
    int32_t d_idx;       /* indexer head dim (128); h_idx*d_idx/8 in {16..512},
                            power of two; d_idx/8 a power of two <= 64            */
    int32_t block;       /* tokens per pooled block; must be 4                   */
    int32_t topk_blocks; /* k, blocks kept (512 = 2048 tokens / 4); 1..1024      */
    int32_t hq;          /* attention query heads (32)                           */
    int32_t hkv;         /* attention KV heads (4); hq/hkv in {1,2,4,8,16}       */
    int32_t d;           /* attention key/query head dim (128)                   */
    int32_t dv;          /* attention value head dim (128)                       */
    int32_t cap_tokens;  /* capacity of the caches in tokens; multiple of 4,
                            at most 2^21                                          */
    float rope_base;     /* RoPE base (1e4)                                      */
    float rms_eps;       /* RMS-norm epsilon, added to the mean square (1e-6)    */
    float attn_scale;    /* softmax scale (1/sqrt(d))                            */
} qsa_config;

/* Caller-owned per-layer state (see the layouts above). */
typedef struct qsa_layer_bufs {
    uint16_t *k_raw;
    uint16_t *k_pool;
    uint16_t *k_cache;
    uint16_t *v_cache;
    const float *rms_w; /* [d_idx] RMS-norm weight, or NULL for all ones */
} qsa_layer_bufs;

/* Text for a status code. */
QSA_API const char *qsa_status_string(int status);

/* Message for the calling thread's last failed call ("" if none). */
QSA_API const char *qsa_last_error(void);

/* QSA_OK if cfg describes a shape the kernels implement. */
QSA_API int qsa_config_check(const qsa_config *cfg);

/*
 * Workspace bytes for calls with up to n_q query rows over contexts of up to
 * n_ctx tokens (n_ctx <= cap_tokens).  Returns 0 for an invalid cfg.
 */
QSA_API size_t qsa_workspace_size(const qsa_config *cfg, int32_t n_q, int32_t n_ctx);

/* Clears a workspace (a fill kernel on `stream`).  Optional: no call reads a
 * workspace byte it has not written in the same call. */
QSA_API int qsa_workspace_init(void *ws, size_t ws_bytes, qsa_stream_t stream);

/*
 * Pooled-key cache append (Qiita part 10, "QSAとQSA indexerについて" and
 * "incremental pooled-key cache（COMMON-004）").  Copies k_new [n_new][h_idx][d_idx]
 * to k_raw rows [n_before, n_before+n_new) and writes the pooled row of every
 * block that completes in that range: mean of the block's 4 raw keys, RMS norm
 * per head over d_idx (eps inside the root, times rms_w), RoPE (pair i with
 * i+d_idx/2, angle 4b * rope_base^(-2i/d_idx)), rounded to binary16.  Other pooled
 * rows are untouched, so one call with n_before = 0 rebuilds the whole cache and
 * token-by-token calls give the same bits.
 * Errors: INVALID (null, n_new < 0, n_before < 0), CAPACITY (n_before + n_new > cap_tokens).
 */
QSA_API int qsa_pool_append(const qsa_config *cfg, const uint16_t *k_new, int32_t n_new,
                    int32_t n_before, uint16_t *k_raw, uint16_t *k_pool, const float *rms_w,
                    qsa_stream_t stream);

/*
 * Pooled-cache rebuild from the raw indexer cache (Qiita part 10, "incremental
 * pooled-key cache（COMMON-004）": on a state load or a sequence edit the pooled
 * rows are invalidated and rebuilt when needed).  Recomputes the pooled rows of
 * blocks [b_from, floor(n_tokens/4)) from k_raw rows [4*b_from, n_tokens), as
 * qsa_pool_append computes them (same device code, same bits); other rows are
 * untouched.  Typical uses: after loading k_raw from a saved state (b_from = 0),
 * or after editing tokens from position p on (b_from = p / 4).
 * Rolling back rejected draft tokens needs no call: a pooled row is read only
 * once its block is complete in the caller's token count, and the append that
 * completes the block again recomputes it.
 * Errors: INVALID (null k_raw/k_pool, n_tokens outside [0, cap_tokens], b_from
 * outside [0, floor(n_tokens/4)]).
 */
QSA_API int qsa_pool_rebuild(const qsa_config *cfg, const uint16_t *k_raw, uint16_t *k_pool,
                     const float *rms_w, int32_t b_from, int32_t n_tokens, qsa_stream_t stream);

/* Copies k_new/v_new [n_new][hkv][d|dv] to cache rows [n_before, n_before+n_new). */
QSA_API int qsa_kv_append(const qsa_config *cfg, const uint16_t *k_new, const uint16_t *v_new,
                  int32_t n_new, int32_t n_before, uint16_t *k_cache, uint16_t *v_cache,
                  qsa_stream_t stream);

/*
 * Block scores (Qiita part 10, "QSAとQSA indexerについて": the pooled summaries
 * are scored against the query).  Query row r sits at position pos0 + r and sees
 * nb_r = floor((pos0 + r + 1) / 4) blocks; scores[r*ld + b] for b < nb_r is
 * sum over h, i of q_idx[r][h][i] * k_pool[b][h][i], accumulated in fp32.
 * Entries b >= nb_r are left unspecified.  ld >= nb of the last row.
 * n_q == 1 streams the pooled cache once (decode); n_q > 1 runs an MFMA
 * contraction (prefill chunk).
 */
QSA_API int qsa_index_score(const qsa_config *cfg, const uint16_t *q_idx, int32_t n_q, int32_t pos0,
                    const uint16_t *k_pool, float *scores, int32_t ld, qsa_stream_t stream);

/*
 * Top-k blocks per row (Qiita part 10, "QSAとQSA indexerについて" and the
 * COMMON-006 section: selection in the block domain).  Row r keeps
 * n_sel[r] = min(k, nb_r) blocks: the highest fp32 scores, equal scores to the
 * lower block id, -0 equal to +0, NaN lowest.  blk[r*k ..] receives the chosen
 * ids in ascending order.  Deterministic: the result depends only on the scores.
 */
QSA_API int qsa_topk_blocks(const qsa_config *cfg, const float *scores, int32_t n_q, int32_t ld,
                    int32_t pos0, int32_t *blk, int32_t *n_sel, void *ws, size_t ws_bytes,
                    qsa_stream_t stream);

/*
 * Compact K/V gather for one decode query (Qiita part 10, "selected QSA K/V
 * gather（COMMON-005）").  For n_tokens visible tokens and blk[0..n_blk) the chosen
 * blocks, writes k_sel/v_sel rows: the 4 cells of each chosen block in order,
 * then the tail tokens [4*floor(n_tokens/4), n_tokens).  Rows written:
 * 4*n_blk + n_tokens mod 4.  n_blk must equal min(k, floor(n_tokens/4)).
 */
QSA_API int qsa_gather_kv(const qsa_config *cfg, const int32_t *blk, int32_t n_blk, int32_t n_tokens,
                  const uint16_t *k_cache, const uint16_t *v_cache, uint16_t *k_sel,
                  uint16_t *v_sel, qsa_stream_t stream);

/*
 * Attention of one decode query over n_cells compact rows (Qiita part 10,
 * COMMON-005: ordinary attention over the gathered cells).  out[h][j] =
 * sum_c softmax_c(attn_scale * <q[h], k_sel[c][g]>) v_sel[c][g][j] with
 * g = h / (hq/hkv).  Split over cells, fp32 partials, one combining pass.
 */
QSA_API int qsa_sparse_attn(const qsa_config *cfg, const uint16_t *q, const uint16_t *k_sel,
                    const uint16_t *v_sel, int32_t n_cells, float *out, void *ws,
                    size_t ws_bytes, qsa_stream_t stream);

/*
 * Attention of a chunk of n_q query rows (row r at position pos0 + r), each over
 * its own cells: the blocks blk[r*ldb .. + n_sel_r) (n_sel_r = min(k, nb_r), each
 * row's ids ascending and distinct) and its tail, read directly from the caches.
 * The caches must already hold every token up to pos0 + n_q - 1.
 * flags: QSA_PREFILL_PER_ROW (one pass per row; ws may be NULL) or
 * QSA_PREFILL_GROUPED_UNION (the pages' "QSA grouped-union" prompt-processing
 * switch, Qiita part 10, opening paragraphs and the union ON/OFF table of
 * 「Vulkan版のプロファイリングでTGが遅くなった原因を調べる」; its steps are not given,
 * and the reading here keeps the result: groups of 128 / (hq/hkv) consecutive rows
 * stream the union of their chosen blocks and their tails once, on the matrix
 * cores, with a per-row mask so that every row attends to exactly its own cells).
 * A group whose union holds more than 3/8 of its rows x k blocks (rows that share
 * few blocks) is attended per row instead, where that is cheaper; adding
 * QSA_PREFILL_UNION_ALL makes every group take the union form.  All forms give the
 * per-row result up to fp32 summation order and binary16 rounding of the softmax
 * weights.  On an MI355X, for 1,024 rows at depth 126,253: 0.15 ms by the union
 * when neighbouring rows share most of their blocks, 0.40 ms per row when they
 * share almost none (the union alone: 0.78 ms).  The union form needs hq/hkv in
 * {4, 8, 16}, d = dv = 128 and (128 / (hq/hkv)) * topk_blocks <= 16384 (else
 * QSA_ERR_UNSUPPORTED) and a workspace of qsa_workspace_size(cfg, n_q, pos0 + n_q).
 * Every form drops a chosen id outside the row's [0, nb_r).
 * Errors: INVALID (unknown flags, QSA_PREFILL_UNION_ALL without
 * QSA_PREFILL_GROUPED_UNION, bad pointers), UNSUPPORTED, CAPACITY (workspace).
 */
QSA_API int qsa_prefill_attn(const qsa_config *cfg, const uint16_t *q, int32_t n_q, int32_t pos0,
                     const int32_t *blk, int32_t ldb, const uint16_t *k_cache,
                     const uint16_t *v_cache, float *out, uint32_t flags, void *ws,
                     size_t ws_bytes, qsa_stream_t stream);

/*
 * One decode step of one layer: steps 1-5 above for the token at position
 * n_before (the context grows to N = n_before + 1).  Appends k_idx_new [h_idx][d_idx]
 * to the indexer caches and k_new/v_new [hkv][d|dv] to the K/V caches, then
 * scores, selects and attends; out [hq][dv] fp32.  Optional outputs (NULL to
 * skip): scores_out [floor(N/4)] fp32 block scores, blk_out [min(k, floor(N/4))]
 * chosen blocks in ascending order.
 * flags: QSA_STEP_FUSED_GATHER (the selection runs inside the attention launch,
 * which reads the chosen cells straight from the caches) or
 * QSA_STEP_COMPACT_GATHER (separate top-k and gather launches, then attention
 * over the compact rows).
 */
QSA_API int qsa_decode_step(const qsa_config *cfg, const qsa_layer_bufs *L, int32_t n_before,
                    const uint16_t *q_idx, const uint16_t *k_idx_new, const uint16_t *q,
                    const uint16_t *k_new, const uint16_t *v_new, float *out, float *scores_out,
                    int32_t *blk_out, uint32_t flags, void *ws, size_t ws_bytes,
                    qsa_stream_t stream);

/*
 * qsa_decode_step for callers that cannot allocate or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid device allocation.
 * Same arguments, results and kernels as qsa_decode_step, without ws/ws_bytes: the
 * scratch is a static array of QSA_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU, which each GPU keeps until the process ends (its address is looked up
 * once per device, on that device's first call).  The call allocates nothing.
 * The device current on the calling thread must be the stream's device.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (other streams, other threads) race and give undefined results; serialise
 * them.  The array keeps the last call's contents; no call reads a byte of it that
 * the same call did not write, so nothing needs clearing.
 * Errors: as qsa_decode_step; CAPACITY also when the shape's scratch
 * (qsa_workspace_size(cfg, 1, n_before + 1)) exceeds QSA_NOALLOC_SCRATCH_BYTES;
 * INVALID when the stream belongs to another device.
 */
#define QSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
QSA_API int qsa_decode_step_noalloc(const qsa_config *cfg, const qsa_layer_bufs *L, int32_t n_before,
                            const uint16_t *q_idx, const uint16_t *k_idx_new, const uint16_t *q,
                            const uint16_t *k_new, const uint16_t *v_new, float *out,
                            float *scores_out, int32_t *blk_out, uint32_t flags,
                            qsa_stream_t stream);

/*
 * Multi-query decode step for checking speculative draft tokens (Qiita part 12,
 * 「MTPを入れたらPPが遅くなるのは仕方がないのか？」: the target model checks the
 * draft's tokens together; its setup table runs DraftMax = 2, so a step carries
 * up to 3 tokens).  Appends the n_q tokens at positions [n_before, n_before + n_q)
 * to all four caches; row r then runs steps 2-5 causally with N_r = n_before + r + 1
 * visible tokens, its own top-k and its own cells.  The pooled cache is streamed
 * once for all rows.  The result equals n_q qsa_decode_step calls in order.
 * n_q in [1, 4]; q_idx [n_q][h_idx][d_idx], k_idx_new [n_q][h_idx][d_idx],
 * q [n_q][hq][d], k_new/v_new [n_q][hkv][d|dv], out [n_q][hq][dv] fp32.
 * Optional: scores_out [n_q][ld_scores] (ld_scores >= floor((n_before + n_q)/4);
 * row r defined for b < floor(N_r/4)), blk_out [n_q][k] (row r: min(k, floor(N_r/4))
 * ids, ascending).  Rejected rows need no undo: see qsa_pool_rebuild.
 * Errors: INVALID (n_q outside [1, 4], ld_scores too small, null or misaligned
 * pointers), CAPACITY (n_before + n_q > cap_tokens, workspace too small).
 */
QSA_API int qsa_decode_multi(const qsa_config *cfg, const qsa_layer_bufs *L, int32_t n_before,
                     int32_t n_q, const uint16_t *q_idx, const uint16_t *k_idx_new,
                     const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, float *out,
                     float *scores_out, int32_t ld_scores, int32_t *blk_out, void *ws,
                     size_t ws_bytes, qsa_stream_t stream);

/*
 * One prefill chunk of one layer: appends n_new tokens at positions
 * [n_before, n_before + n_new) to all four caches, then every chunk row runs
 * steps 2-5 causally (row r sees N_r = n_before + r + 1 tokens).
 * q_idx [n_new][h_idx][d_idx], q [n_new][hq][d], out [n_new][hq][dv].
 * Optional outputs: scores_out [n_new][ld_scores], blk_out [n_new][k].
 * flags: as for qsa_prefill_attn.
 */
QSA_API int qsa_prefill_step(const qsa_config *cfg, const qsa_layer_bufs *L, int32_t n_before,
                     int32_t n_new, const uint16_t *q_idx, const uint16_t *k_idx_new,
                     const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, float *out,
                     float *scores_out, int32_t ld_scores, int32_t *blk_out, uint32_t flags,
                     void *ws, size_t ws_bytes, qsa_stream_t stream);

/*
 * MLA-style list attention (devotd.net news on the llama.cpp CDNA sparse path,
 * sections 2-3).  mask [n] is additive binary16: -inf hides a position, any other
 * value is added to its logit.  The visible positions are listed in ascending
 * order (one 64-bit ballot per 64 positions, popcount ranks), then each of the hq
 * query heads attends over the listed rows of one shared KV head:
 * logit = scale * <q[h], kv[j][0:dkq]> + mask[j]; value = v[j][0:dv] if v is not
 * NULL, else kv[j][0:dv].  q [hq][dkq], kv [n][dkq], v [n][dv], out [hq][dv] fp32.
 * list_out [list_cap] (optional) and n_list [1] (device) receive the list and its
 * length.  Preconditions (else QSA_ERR_UNSUPPORTED): mask != NULL, n >= 4096,
 * n >= 2*list_cap, dkq == 576, dv == 512, hq in {1, 2, 4, 8, 16}.  If more
 * than list_cap positions are visible, n_list receives the true count, nothing
 * past list_cap is read and out is filled with NaN.  The list length is known only
 * on the device when the call returns, so the capacity error reaches the host
 * through qsa_mla_list_status() below (the call itself stays asynchronous).
 */
QSA_API size_t qsa_mla_workspace_size(int32_t hq, int32_t dv, int32_t list_cap);
QSA_API int qsa_mla_sparse_attn(const uint16_t *q, int32_t hq, const uint16_t *kv, const uint16_t *v,
                        int32_t dkq, int32_t dv, const uint16_t *mask, int32_t n,
                        int32_t list_cap, float scale, int32_t *list_out, int32_t *n_list,
                        float *out, void *ws, size_t ws_bytes, qsa_stream_t stream);

/*
 * Capacity status of a qsa_mla_sparse_attn call (devotd.net news, section 3: the
 * list holds at most list_cap positions).  Waits for `stream`, reads the device
 * count n_list [1] that the call wrote and returns QSA_ERR_CAPACITY if it exceeds
 * list_cap (that call's out is NaN), else QSA_OK.  n_list_host (optional, host
 * memory) receives the count.  Blocks the calling thread; not for graph capture.
 * Errors: INVALID (n_list NULL, list_cap < 1), HIP (copy or wait failed).
 */
QSA_API int qsa_mla_list_status(const int32_t *n_list, int32_t list_cap, int32_t *n_list_host,
                        qsa_stream_t stream);

/*
 * Kernel timing of one scoring launch, for tracing (no part of the method; results
 * do not change).  start_event and stop_event are hipEvent_t handles that the
 * caller created, with timing enabled, on the device of the call's stream.  The
 * calling thread's next qsa_decode_step, qsa_decode_step_noalloc, qsa_decode_multi
 * or qsa_index_score launches its scoring kernel (in a decode step: the appends,
 * the block scores and the candidate lists) so that the two events take that
 * kernel's own start and end times (hipEventElapsedTime then gives its duration);
 * that call clears the setting, whatever it returns.  Both NULL clear it.  The
 * events stay the caller's.  The call must not be under stream capture.
 * Errors: INVALID (exactly one of the two is NULL).
 */
QSA_API int qsa_trace_scan(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
