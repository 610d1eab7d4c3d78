// Host-side launchers shared between the entry points (qsa_api.hip) and the
// kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qsa_device.h"

namespace qsa {

// A contiguous copy of n16 16-byte units.
struct CopySeg {
    const void *src;
    void *dst;
    int64_t n16;
};

constexpr int kHistBits = 12;  // top-k: bins of the top 12 bits of a score key
constexpr int kHistBins = 1 << kHistBits;

// ---- append (k_pool.hip) ----------------------------------------------------
struct AppendArgs {
    CopySeg seg[3];      // raw rows, K rows, V rows (unused entries have n16 == 0)
    const h16 *k_new;    // new raw indexer keys, token n_before first
    int32_t n_before;
    h16 *k_raw;
    h16 *k_pool;
    const float *rms_w;
    int32_t H, d;
    int32_t b_lo, n_blocks;  // blocks [b_lo, b_lo + n_blocks) complete in this call
    float eps;
    float base;
};
hipError_t launch_append(const AppendArgs &a, hipStream_t s);

// ---- decode top-k candidate lists (written by the scan, read by the top-k) ----
// Each work group of the decode-step scan keeps the kListLen highest rank keys
// (rank_key) of the rows it scored, in any order (0 = empty slot), and the
// number of rows it scored.  The global top-k is contained in the union of the
// lists unless some work group scored more than kListLen rows and the smallest
// entry of its list is itself chosen; the top-k kernel checks exactly that.
constexpr int kListLen = 8;
constexpr int kListWgs = 1024;  // lists at most (one per thread of the top-k kernel)
struct CandLists {
    uint64_t *list;  // [kListWgs][kListLen]
    uint32_t *rows;  // [kListWgs]
};

// ---- scores (k_score.hip) ---------------------------------------------------
// Events that a launch records with its kernel's own start and end times
// (hipExtLaunchKernelGGL); both NULL: a plain launch.
struct KernelEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
// A launch of kern with the events of ev, else plain.
template <typename F, typename... Args>
void launch_ev(F kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, KernelEvents ev,
               Args... args)
{
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kern, grid, block, lds, s, args...);
}
// Stand-alone scan (qsa_index_score, ap NULL, n_q = 1): scores[0, nb).
// Decode-step scan (ap non-NULL): the append work runs in the same launch (at
// most one completed block, block nb; its scores are written too); n_q queries
// (rows of q) score every row read once, query i into scores[i * ld ..]; with
// cl (n_q = 1 only) every work group also writes its candidate list and
// *n_lists gets the list count.  ev: the scoring launch records them.
hipError_t launch_score_decode(const h16 *q, int32_t n_q, const h16 *pool, int32_t nb,
                               int32_t row_elems, float *scores, int32_t ld, const AppendArgs *ap,
                               const CandLists *cl, int32_t *n_lists, hipStream_t s,
                               KernelEvents ev = {});
// The decode-step scan's list layout: list 0 is the append work group's; scan work
// group b = list - 1 (of n_lists - 1) owns the runs of 4 consecutive row groups
// 4 b + 4 (n_lists - 1) m .. + 3, a row group being this many consecutive rows.
int32_t scan_rows_per_group(int32_t row_elems);
hipError_t launch_score_prefill(const h16 *q, int32_t n_q, int32_t pos0, const h16 *pool,
                                int32_t row_elems, float *scores, int32_t ld, hipStream_t s,
                                KernelEvents ev = {});

// ---- top-k (k_topk.hip) -----------------------------------------------------
// One decode row: candidate lists built from the scores (in cl), then the list
// selection.  Keeps no state between calls.
hipError_t launch_topk_decode(const float *scores, int32_t nb, int32_t k, int32_t *blk,
                              int32_t *n_sel, CandLists cl, hipStream_t s);
// Candidate lists of `rows` score rows (stride ld; row r sees (pos0 + r + 1) / 4
// blocks), laid out as the decode scan lays them out, row r's at
// cl.list + r * kListWgs * kListLen; *n_lists gets the lists per row.
hipError_t launch_score_lists(const float *scores, int32_t rows, int32_t ld, int32_t pos0,
                              CandLists cl, int32_t *n_lists, hipStream_t s);
// Top-k of one row from the scan's candidate lists (n_lists of them); when the
// lists cannot be shown to hold the top-k, the lists that may hide chosen rows are
// widened with their work groups' rows, else it selects from the whole score row.
// scan_rpw: the lists come from the decode-step scan (scan_rows_per_group() of its
// rows; they cover rows < n_scan); 0: from launch_score_lists (rows < nb).
hipError_t launch_topk_lists(const float *scores, int32_t nb, int32_t k, CandLists cl,
                             int32_t n_lists, int32_t *blk, int32_t *n_sel, hipStream_t s,
                             int32_t scan_rpw = 0, int32_t n_scan = 0);
hipError_t launch_topk_rows(const float *scores, int32_t n_q, int32_t ld, int32_t pos0,
                            int32_t k, int32_t *blk, int32_t *n_sel, hipStream_t s);
int32_t topk_max_blocks();

// ---- gather / attention (k_attn.hip) -----------------------------------------
hipError_t launch_gather(const int32_t *blk, int32_t n_blk, int32_t n_tokens,
                         const h16 *k_cache, const h16 *v_cache, int32_t k_row16,
                         int32_t v_row16, h16 *k_sel, h16 *v_sel, hipStream_t s);

enum CellMode : int32_t { kCellsCompact = 0, kCellsBlocks = 1, kCellsList = 2 };
constexpr int kAttnChunk = 64;
constexpr int kAttnMaxSplits = 64;
constexpr int kAttnChunksPerSplit = 1;

struct AttnArgs {
    const h16 *q;           // [rows][hq][D]
    const h16 *kbase;       // token-major K rows
    const h16 *vbase;       // token-major V rows
    int64_t k_tok;          // elements per token row of K (hkv * D, or dkq for MLA)
    int64_t v_tok;          // elements per token row of V
    int32_t hq, hkv;
    int32_t mode;
    int32_t n_cells;        // compact: rows of k_sel/v_sel
    const int32_t *blk;     // blocks: [rows][ldb] (NULL: every block, in order)
    int32_t ldb;
    int32_t pos0;           // blocks: row r sees pos0 + r + 1 tokens
    int32_t topk;
    const int32_t *list;    // list: token of cell c
    const int32_t *n_list;  // list: device count
    int32_t list_cap;
    const h16 *bias;        // list: additive per-token mask (NULL: none)
    float scale;
    int32_t splits;         // work groups per (row, kv head)
    int32_t chunks;         // chunks of kAttnChunk cells per work group
    float *part;            // [rows][hq][splits][dv + 2] when splits > 1
    float *out;             // [rows][hq][dv]
    int32_t rows;
    int32_t tok_bound;      // list: tokens must be < tok_bound (the mask length)
    int32_t kv_shared;      // 1: every KV-head group reads the same K/V rows (one latent
                            // head, its query heads split into hkv groups)
    int32_t v_in_k;         // 1: each V row is the first DV elements of its K row
                            // (vbase == kbase, v_tok == k_tok; the MLA latent view)
};
hipError_t launch_attn(const AttnArgs &a, int32_t D, int32_t DV, hipStream_t s);
// Merge of split-K partials [rows][hq][splits][dv + 2] into out [rows][hq][dv].
hipError_t launch_combine(const float *part, int32_t hq, int32_t splits, int32_t dv, int32_t rows,
                          float *out, hipStream_t s);

// ---- decode-step tail (k_step.hip) -----------------------------------------
// Top-k from the scan's candidate lists and attention over the chosen cells in
// one launch, then the combine.
constexpr int kMaxTopk = 1024;
constexpr int kMaxDecodeRows = 4;  // query rows of one multi-query decode step
struct StepTail {
    CandLists cl;         // row r's lists at r * kListWgs * kListLen (rows at r * kListWgs)
    int32_t n_lists;
    const float *scores;  // [rows][ld] score rows (used when the lists are not enough)
    int32_t ld;
    int32_t pos0;         // row r is the token at position pos0 + r
    int32_t rows;
    int32_t k;
    const h16 *q;         // [rows][hq][d]
    const h16 *k_cache;
    const h16 *v_cache;
    int32_t hq, hkv, d, dv;
    float scale;
    float *part;          // [rows][hq][splits][dv + 2]
    float *out;           // [rows][hq][dv]
    int32_t *blk_out;     // optional: [rows][k] chosen ids, ascending
    int32_t scan_rpw;     // scan_rows_per_group() of the scan that wrote the lists
};
hipError_t launch_step_tail(const StepTail &st, hipStream_t s);

// ---- grouped-union prefill attention (k_union.hip) ----------------------------
// Consecutive query rows (128 / (hq / hkv) of them) share one pass over the union
// of their chosen blocks; each row keeps exactly its own cells through a mask.
constexpr int kUnionCap = 16384;      // union slots per group (rows x k)
constexpr int kUnionMaxSplits = 8;
constexpr int kUnionSets = 1;         // 4-wave sets per work group
constexpr int kUnionTargetWgs = 512;  // work groups per launch the splits aim for
constexpr int kUnionPartStride = 132; // floats per split partial: (m, l, -, -) + 128 dims
struct UnionArgs {
    const h16 *q;           // [n_q][hq][128]
    const int32_t *blk;     // [n_q][ldb] chosen ids per row, ascending
    int32_t ldb;
    const h16 *k_cache, *v_cache;
    int32_t n_q, pos0, k, hq, hkv;
    float scale;
    int32_t splits;         // union_splits()
    int32_t u_limit;        // groups of more union blocks go to the per-row kernel
                            // (union_limit(); at least rows * k: every group here)
    int32_t *uid;           // [groups][rows * k]
    uint32_t *umask;        // [groups][rows * k]
    int32_t *n_u;           // [groups]
    float *part;            // [n_q][hq][splits][kUnionPartStride] when splits > 1
    float *out;             // [n_q][hq][128]
};
bool union_supported(int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t k);
int32_t union_group_rows(int32_t hq, int32_t hkv);
int32_t union_splits(int32_t n_q, int32_t hq, int32_t hkv);
int32_t union_limit(int32_t hq, int32_t hkv, int32_t k);
hipError_t launch_union_attn(const UnionArgs &u, hipStream_t s);

// ---- per-row prefill attention on the matrix cores (k_rows.hip) ---------------
// One work group per (KV head, row); d = dv = 128, hq / hkv in {4, 8, 16}.
struct RowsArgs {
    const h16 *q;           // [n_q][hq][128]
    const int32_t *blk;     // [n_q][ldb] chosen ids per row
    int32_t ldb;
    const h16 *k_cache, *v_cache;  // token-major [tok][hkv][128]
    int32_t n_q, pos0, k, hq, hkv;
    float scale;
    float *out;             // [n_q][hq][128]
    const int32_t *n_u;     // union blocks per row group (NULL: every row here)
    int32_t group_rows;     // rows per group of n_u
    int32_t u_limit;        // rows of a group with n_u <= u_limit are the union's:
    const float *part;      // their split partials (splits > 1), merged here
    int32_t splits;
};
// n_tokens: tokens in the caches the rows read (pos0 + n_q)
bool rows_supported(int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t k, int64_t n_tokens);
hipError_t launch_rows_attn(const RowsArgs &a, hipStream_t s);

// ---- MLA list (k_mla.hip) ---------------------------------------------------
constexpr int kListSeg = 1024;     // positions per list-building work group
constexpr int kListSegMax = 8192;  // segments: masks of up to 8,388,608 positions
constexpr uint16_t kF16NegInf = 0xFC00u;  // binary16 -inf: a hidden position
// Counts per segment, then the whole ascending list and its count.
hipError_t launch_mask_list(const h16 *mask, int32_t n, int32_t list_cap, uint32_t *seg_cnt,
                            int32_t *list, int32_t *n_list, hipStream_t s);

// ---- misc -------------------------------------------------------------------
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);

}  // namespace qsa
