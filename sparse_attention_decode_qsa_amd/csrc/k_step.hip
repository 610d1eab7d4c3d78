// Decode-step tail in one launch: block-domain top-k, then attention over the
// chosen cells only (Qiita part 10, "QSAとQSA indexerについて": keep the
// highest-scoring blocks plus the incomplete tail block; "selected QSA K/V
// gather（COMMON-005）": attention over those cells; the COMMON-006 section:
// selection in the block domain).
//
// Grid: (split, KV head, query row), 1024 threads.  Every work group first selects the
// same top-k blocks from the decode scan's candidate lists (lists_select; the
// lists that may hide chosen rows are widened with their work groups' rows, and
// the whole score row is the last resort), in the deterministic order of
// the selection (attention does not depend on the order of its cells); the
// threads holding the chosen blocks of this work group's split write its 64
// cell tokens to LDS.  Then all 16 waves attend those 64 cells for one KV head:
// thread (cell, 16-byte piece) loads one piece of the cell's K row and one of
// its V row, dots the K piece with the G query heads and the partial dots of a
// cell meet by DPP across its lanes; wave h runs the softmax of head h (log2
// domain); thread (head, dim) sums P x V from LDS; each head leaves an (m, l, o)
// partial for attn_combine_kernel.  Selecting in every work group costs a few
// microseconds of LDS work but saves a kernel boundary and a round trip through
// global memory for the chosen ids.
//
// Work group (0, 0, r) also writes row r's blk_out (ascending ids, through an
// LDS bitmap) when asked for.  Rows of a multi-query step see N_r = pos0 + r + 1
// tokens, each its own selection; splits past a row's cells leave a partial the
// combine weighs 0.
#include "qsa_select.h"

namespace qsa {
namespace {

constexpr int kNT = kSelThreads;  // 16 waves
constexpr int kMaxChunks = 4;      // 64-cell chunks per split
constexpr float kLog2e = 1.4426950408889634f;

struct TailArgs {
    CandLists cl;         // row r's lists at list + r * kListWgs * kListLen, rows + r * kListWgs
    int32_t n_lists;
    const float *scores;  // [rows][ld] score rows (fallback selection)
    int32_t ld;
    int32_t pos0;         // row r is the token at position pos0 + r: N_r = pos0 + r + 1
    int32_t k;
    const h16 *q;         // [rows][hq][D]
    const h16 *kc;        // [N][hkv][D]
    const h16 *vc;        // [N][hkv][DV]
    int32_t hq, hkv;
    float scale;
    int32_t chunks;       // 64-cell chunks per split
    int32_t splits;       // ceil(cells / (64 chunks)) of the row with the most cells
    float *part;          // [rows][hq][splits][DV + 2]
    int32_t *blk_out;     // optional, [rows][k]
    int32_t scan_rpw;     // rows per row group of the decode scan (its list layout)
};

template <int G, int D, int DV>
struct alignas(16) TailLds {
    union alignas(16) {
        struct {
            uint32_t bitmap[kMaxBlocks / 32];
            uint64_t cand[kCandCap];
        } sel;  // the fallback selection and the blk_out sort
        struct {
            alignas(16) h16 vs[kAttnChunk * DV];
            alignas(16) float ps[G][kAttnChunk];
            float ml[G][3];  // running max, running sum, rescale of the last chunk
        } att;
    } u;
    ListSelLds L;
    alignas(16) h16 qs[G * D];
    alignas(16) int32_t ids[kMaxTopk];
    alignas(16) int32_t toks[kMaxChunks * kAttnChunk];
    alignas(16) uint32_t wsum[kNT / kWave];
};

// Sum over aligned groups of W lanes (W = 8 or 16) by DPP within 16-lane rows.
template <int W>
__device__ __forceinline__ float row_group_sum(float x)
{
    static_assert(W == 8 || W == 16, "group");
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    x += dpp<kDppRowHalfMirror>(x);
    if (W == 16)
        x += dpp<kDppRowMirror>(x);
    return x;
}

// Places the chosen blocks once the lists hold the top-k exactly (every key >= rs):
// an exclusive prefix over the work group (wave scans, one barrier, then the
// totals of the waves below) gives each thread the positions of its keys, and
// place(pos, id) is called for positions below k.
template <typename Place>
__device__ __forceinline__ void place_chosen(const uint64_t (&R)[kListLen], uint64_t rs,
                                             uint32_t k, uint32_t nb, uint32_t *wsum,
                                             Place place)
{
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kListLen; j++)
        c += R[j] >= rs ? 1u : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (lane == kWave - 1)
        wsum[wave] = incl;
    __syncthreads();
    uint32_t pos = incl - c;
#pragma unroll
    for (int i = 0; i < kNT / kWave; i += 4) {
        const uint4 v = *(const uint4 *)&wsum[i];
        pos += (i < wave ? v.x : 0u) + (i + 1 < wave ? v.y : 0u) +
               (i + 2 < wave ? v.z : 0u) + (i + 3 < wave ? v.w : 0u);
    }
#pragma unroll
    for (int j = 0; j < kListLen; j++)
        if (R[j] >= rs) {
            uint32_t id = rank_id(R[j]);
            id = id < nb ? id : 0u;
            if (pos < k)
                place((int32_t)pos, (int32_t)id);
            pos++;
        }
}

// Where the chosen blocks of one split go: position i to cells 4i .. 4i + 3 of the
// split's token table (positions b_lo .. b_hi - 1), and to ids[i] when want_ids.
struct SplitPlace {
    int32_t *toks;
    int32_t *ids;
    uint32_t *wsum;
    int32_t b_lo, b_hi;
    bool want_ids;
    __device__ void operator()(int32_t pos, int32_t id) const
    {
        if (pos >= b_lo && pos < b_hi) {
#pragma unroll
            for (int e = 0; e < kBlockTokens; e++)
                toks[(pos - b_lo) * kBlockTokens + e] = kBlockTokens * id + e;
        }
        if (want_ids)
            ids[pos] = id;
    }
};

struct ListKeys {
    uint64_t v[kListLen];
};

// The lists hide chosen rows (rs = R* of the lists): widen them with their work
// groups' rows (widen_lists), select again and, when that is exact, place the
// chosen blocks.  Returns false if the lists are still not enough (the caller then
// selects from the whole score row).  Out of line, so that the step's usual path
// carries none of this code.  All kNT threads call it.
__device__ __noinline__ bool widen_select_place(ListKeys keys, uint32_t nrows, int32_t W,
                                                uint64_t rs, const float *scores,
                                                ListLayout lay, uint32_t k, uint32_t nb,
                                                ListSelLds &L, SplitPlace pl)
{
    uint64_t(&R)[kListLen] = keys.v;
    if (!widen_lists(R, &nrows, W, rs, scores, lay, L))
        return false;
    __syncthreads();
    if (lists_select(R, nrows, (int)threadIdx.x < W, k, L, &rs) != kListsExact)
        return false;
    place_chosen(R, rs, k, nb, pl.wsum, pl);
    return true;
}

template <int G, int D, int DV>
__global__ __launch_bounds__(kNT) void step_tail_kernel(TailArgs a)
{
    constexpr int PK = D / 8;                  // 16-byte pieces per K row
    constexpr int PV = DV / 8;                 // 16-byte pieces per V row
    static_assert(PK == 8 || PK == 16, "K row pieces");
    static_assert(kAttnChunk * PK <= kNT && kAttnChunk * PV <= kNT, "one piece per thread");
    static_assert(G <= kNT / kWave, "one wave per head in the softmax");

    __shared__ TailLds<G, D, DV> sm;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    const int split = blockIdx.x, g = blockIdx.y, row = blockIdx.z;
    const int32_t N = a.pos0 + row + 1, nb = N / kBlockTokens;
    const int32_t nsel = nb < a.k ? nb : a.k;
    const int32_t cells = kBlockTokens * nsel + (N - kBlockTokens * nb);
    float *part = a.part + (int64_t)row * a.hq * a.splits * (DV + 2);
    const int chunks = a.chunks;
    const int32_t c_lo = split * chunks * kAttnChunk;  // this split's cells
    if (c_lo >= cells) {
        // past this row's cells (rows of one call differ by up to 3): a partial
        // that the combine weighs 0
        for (int o = t; o < G * (DV + 2); o += kNT) {
            const int h = o / (DV + 2), j = o % (DV + 2);
            part[(((int64_t)g * G + h) * a.splits + split) * (DV + 2) + j] = j == 0 ? -INFINITY : 0.f;
        }
        return;
    }
    const float *scores = a.scores + (int64_t)row * a.ld;
    CandLists cl = a.cl;
    cl.list += (int64_t)row * kListWgs * kListLen;
    cl.rows += (int64_t)row * kListWgs;
    const int32_t b_lo = c_lo / kBlockTokens;  // its chosen-block positions
    const int32_t b_hi = b_lo + chunks * kAttnChunk / kBlockTokens;
    const bool from_lists = nb > a.k;  // else every complete block is chosen

    // the query rows of this KV head (independent of the selection) and candidate
    // list t: every load issued (indexes clamped, no branch) before any result is
    // used, so that the two round trips overlap
    constexpr int QN = G * D / 8;  // 16-byte pieces of the query rows
    static_assert(QN <= kNT, "one query piece per thread");
    const h16x8 *qrow8 = (const h16x8 *)(a.q + ((int64_t)row * a.hq + (int64_t)g * G) * D);
    const h16x8 qv = qrow8[t < QN ? t : QN - 1];
    uint64_t R[kListLen];
    uint32_t nrows = 0;
    if (from_lists)
        load_list_raw(cl, a.n_lists, R, &nrows);
    if (t < QN)
        ((h16x8 *)sm.qs)[t] = qv;
    // the split's tail cells (the incomplete block, after the chosen ones)
    for (int i = t; i < chunks * kAttnChunk; i += kNT) {
        const int32_t c = c_lo + i;
        sm.toks[i] = (c >= kBlockTokens * nsel && c < cells)
                         ? kBlockTokens * nb + (c - kBlockTokens * nsel)
                         : -1;
    }
    // the selection's first stage shares this barrier
    if (from_lists) {
        drop_absent_list(a.n_lists, R, &nrows);
        lists_prepare(R, nrows, t < a.n_lists, sm.L);
    }
    __syncthreads();
    // the chosen blocks; position i goes to cells 4i .. 4i + 3
    auto place = [&](int32_t pos, int32_t id) {
        if (pos >= b_lo && pos < b_hi) {
#pragma unroll
            for (int e = 0; e < kBlockTokens; e++)
                sm.toks[(pos - b_lo) * kBlockTokens + e] = kBlockTokens * id + e;
        }
    };

    // ---- 1. selection
    const bool want_blk = a.blk_out && blockIdx.x == 0 && blockIdx.y == 0;
    int32_t *blk_out = a.blk_out ? a.blk_out + (int64_t)row * a.k : nullptr;
    if (!from_lists) {
        for (int32_t i = t; i < nb; i += kNT) {
            place(i, i);
            if (want_blk)
                sm.ids[i] = i;
        }
    } else {
        uint64_t rs = 0;
        const int sel = lists_select_rest(R, (uint32_t)a.k, sm.L, &rs);
        const SplitPlace pl{sm.toks, sm.ids, sm.wsum, b_lo, b_hi, want_blk};
        bool placed = false;
        if (sel == kListsExact) {
            place_chosen(R, rs, (uint32_t)a.k, (uint32_t)nb, sm.wsum, pl);
            placed = true;
        } else if (sel == kListsHide) {
            // the scan's row layout: list 0 is the append's, scan work group
            // b = list - 1 of n_lists - 1 owns runs of 4 row groups
            ListKeys keys;
#pragma unroll
            for (int j = 0; j < kListLen; j++)
                keys.v[j] = R[j];
            const ListLayout lay{1, a.n_lists - 1, a.scan_rpw, (uint32_t)(a.pos0 / kBlockTokens)};
            placed = widen_select_place(keys, nrows, a.n_lists, rs, scores, lay, (uint32_t)a.k,
                                        (uint32_t)nb, sm.L, pl);
        }
        if (!placed) {
            __syncthreads();
            select_row_global<kNT>(scores, (uint32_t)nb, a.k, sm.ids, sm.L.hist[0],
                                   sm.u.sel.cand, sm.u.sel.bitmap, sm.L.S);
            __syncthreads();
            for (int32_t i = t; i < nsel; i += kNT)
                place(i, sm.ids[i]);
        }
    }
    __syncthreads();

    if (want_blk) {
        zero_words<kNT>(sm.u.sel.bitmap, ((uint32_t)nb + 31) / 32);
        __syncthreads();
        for (int32_t i = t; i < nsel; i += kNT)
            set_bit(sm.u.sel.bitmap, (uint32_t)sm.ids[i]);
        __syncthreads();
        compact_bitmap<kNT>(sm.u.sel.bitmap, (uint32_t)nb, blk_out, (uint32_t)a.k, sm.L.S);
        __syncthreads();  // the bitmap shares LDS with the attention arrays
    }

    // ---- 2. attention over the split's chunks of 64 cells for KV head g, with
    // an online softmax across chunks (running max and sum per head in LDS,
    // kept by wave h; the output of (head, dim) in a register of its thread)
    constexpr int OPT = (G * DV + kNT - 1) / kNT;  // outputs per thread
    const int64_t k_tok = (int64_t)a.hkv * D, v_tok = (int64_t)a.hkv * DV;
    const int kc = t / PK, kp = t % PK;
    const int vc = t / PV, vp = t % PV;
    const bool k_on = kc < kAttnChunk, v_on = vc < kAttnChunk;
    const float sl2 = a.scale * kLog2e;
    float oacc[OPT];
#pragma unroll
    for (int i = 0; i < OPT; i++)
        oacc[i] = 0.f;
    if (wave < G && lane == 0) {
        sm.u.att.ml[wave][0] = -INFINITY;
        sm.u.att.ml[wave][1] = 0.f;
    }
    for (int ch = 0; ch < chunks; ch++) {
        // K: thread (cell, piece); V: thread (cell, piece); both loads in flight
        const int32_t ktok = k_on ? sm.toks[ch * kAttnChunk + kc] : -1;
        const int32_t vtok = v_on ? sm.toks[ch * kAttnChunk + vc] : -1;
        h16x8 kv = h16x8{0, 0, 0, 0, 0, 0, 0, 0}, vv = h16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (ktok >= 0)
            kv = *(const h16x8 *)(a.kc + (int64_t)ktok * k_tok + (int64_t)g * D + kp * 8);
        if (vtok >= 0)
            vv = *(const h16x8 *)(a.vc + (int64_t)vtok * v_tok + (int64_t)g * DV + vp * 8);
        {
            float acc[G];
#pragma unroll
            for (int h = 0; h < G; h++)
                acc[h] = dot8(*(const h16x8 *)&sm.qs[h * D + kp * 8], kv, 0.f);
#pragma unroll
            for (int h = 0; h < G; h++)
                acc[h] = row_group_sum<PK>(acc[h]);
            if (k_on && kp == 0) {
#pragma unroll
                for (int h = 0; h < G; h++)
                    sm.u.att.ps[h][kc] = ktok >= 0 ? acc[h] * sl2 : -INFINITY;
            }
        }
        if (v_on)
            *(h16x8 *)&sm.u.att.vs[vc * DV + vp * 8] = vv;
        __syncthreads();

        // softmax of head `wave` over the chunk (lane = cell).  The first chunk of
        // a split always holds a cell, so the running maximum is finite from then on
        if (wave < G) {
            const float s = sm.u.att.ps[wave][lane];
            const float m_old = sm.u.att.ml[wave][0];
            const float m = fmaxf(m_old, wave_max(s));
            const float alpha = exp2f(m_old - m);  // 0 for the first chunk
            const float p = (s == -INFINITY) ? 0.f : exp2f(s - m);
            sm.u.att.ps[wave][lane] = p;
            const float l = sm.u.att.ml[wave][1] * alpha + wave_sum(p);
            if (lane == 0) {
                sm.u.att.ml[wave][0] = m;
                sm.u.att.ml[wave][1] = l;
                sm.u.att.ml[wave][2] = alpha;
            }
        }
        __syncthreads();

        // thread (head, dim): o = o * alpha + sum over cells of p x v; cells past
        // the end have p = 0 and zeroed V rows
#pragma unroll
        for (int i = 0; i < OPT; i++) {
            const int o = t + i * kNT;
            if (o < G * DV) {
                const int h = o / DV, d = o % DV;
                float acc = oacc[i] * sm.u.att.ml[h][2];
#pragma unroll 4
                for (int c4 = 0; c4 < kAttnChunk; c4 += 4) {
                    const f32x4 p4 = *(const f32x4 *)&sm.u.att.ps[h][c4];
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        acc += p4[u] * (float)sm.u.att.vs[(c4 + u) * DV + d];
                }
                oacc[i] = acc;
            }
        }
        if (ch + 1 < chunks)
            __syncthreads();  // the next chunk overwrites ps and vs
    }
#pragma unroll
    for (int i = 0; i < OPT; i++) {
        const int o = t + i * kNT;
        if (o < G * DV) {
            const int h = o / DV, d = o % DV;
            float *pb = part + (((int64_t)g * G + h) * a.splits + split) * (DV + 2);
            if (d == 0) {
                pb[0] = sm.u.att.ml[h][0];
                pb[1] = sm.u.att.ml[h][1];
            }
            pb[2 + d] = oacc[i];
        }
    }
}

template <int D, int DV>
hipError_t launch_d(const TailArgs &a, int G, int rows, hipStream_t s)
{
    const dim3 grid((uint32_t)a.splits, (uint32_t)a.hkv, (uint32_t)rows);
    switch (G) {
    case 1: hipLaunchKernelGGL((step_tail_kernel<1, D, DV>), grid, dim3(kNT), 0, s, a); break;
    case 2: hipLaunchKernelGGL((step_tail_kernel<2, D, DV>), grid, dim3(kNT), 0, s, a); break;
    case 4: hipLaunchKernelGGL((step_tail_kernel<4, D, DV>), grid, dim3(kNT), 0, s, a); break;
    case 8: hipLaunchKernelGGL((step_tail_kernel<8, D, DV>), grid, dim3(kNT), 0, s, a); break;
    case 16: hipLaunchKernelGGL((step_tail_kernel<16, D, DV>), grid, dim3(kNT), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step_tail(const StepTail &st, hipStream_t s)
{
    const int32_t n_last = st.pos0 + st.rows;  // tokens seen by the last row
    if (st.rows < 1 || st.pos0 < 0 || st.k < 1 || st.k > kMaxTopk ||
        n_last / kBlockTokens > kMaxBlocks || st.n_lists < 1 || st.n_lists > kListWgs ||
        st.hq % st.hkv || st.scan_rpw < 1)
        return hipErrorInvalidValue;
    TailArgs a;
    a.cl = st.cl;
    a.n_lists = st.n_lists;
    a.scores = st.scores;
    a.ld = st.ld;
    a.pos0 = st.pos0;
    a.k = st.k;
    a.q = st.q;
    a.kc = st.k_cache;
    a.vc = st.v_cache;
    a.hq = st.hq;
    a.hkv = st.hkv;
    a.scale = st.scale;
    int32_t max_cells = 0;
    for (int32_t r = 0; r < st.rows; r++) {
        const int32_t n = st.pos0 + r + 1, nb = n / kBlockTokens;
        const int32_t c = kBlockTokens * (nb < st.k ? nb : st.k) + n % kBlockTokens;
        max_cells = c > max_cells ? c : max_cells;
    }
    // one 64-cell chunk per split, unless that would take more than one round of
    // work groups (one per CU, 256 CUs): then longer splits
    const int32_t n_chunks = (max_cells + kAttnChunk - 1) / kAttnChunk;
    const int64_t wgs = (int64_t)n_chunks * st.hkv * st.rows;
    a.chunks = (int32_t)((wgs + 255) / 256);
    a.chunks = a.chunks < 1 ? 1 : (a.chunks > kMaxChunks ? kMaxChunks : a.chunks);
    // never more splits than the partial buffer holds (k = 1024 has up to 65 chunks)
    const int32_t c_min = (n_chunks + kAttnMaxSplits - 1) / kAttnMaxSplits;
    a.chunks = a.chunks < c_min ? c_min : a.chunks;
    a.splits = (n_chunks + a.chunks - 1) / a.chunks;
    if (a.splits > kAttnMaxSplits)
        return hipErrorInvalidValue;
    a.part = st.part;
    a.blk_out = st.blk_out;
    a.scan_rpw = st.scan_rpw;
    const int G = st.hq / st.hkv;
    hipError_t e;
    if (st.d == 128 && st.dv == 128)
        e = launch_d<128, 128>(a, G, st.rows, s);
    else if (st.d == 64 && st.dv == 64)
        e = launch_d<64, 64>(a, G, st.rows, s);
    else
        return hipErrorInvalidValue;
    if (e != hipSuccess)
        return e;
    return launch_combine(st.part, st.hq, a.splits, st.dv, st.rows, st.out, s);
}

}  // namespace qsa
