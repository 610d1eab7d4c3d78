// Selection building blocks shared by the top-k kernels (k_topk.hip) and the
// fused decode tail (k_step.hip): block-domain top-k in the sense of Qiita part
// 10, "QSAとQSA indexerについて" (keep the highest-scoring blocks) and the
// COMMON-006 section (select pools, then expand only the chosen ones).
//
// Scores are compared through score_key / rank_key (qsa_device.h); every
// result depends only on the fp32 scores, never on the order of atomics.
#pragma once

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kCandCap = 4096;
constexpr int kMaxBlocks = 1 << 19;  // bitmap of 64 KiB in LDS
constexpr int kSelThreads = 1024;    // work-group size of the list selection
constexpr int kSmallRank = 64;       // entries ranked by counting (one per lane of a wave)
static_assert(kListWgs <= kSelThreads, "one candidate list per thread");

template <int NT>
struct Scratch {
    uint32_t tmp[NT];
    uint32_t res[4];
    uint32_t cnt;
    uint32_t cnt2;
    uint32_t flag;
};

// Over NBINS (4096 or 256) LDS bins, finds the bin where the count taken from
// the top reaches need (need >= 1).  res[0] = bin (0xffffffff if the total is
// below need), res[1] = count in the bins above it, res[2] = total, res[3] =
// count in the bin.  All NT
// threads call it; wave 0 does the work: lane l sums bins [l*per, (l+1)*per), a
// wave scan finds the lane where the count from the top crosses need, and a
// second wave scan over that lane's bins finds the bin.  hist is 16-byte aligned;
// NBINS is 256 or 4096.
template <int NT, int NBINS>
__device__ void find_from_top(const uint32_t *hist, uint32_t need, Scratch<NT> &S)
{
    static_assert(NBINS == 256 || NBINS == 4096, "bins");
    if (threadIdx.x < kWave) {
        // opaque copy of the lane: keeps the compiler from hoisting the 64 bin
        // addresses out of a caller's loop (they would stay live and spill)
        uint32_t lane = threadIdx.x;
        asm volatile("" : "+v"(lane));
        constexpr int per = NBINS / kWave;  // 4 or 64
        uint32_t c = 0;
        if (per == 4) {
            const uint4 v = *(const uint4 *)(hist + lane * 4);
            c = v.x + v.y + v.z + v.w;
        } else {
            // rotated order: at step i the 64 lanes read 64 different banks; all
            // loads are issued before the sum
            uint32_t h[per];
#pragma unroll
            for (int i = 0; i < per; i++)
                h[i] = hist[lane * per + ((i + (int)lane) & (per - 1))];
#pragma unroll
            for (int i = 0; i < per; i++)
                c += h[i];
        }
        const uint32_t incl = wave_incl_scan(c);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
        const uint32_t above = total - incl;  // in the bins of the lanes above
        if (need > total) {
            if (lane == 0) {
                S.res[0] = 0xffffffffu;
                S.res[2] = total;
            }
        } else {
            const uint64_t m = __ballot(above < need && need <= above + c);
            const int L = __ffsll((unsigned long long)m) - 1;
            const uint32_t aboveL = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
            const uint32_t h = ((int)lane < per) ? hist[L * per + (int)lane] : 0u;
            const uint32_t incl2 = wave_incl_scan(h);
            const uint32_t tot2 = (uint32_t)__builtin_amdgcn_readlane((int)incl2, kWave - 1);
            const uint32_t above2 = aboveL + (tot2 - incl2);
            if ((int)lane < per && above2 < need && need <= above2 + h) {
                S.res[0] = (uint32_t)(L * per + (int)lane);
                S.res[1] = above2;
                S.res[3] = h;
            }
            if (lane == 0)
                S.res[2] = total;
        }
    }
    __syncthreads();
}

// As find_from_top for NBINS = 4 * NT, with every thread taking part: thread t
// owns bins 4t..4t+3, a work-group prefix sum (wave scans, then the NT/64 wave
// totals through wtot) gives the count in the bins of higher threads, and the
// one thread whose bins reach `need` finds the bin.  Sets res[0..3] as
// find_from_top does.
template <int NT>
__device__ void find_from_top_wg(const uint32_t *hist, uint32_t need, Scratch<NT> &S,
                                 uint32_t *wtot)
{
    constexpr int NW = NT / kWave;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const uint4 v = ((const uint4 *)hist)[t];
    const uint32_t c = v.x + v.y + v.z + v.w;
    const uint32_t incl = wave_incl_scan(c);
    if (lane == kWave - 1)
        wtot[w] = incl;
    __syncthreads();
    uint32_t total = 0, above = 0;
#pragma unroll
    for (int i = 0; i < NW; i++) {
        const uint32_t x = wtot[i];
        total += x;
        above += i > w ? x : 0u;
    }
    above += wtot[w] - incl;  // higher lanes of this wave
    if (need > total) {
        if (t == 0) {
            S.res[0] = 0xffffffffu;
            S.res[2] = total;
        }
    } else if (above < need && need <= above + c) {
        const uint32_t h[4] = {v.w, v.z, v.y, v.x};  // bins 4t+3 .. 4t
        uint32_t a = above;
        int i = 0;
        while (a + h[i] < need) {
            a += h[i];
            i++;
        }
        S.res[0] = (uint32_t)(4 * t + 3 - i);
        S.res[1] = a;
        S.res[2] = total;
        S.res[3] = h[i];
    }
    __syncthreads();
}

// Calls f(score_key(row[i]), i) for every i < nb, thread by thread in strides of
// NT.  The loads of kRowBatch strides are all issued (indexes clamped into the
// row) before the first key is used, so a pass over a row costs one memory round
// trip per batch rather than one per stride.
constexpr int kRowBatch = 8;
template <int NT, class F>
__device__ __forceinline__ void each_row_key(const float *row, uint32_t nb, F f)
{
    for (uint32_t i0 = threadIdx.x; i0 < nb; i0 += NT * kRowBatch) {
        float x[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; u++)
            x[u] = row[min(i0 + (uint32_t)(u * NT), nb - 1)];
#pragma unroll
        for (int u = 0; u < kRowBatch; u++)
            if (i0 + (uint32_t)(u * NT) < nb)
                f(score_key(x[u]), i0 + (uint32_t)(u * NT));
    }
}

// Candidate sources: each calls f(key, id) for every block of bin B.
template <int NT>
struct LdsCands {
    const uint64_t *c;
    uint32_t n;
    template <class F>
    __device__ void each(F f) const
    {
        for (uint32_t i = threadIdx.x; i < n; i += NT)
            f((uint32_t)(c[i] >> 32), (uint32_t)c[i]);
    }
};

template <int NT>
struct GlobalCands {
    const uint64_t *c;
    uint32_t n;
    template <class F>
    __device__ void each(F f) const
    {
        for (uint32_t i = threadIdx.x; i < n; i += NT) {
            const uint64_t v = c[i];
            f((uint32_t)(v >> 32), (uint32_t)v);
        }
    }
};

template <int NT>
struct RowCands {
    const float *row;
    uint32_t nb;
    uint32_t bin;
    template <class F>
    __device__ void each(F f) const
    {
        each_row_key<NT>(row, nb, [&](uint32_t key, uint32_t i) {
            if ((key >> (32 - kHistBits)) == bin)
                f(key, i);
        });
    }
};

// Exact threshold among the candidates: on return S.res[0] = T (key), S.res[1]
// = I (largest chosen id among keys equal to T).
template <int NT, class Src>
__device__ void resolve(const Src &src, uint32_t bin, uint32_t need, uint32_t nb, uint32_t *h256,
                        Scratch<NT> &S)
{
    uint32_t prefix = bin;
    int shift = 32 - kHistBits;
    const int widths[3] = {8, 8, 4};
    uint32_t last_count = 0;
    for (int p = 0; p < 3; p++) {
        const int w = widths[p];
        shift -= w;
        if (threadIdx.x < 256)
            h256[threadIdx.x] = 0;
        __syncthreads();
        const uint32_t pf = prefix, sh = (uint32_t)shift, mask = (1u << w) - 1u;
        src.each([&](uint32_t key, uint32_t) {
            if ((key >> (sh + w)) == pf)
                atomicAdd(&h256[(key >> sh) & mask], 1u);
        });
        __syncthreads();
        find_from_top<NT, 256>(h256, need, S);
        const uint32_t d = S.res[0];
        need -= S.res[1];
        last_count = h256[d];
        prefix = (prefix << w) | d;
        __syncthreads();
    }
    const uint32_t T = prefix;
    uint32_t I = 0xffffffffu;
    if (need < last_count) {
        // the `need` lowest ids among keys equal to T
        const int nbits = 32 - __clz((int)(nb - 1));
        const int top = ((nbits + 7) / 8) * 8;
        uint32_t ip = 0;
        for (int sh = top - 8; sh >= 0; sh -= 8) {
            if (threadIdx.x < 256)
                h256[threadIdx.x] = 0;
            __syncthreads();
            const uint32_t ipf = ip, s2 = (uint32_t)sh;
            src.each([&](uint32_t key, uint32_t id) {
                if (key == T && (s2 + 8 >= 32 || (id >> (s2 + 8)) == ipf))
                    atomicAdd(&h256[255u - ((id >> s2) & 255u)], 1u);
            });
            __syncthreads();
            find_from_top<NT, 256>(h256, need, S);
            const uint32_t d = 255u - S.res[0];
            need -= S.res[1];
            ip = (ip << 8) | d;
            __syncthreads();
        }
        I = ip;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        S.res[0] = T;
        S.res[1] = I;
    }
    __syncthreads();
}

// Exclusive prefix sum over the work group; returns this thread's offset.
template <int NT>
__device__ uint32_t wg_exclusive_scan(uint32_t v, Scratch<NT> &S)
{
    constexpr int NW = NT / kWave;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const uint32_t s = wave_incl_scan(v);
    __syncthreads();
    if (lane == kWave - 1)
        S.tmp[w] = s;
    __syncthreads();
    const uint32_t wt = lane < NW ? S.tmp[lane] : 0u;
    const uint32_t ws = wave_incl_scan(wt);
    const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(ws - wt), w);  // waves below
    __syncthreads();
    return base + s - v;
}

// Writes the ids of the set bits of bitmap[0 .. ceil(nb/32)) in ascending order;
// never more than cap of them.
template <int NT>
__device__ void compact_bitmap(const uint32_t *bitmap, uint32_t nb, int32_t *out, uint32_t cap,
                               Scratch<NT> &S)
{
    const uint32_t W = (nb + 31) / 32;
    const uint32_t per = (W + NT - 1) / NT;
    const uint32_t w0 = threadIdx.x * per;
    const uint32_t w1 = min(W, w0 + per);
    uint32_t c = 0;
    for (uint32_t w = w0; w < w1; w++)
        c += __popc(bitmap[w]);
    uint32_t pos = wg_exclusive_scan<NT>(c, S);
    for (uint32_t w = w0; w < w1; w++) {
        uint32_t m = bitmap[w];
        while (m) {
            const uint32_t b = (uint32_t)__ffs((int)m) - 1u;
            if (pos < cap)
                out[pos] = (int32_t)(w * 32 + b);
            pos++;
            m &= m - 1u;
        }
    }
}

__device__ void set_bit(uint32_t *bitmap, uint32_t id) { atomicOr(&bitmap[id >> 5], 1u << (id & 31)); }

template <int NT>
__device__ void zero_words(uint32_t *p, uint32_t n)
{
    for (uint32_t i = threadIdx.x; i < n; i += NT)
        p[i] = 0;
}

// Generic exact selection of one row straight from global memory (any nb up to
// kMaxBlocks): histogram pass, candidates of the threshold bin to LDS (or
// re-read from L2 when there are too many), digit passes, bitmap compaction.
template <int NT>
__device__ void select_row_global(const float *row, uint32_t nb, int32_t k, int32_t *outr,
                                  uint32_t *hist, uint64_t *cand, uint32_t *bitmap,
                                  Scratch<NT> &S)
{
    zero_words<NT>(hist, kHistBins);
    if (threadIdx.x == 0)
        S.cnt = 0;
    __syncthreads();
    each_row_key<NT>(row, nb,
                     [&](uint32_t key, uint32_t) { atomicAdd(&hist[key >> (32 - kHistBits)], 1u); });
    __syncthreads();
    find_from_top<NT, kHistBins>(hist, (uint32_t)k, S);
    const uint32_t B = S.res[0];
    const uint32_t need = (uint32_t)k - S.res[1];
    zero_words<NT>(bitmap, (nb + 31) / 32);
    __syncthreads();
    each_row_key<NT>(row, nb, [&](uint32_t key, uint32_t i) {
        const uint32_t bin = key >> (32 - kHistBits);
        if (bin > B) {
            set_bit(bitmap, i);
        } else if (bin == B) {
            const uint32_t slot = atomicAdd(&S.cnt, 1u);
            if (slot < kCandCap)
                cand[slot] = ((uint64_t)key << 32) | i;
        }
    });
    __syncthreads();
    const uint32_t c = S.cnt;
    uint32_t *h256 = hist;  // the 12-bit histogram is no longer needed
    if (c <= (uint32_t)kCandCap) {
        LdsCands<NT> src{cand, c};
        resolve<NT>(src, B, need, nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    } else {
        RowCands<NT> src{row, nb, B};
        resolve<NT>(src, B, need, nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    }
    __syncthreads();
    compact_bitmap<NT>(bitmap, nb, outr, (uint32_t)k, S);
}

// ---------------------------------------------------------------- list selection
// Exact top-k from the decode scan's candidate lists: thread t < W holds list t
// (kListLen rank keys, any order, 0 = empty) in R and its work group's row
// count in nrows.
//   1. R*, the k-th largest rank key of the lists: 4096-bucket histograms over
//      the range of the live score keys (the whole range of the lists' keys
//      first, then the chosen bucket; equal-width buckets over the actual
//      range keep the LDS atomics spread out, where fixed float-bit digits
//      would pile the candidates into a few bins), then digits of the block id
//      when one key is shared by many entries, until at most 64 entries are
//      live; those are ranked by counting.  Rank keys are distinct (ids are),
//      so R* is exact and the chosen set is {R >= R*};
//   2. a full list (its work group scored more than kListLen rows) whose
//      smallest key is >= R* may hide chosen rows of that work group (checked
//      on the per-wave maxima of those smallest keys); then the lists are not
//      enough (kListsHide): the caller widens those lists with their work
//      groups' rows (widen_lists) and selects again, or, when the rows do not
//      fit, selects from the whole score row.  Otherwise every row outside the
//      lists ranks below the smallest key of its own list, hence below R*, and
//      the lists hold the top-k exactly.
// A list that may hide rows holds kListLen keys >= R*, and only k keys are, so at
// most k / kListLen lists need widening: 128 at k = 1024.
constexpr int kMaxWiden = 128;
struct alignas(16) ListSelLds {
    alignas(16) uint32_t hist[2][kHistBins];
    uint64_t small[kSmallRank];
    Scratch<kSelThreads> S;
    uint32_t wtot[kSelThreads / kWave];
    uint64_t wlast[kSelThreads / kWave];
    alignas(16) uint32_t wkey[2][kSelThreads / kWave];
    uint64_t rstar;
    uint32_t hidden;
    uint32_t widen[kMaxWiden];  // work groups whose rows replace their lists
};

// Outcome of lists_select_rest.
enum ListSel : int { kListsExact = 0, kListsHide = 1, kListsShort = 2 };

// The part of the selection before its first barrier: clears the histograms and
// writes each wave's key range and largest full-list minimum.  All kSelThreads
// threads call it; a barrier must follow before lists_select_rest.
__device__ void lists_prepare(const uint64_t (&R)[kListLen], uint32_t nrows, bool has_list,
                              ListSelLds &L)
{
    const int t = threadIdx.x;
    Scratch<kSelThreads> &S = L.S;
    ((uint4 *)L.hist[0])[t] = uint4{0, 0, 0, 0};
    ((uint4 *)L.hist[1])[t] = uint4{0, 0, 0, 0};
    if (t == 0)
        S.cnt = 0;
    // per wave: the smallest and largest score key of the nonempty entries, and
    // the largest smallest entry of a full list (for step 2)
    {
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        uint64_t last = ~0ull;
#pragma unroll
        for (int j = 0; j < kListLen; j++) {
            const uint32_t key = (uint32_t)(R[j] >> 32);
            if (R[j] != 0ull) {
                kmin = min(kmin, key);
                kmax = max(kmax, key);
            }
            last = R[j] < last ? R[j] : last;
        }
        if (!(has_list && nrows > (uint32_t)kListLen))
            last = 0ull;
        last = wave_max_u64(last);
        kmin = wave_min_u32(kmin);
        kmax = wave_max_u32(kmax);
        if ((t & (kWave - 1)) == 0) {
            L.wlast[t / kWave] = last;
            L.wkey[0][t / kWave] = kmin;
            L.wkey[1][t / kWave] = kmax;
        }
    }
}

// The rest of the selection, after lists_prepare and a barrier.  All kSelThreads
// threads call it with the same R.  Returns kListsExact (the lists hold the top-k;
// *rs = R*), kListsHide (a full list may hide chosen rows; *rs = R* of the lists)
// or kListsShort (fewer than k keys in the lists).  Leaves L.hist cleared.
__device__ int lists_select_rest(const uint64_t (&R)[kListLen], uint32_t k, ListSelLds &L,
                                 uint64_t *rs)
{
    constexpr int NT = kSelThreads;
    const int t = threadIdx.x;
    Scratch<NT> &S = L.S;

    // 1. key passes over [lo, lo + span] in 4096 buckets ((key - lo) >> s), then
    // id digits (bits 18..0 of the id; bits 31..19 of ~id are 1 for every id
    // below kMaxBlocks = 2^19) in 8, 8 and 3 bits, (imask, ival) the low-word
    // bits fixed so far
    static_assert(kMaxBlocks == 1 << 19, "id digits cover 19 bits");
    uint32_t lo = 0xffffffffu, hi_key = 0u;
#pragma unroll
    for (int i = 0; i < NT / kWave; i += 4) {
        const uint4 a = *(const uint4 *)&L.wkey[0][i], b = *(const uint4 *)&L.wkey[1][i];
        lo = min(min(lo, min(a.x, a.y)), min(a.z, a.w));
        hi_key = max(max(hi_key, max(b.x, b.y)), max(b.z, b.w));
    }
    uint32_t span = hi_key - lo;
    uint32_t imask = 0u, ival = 0u;
    auto live = [&](uint64_t r) {
        const uint32_t key = (uint32_t)(r >> 32);
        return r != 0ull && key >= lo && key - lo <= span && ((uint32_t)r & imask) == ival;
    };
    uint32_t need = k, cnt = 0;
    if (hi_key < lo)  // no entry at all
        return kListsShort;
    int p = 0;
    for (;;) {
        const int s = span >= (uint32_t)kHistBins ? 32 - __clz((int)span) - kHistBits : 0;
        uint32_t *h = L.hist[p & 1];
#pragma unroll
        for (int j = 0; j < kListLen; j++)
            if (live(R[j]))
                atomicAdd(&h[((uint32_t)(R[j] >> 32) - lo) >> s], 1u);
        __syncthreads();
        find_from_top_wg<NT>(h, need, S, L.wtot);
        const uint32_t d = S.res[0];
        if (d == 0xffffffffu)  // fewer than k keys in the lists
            return kListsShort;
        need -= S.res[1];
        cnt = S.res[3];
        // nobody reads h again in this pass; the next pass uses the other one
        ((uint4 *)h)[t] = uint4{0, 0, 0, 0};
        p++;
        lo += d << s;
        span = s == 0 ? 0u : min(span - (d << s), (1u << s) - 1u);
        if (span == 0 || cnt <= (uint32_t)kSmallRank)
            break;
    }
    if (cnt > (uint32_t)kSmallRank) {
        // one key, many entries: id digits
        imask = 0xfff80000u;
        ival = 0xfff80000u;
        const int shifts[3] = {11, 3, 0};
        const int widths[3] = {8, 8, 3};
        for (int q = 0; q < 3; q++) {
            const int w = widths[q], sh = shifts[q];
            uint32_t *h = L.hist[p & 1];
#pragma unroll
            for (int j = 0; j < kListLen; j++)
                if (live(R[j]))
                    atomicAdd(&h[((uint32_t)R[j] >> sh) & ((1u << w) - 1u)], 1u);
            __syncthreads();
            find_from_top<NT, 256>(h, need, S);
            const uint32_t d = S.res[0];
            need -= S.res[1];
            cnt = S.res[3];
            if (t < 64)
                ((uint4 *)h)[t] = uint4{0, 0, 0, 0};
            p++;
            imask |= ((1u << w) - 1u) << sh;
            ival |= d << sh;
            if (cnt <= (uint32_t)kSmallRank)
                break;
        }
    }
    // the <= 64 live entries; R* is the one with `need - 1` of them above it
#pragma unroll
    for (int j = 0; j < kListLen; j++) {
        if (live(R[j])) {
            const uint32_t slot = atomicAdd(&S.cnt, 1u);
            if (slot < (uint32_t)kSmallRank)
                L.small[slot] = R[j];
        }
    }
    __syncthreads();
    if (t < kWave) {
        const uint64_t me = (uint32_t)t < cnt ? L.small[t] : 0ull;
        uint32_t above = 0;
        for (uint32_t j = 0; j < cnt; j++)
            above += L.small[j] > me ? 1u : 0u;
        const bool is_rs = (uint32_t)t < cnt && above == need - 1u;
        if (is_rs)
            L.rstar = me;
        // 2. a full list whose smallest key is chosen may hide chosen rows
        const uint64_t last = t < NT / kWave ? L.wlast[t] : 0ull;
        const uint64_t r = __shfl(me, __ffsll((unsigned long long)__ballot(is_rs)) - 1, kWave);
        const bool hid = __ballot(last >= r) != 0ull;
        if (t == 0)
            L.hidden = hid ? 1u : 0u;
    }
    __syncthreads();
    *rs = L.rstar;
    return L.hidden == 0u ? kListsExact : kListsHide;
}

// The whole selection: lists_prepare, a barrier, lists_select_rest.
__device__ int lists_select(const uint64_t (&R)[kListLen], uint32_t nrows, bool has_list,
                            uint32_t k, ListSelLds &L, uint64_t *rs)
{
    lists_prepare(R, nrows, has_list, L);
    __syncthreads();
    return lists_select_rest(R, k, L, rs);
}

// The rows behind a set of candidate lists: list li >= base was written by the
// work group b = li - base, which owns the rows r < n_rows whose group g = r / rpw
// lies in its runs of 4 groups, 4 b + 4 nwg m .. 4 b + 4 nwg m + 3 (m = 0, 1, ...);
// lists below base own no such rows (the decode scan's list 0 is its append's).
struct ListLayout {
    int32_t base;
    int32_t nwg;
    int32_t rpw;
    uint32_t n_rows;
};

// Targeted fallback, after lists_select_rest returned kListsHide with rs = R* of
// the lists: every full list whose smallest key is >= R* is dropped, and all rows
// of its work group (their scores re-read from the score row) go to the threads
// past the W lists, kListLen rows each, as lists that hide nothing.  The top-k of
// the widened set is the true top-k: adding candidates cannot lower the k-th key,
// so a list that hid nothing before (not full, or its smallest key below R*) hides
// nothing after, and the dropped lists' work groups are now complete.  Returns
// false, leaving R as it was, when those rows do not fit the spare threads (the
// caller then selects from the whole score row).  All kSelThreads threads call it;
// lists_prepare (after a barrier) and lists_select_rest then run on the new R.
__device__ bool widen_lists(uint64_t (&R)[kListLen], uint32_t *nrows, int32_t W, uint64_t rs,
                            const float *scores, const ListLayout &lay, ListSelLds &L)
{
    constexpr int NT = kSelThreads;
    const int t = threadIdx.x;
    Scratch<NT> &S = L.S;
    if (lay.nwg < 1 || lay.rpw < 1 || lay.n_rows == 0u)
        return false;
    // rows of one work group at most, and the threads that take them
    const uint32_t rpw = (uint32_t)lay.rpw, nwg = (uint32_t)lay.nwg;
    const uint32_t groups = (lay.n_rows + rpw - 1u) / rpw;
    const uint32_t per = 4u * ((groups + 4u * nwg - 1u) / (4u * nwg)) * rpw;
    const uint32_t P = (per + kListLen - 1u) / kListLen;
    uint64_t mn = ~0ull;
#pragma unroll
    for (int j = 0; j < kListLen; j++)
        mn = R[j] < mn ? R[j] : mn;
    const bool hides = t < W && t >= lay.base && *nrows > (uint32_t)kListLen && mn >= rs;
    // the dropped lists in list order (a prefix sum, not atomics: every work group
    // that runs this selection must hand the same rows to the same threads, since
    // the chosen blocks are placed in thread order)
    const uint32_t o = wg_exclusive_scan<NT>(hides ? 1u : 0u, S);
    if (t == NT - 1)
        S.cnt = o + (hides ? 1u : 0u);
    if (hides && o < (uint32_t)kMaxWiden)
        L.widen[o] = (uint32_t)(t - lay.base);
    __syncthreads();
    const uint32_t n_off = S.cnt;
    if (n_off == 0u || n_off > (uint32_t)kMaxWiden || W > NT ||
        (uint64_t)n_off * P > (uint64_t)(NT - W))
        return false;  // the same on every thread
    if (hides) {
#pragma unroll
        for (int j = 0; j < kListLen; j++)
            R[j] = 0ull;
        *nrows = 0u;
    }
    const int sp = t - W;
    if (sp >= 0 && (uint32_t)sp < n_off * P) {
        const uint32_t b = L.widen[(uint32_t)sp / P], part = (uint32_t)sp % P;
        uint32_t r[kListLen];
        float v[kListLen];
#pragma unroll
        for (int e = 0; e < kListLen; e++) {
            const uint32_t j = part * kListLen + (uint32_t)e;  // the work group's j-th row
            const uint32_t jg = j / rpw;
            const uint32_t g = 4u * b + (jg & 3u) + 4u * nwg * (jg >> 2);
            r[e] = j < per ? g * rpw + j % rpw : 0xffffffffu;
            v[e] = scores[r[e] < lay.n_rows ? r[e] : lay.n_rows - 1u];  // all loads in flight
        }
        uint32_t n = 0;
#pragma unroll
        for (int e = 0; e < kListLen; e++) {
            const bool on = r[e] < lay.n_rows;
            R[e] = on ? rank_key(v[e], r[e]) : 0ull;
            n += on ? 1u : 0u;
        }
        *nrows = n;
    }
    return true;
}

// Issues the loads of list min(t, W - 1) and its row count (W >= 1): no branch,
// so the loads stay in flight while the caller issues others.  Threads t >= W
// must call drop_absent_list before using R.
__device__ void load_list_raw(const CandLists &cl, int32_t W, uint64_t (&R)[kListLen],
                              uint32_t *nrows)
{
    const int t = threadIdx.x < W ? (int)threadIdx.x : W - 1;
    const uint4 *src = (const uint4 *)(cl.list + (int64_t)t * kListLen);
#pragma unroll
    for (int j = 0; j < kListLen / 2; j++) {
        const uint4 v = src[j];
        R[2 * j] = ((uint64_t)v.y << 32) | v.x;
        R[2 * j + 1] = ((uint64_t)v.w << 32) | v.z;
    }
    *nrows = cl.rows[t];
}

// Empties the list of a thread that holds none (t >= W).
__device__ void drop_absent_list(int32_t W, uint64_t (&R)[kListLen], uint32_t *nrows)
{
    const bool on = (int)threadIdx.x < W;
#pragma unroll
    for (int j = 0; j < kListLen; j++)
        R[j] = on ? R[j] : 0ull;
    *nrows = on ? *nrows : 0u;
}

// Loads list t (thread t < W) and its row count; empty otherwise.
__device__ void load_list(const CandLists &cl, int32_t W, uint64_t (&R)[kListLen], uint32_t *nrows)
{
    load_list_raw(cl, W, R, nrows);
    drop_absent_list(W, R, nrows);
}

}  // namespace
}  // namespace qsa
