// Block scores for one decode query (Qiita part 10, "QSAとQSA indexerについて":
// each pooled summary is scored against the query; the score is the sum over
// indexer heads of the dot products).
//
// The pooled cache is the only O(N) stream of a decode step, so this kernel is
// the HBM-bound one.  Each row of the cache is ROWC 16-byte chunks.  A wave
// reads whole rows with one 16-byte load per lane per chunk (1 KiB per wave
// instruction, fully coalesced), keeps the query chunk that matches each lane in
// registers, accumulates with v_dot2_f32_f16 and reduces across the lanes of the
// row.  U row groups are loaded before any is consumed, to keep enough bytes in
// flight per CU.  Waves stride the rows in round-robin order, in runs of 4
// neighbouring row groups per work group.
//
// The decode step runs its append in the same launch: one extra work group
// copies the new token's rows, builds the pooled row of the block the token
// completes (if any) and scores that row with the same lane arithmetic as the
// scan, so the score is bit-identical to scanning the appended cache.  The
// scan work groups only read rows of blocks that were complete before.
//
// In the decode step every wave also keeps, per query row, the kListLen best
// (score, id) pairs of the rows it scored as 64-bit rank keys spread over 8 lanes
// (one entry per lane); the last wave of the work group to finish picks, per
// query row, the kListLen best of their union (in any order) and writes them, so
// the top-k reads a few thousand candidates per query row instead of the whole
// score row.
#include "qsa_append.h"

namespace qsa {
namespace {

constexpr int kThreads = 512;   // stand-alone scan: 8 waves per work group
constexpr int kStepThreads = 512;  // decode-step scan: 8 waves, so one list per 8 waves

// Sum of a row's lane partials: a whole-wave row by DPP within the 16-lane rows
// and the four row totals added in a fixed order (no LDS permutes); narrower rows
// by a butterfly within their lane group.  Every lane of the row gets the same
// value, and the scan and the appended row use this same order.
template <int LPR>
__device__ __forceinline__ float row_sum(float a)
{
    if constexpr (LPR == kWave)
        return wave_sum(a);
    else
        return group_sum<LPR>(a);
}

// Score of one row held in LDS, by one wave, in the scan's lane order; lane 0
// returns it.
template <int ROWC>
__device__ __forceinline__ float score_row_lds(const h16 *q, const h16 *row)
{
    constexpr int LPR = ROWC < kWave ? ROWC : kWave;
    constexpr int CPL = ROWC / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane % LPR;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; j++)
        acc = dot8(((const h16x8 *)q)[sub + LPR * j], ((const h16x8 *)row)[sub + LPR * j], acc);
    return row_sum<LPR>(acc);
}

// A wave's candidate lists live across its lanes: lane 8 g + i holds entry i of
// query g's descending list of kListLen rank keys (0 = empty).  Inserting x (the
// key of query g's score, the same in the 8 lanes of group g): slot i keeps its
// entry if x does not outrank it, else takes x or, when x also outranks the entry
// above, that entry (a shift down by one, through a DPP row shift).
static_assert(kListLen == 8, "8 lanes per list");
constexpr int kDppRowShr1 = 0x111;  // row_shr:1
__device__ __forceinline__ uint64_t lane_list_insert(uint64_t v, uint64_t x, int slot)
{
    const uint32_t plo =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, kDppRowShr1, 0xf, 0xf, false);
    const uint32_t phi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), kDppRowShr1, 0xf, 0xf, false);
    const uint64_t above = slot == 0 ? ~0ull : (((uint64_t)phi << 32) | plo);
    return x > v ? (x > above ? above : x) : v;
}

// A 64-bit value moved across lanes by a DPP pattern (both halves).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}
constexpr int kDppRowRor4 = 0x124;   // lane i takes lane i - 4 of its row
constexpr int kDppRowRor12 = 0x12C;  // lane i takes lane i + 4 of its row
constexpr int kDppRowMirrorC = 0x140;
constexpr int kDppRowHalfMirrorC = 0x141;
constexpr int kDppQuadXor1C = 0xb1, kDppQuadXor2C = 0x4e;

// The value of lane l ^ 16 (l ^ 32): the 16- (32-) lane swaps return, in every lane,
// its own value and its partner's; which is which depends on the lane's row (half).
__device__ __forceinline__ uint64_t lane_xor16_u64(uint64_t v, int lane)
{
    const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto b =
        __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    const bool odd_row = (lane & 16) != 0;
    return ((uint64_t)(odd_row ? b[0] : b[1]) << 32) | (odd_row ? a[0] : a[1]);
}
__device__ __forceinline__ uint64_t lane_xor32_u64(uint64_t v, int lane)
{
    const auto a = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto b =
        __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    const bool upper = (lane & 32) != 0;
    return ((uint64_t)(upper ? b[0] : b[1]) << 32) | (upper ? a[0] : a[1]);
}

// Sorts each 8-lane group of a bitonic sequence into descending order (compare-
// exchange at distances 4, 2, 1; the lower lane of a pair keeps the larger key).
__device__ __forceinline__ uint64_t bitonic8_desc(uint64_t e, int lane)
{
    const uint64_t dn = dpp_u64<kDppRowRor4>(e), up = dpp_u64<kDppRowRor12>(e);
    uint64_t p = (lane & 4) ? dn : up;
    e = ((lane & 4) == 0) == (e > p) ? e : p;
    p = dpp_u64<kDppQuadXor2C>(e);
    e = ((lane & 2) == 0) == (e > p) ? e : p;
    p = dpp_u64<kDppQuadXor1C>(e);
    e = ((lane & 1) == 0) == (e > p) ? e : p;
    return e;
}

// The 8 largest of 64 keys held one per lane, each 8-lane group sorted descending:
// three rounds of merging two sorted groups (each key against its partner group's
// key in mirrored position keeps the 8 largest of the two, as a bitonic sequence),
// the first two followed by a bitonic sort.  Lanes 0-7 end with the 8 largest, in
// no particular order.  All 64 lanes take part.
__device__ __forceinline__ uint64_t top8_of_64(uint64_t e, int lane)
{
    uint64_t p = dpp_u64<kDppRowMirrorC>(e);  // the other group of the row, reversed
    e = e > p ? e : p;
    e = bitonic8_desc(e, lane);
    p = dpp_u64<kDppRowHalfMirrorC>(lane_xor16_u64(e, lane));  // the paired row's, reversed
    e = e > p ? e : p;
    e = bitonic8_desc(e, lane);
    p = dpp_u64<kDppRowHalfMirrorC>(lane_xor32_u64(e, lane));  // the other half's, reversed
    return e > p ? e : p;
}

// NQ queries (rows of q, ROWC 16-byte chunks each) score every row read once;
// query i's scores go to scores[i * ld + b].  APPEND: work group 0 runs the
// append.  LISTS: candidate lists in the epilogue, one per query row (row i's at
// cl.list + i * kListWgs * kListLen, its row counts at cl.rows + i * kListWgs).
template <int ROWC, int U, int NT, int NQ, bool APPEND, bool LISTS>
__global__ __launch_bounds__(NT) void score_decode_kernel(const h16 *__restrict__ q,
                                                          const h16 *__restrict__ pool,
                                                          int32_t nb, float *__restrict__ scores,
                                                          int32_t ld, AppendArgs ap, CandLists cl)
{
    constexpr int NW = NT / kWave;
    constexpr int LPR = ROWC < kWave ? ROWC : kWave;  // lanes per row
    constexpr int CPL = ROWC / LPR;                   // chunks per lane per row
    constexpr int RPW = kWave / LPR;                  // rows per wave per group
    static_assert(!LISTS || APPEND, "candidate lists: the decode step");
    static_assert(!LISTS || NW * kListLen <= kWave, "one merged entry per lane of wave 0");
    static_assert(NQ >= 1 && NQ <= NW, "one wave per query for the appended row");
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int sub = lane % LPR;
    const int rsub = lane / LPR;

    if (APPEND && blockIdx.x == 0) {
        // append work group (dispatched first): [d/2] (cos, sin) pairs, then the pooled row
        extern __shared__ __align__(16) unsigned char lds[];
        f32x2 *cs = (f32x2 *)lds;
        h16 *row = (h16 *)(lds + sizeof(f32x2) * (ap.d / 2));
        append_copy<NT>(ap, 0, 1);
        uint64_t mine = 0;
        if (ap.n_blocks == 1) {
            append_pool<NT>(ap, ap.b_lo, 1, cs, row);
            __syncthreads();
            if (wave < NQ) {
                const float sc = score_row_lds<ROWC>(q + (int64_t)wave * ROWC * 8, row);
                if (lane == 0)
                    scores[(int64_t)wave * ld + ap.b_lo] = sc;
                mine = rank_key(sc, (uint32_t)ap.b_lo);
            }
        }
        if (LISTS && wave < NQ && lane < kListLen) {
            // query row `wave` (the token at n_before + wave) sees the new block
            // once its token completes it: that row's list holds it, the others
            // are empty
            const bool sees = ap.n_blocks == 1 &&
                              ap.n_before + wave >= kBlockTokens * ap.b_lo + (kBlockTokens - 1);
            const int64_t li = (int64_t)wave * kListWgs;
            cl.list[li * kListLen + lane] = (lane == 0 && sees) ? mine : 0ull;
            if (lane == 0)
                cl.rows[li] = sees ? 1u : 0u;
        }
        return;
    }

    __shared__ uint64_t wtop[LISTS ? NQ : 1][LISTS ? NW * kListLen : 1];
    __shared__ uint32_t wrows[NW];
    __shared__ uint32_t wdone;
    if (LISTS) {
        if (threadIdx.x == 0)
            wdone = 0;
        __syncthreads();
    }

    h16x8 qv[NQ][CPL];
#pragma unroll
    for (int qi = 0; qi < NQ; qi++)
#pragma unroll
        for (int j = 0; j < CPL; j++)
            qv[qi][j] = ((const h16x8 *)q)[qi * ROWC + sub + LPR * j];

    const int64_t groups = ((int64_t)nb + RPW - 1) / RPW;
    // scan wave index: runs of 4 consecutive row groups per work group (16 KiB
    // of neighbouring rows keeps the stream at full rate; runs of 2 or 1 do
    // not), the runs of one round spread over the work groups, so a run of
    // high-scoring neighbours puts at most 4 rows into any candidate list
    constexpr int kRun = NW < 4 ? NW : 4;
    const int64_t nwg = (int64_t)gridDim.x - (APPEND ? 1 : 0);
    const int64_t gw =
        ((int64_t)(wave / kRun) * nwg + (blockIdx.x - (APPEND ? 1 : 0))) * kRun + wave % kRun;
    const int64_t tw = nwg * NW;
    const h16x8 *rows = (const h16x8 *)pool;
    static_assert(!LISTS || NQ * kListLen <= kWave, "one list per 8 lanes");
    const int lgrp = lane / kListLen, lslot = lane % kListLen;
    uint64_t lst = 0ull;  // entry lslot of query lgrp's list
    uint32_t nrows = 0;

    for (int64_t g0 = gw; g0 < groups; g0 += tw * U) {
        h16x8 kv[U][CPL];
        int64_t r[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            r[u] = (g0 + (int64_t)u * tw) * RPW + rsub;
            const bool ok = r[u] < nb;
#pragma unroll
            for (int j = 0; j < CPL; j++) {
                if (ok)
                    kv[u][j] = __builtin_nontemporal_load(&rows[r[u] * ROWC + sub + LPR * j]);
                else
                    kv[u][j] = h16x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            float acc[NQ];
#pragma unroll
            for (int qi = 0; qi < NQ; qi++) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < CPL; j++)
                    a = dot8(qv[qi][j], kv[u][j], a);
                a = row_sum<LPR>(a);
                if (sub == 0 && r[u] < nb)
                    scores[(int64_t)qi * ld + r[u]] = a;
                acc[qi] = a;
            }
            if (LISTS) {
                // the RPW rows of this group, one at a time: lane group g inserts
                // query g's key
#pragma unroll
                for (int rs = 0; rs < RPW; rs++) {
                    const int64_t rr = (g0 + (int64_t)u * tw) * RPW + rs;
                    if (rr < nb) {
                        // one row per wave: the row sum left every query's score in
                        // every lane; otherwise read it from the row's lanes
                        float sc = 0.f;
#pragma unroll
                        for (int qi = 0; qi < NQ; qi++) {
                            const float s_q =
                                RPW == 1 ? acc[qi]
                                         : __int_as_float(__builtin_amdgcn_readlane(
                                               __float_as_int(acc[qi]), rs * LPR));
                            sc = lgrp == qi ? s_q : sc;
                        }
                        const uint64_t x = lgrp < NQ ? rank_key(sc, (uint32_t)rr) : 0ull;
                        lst = lane_list_insert(lst, x, lslot);
                        nrows++;
                    }
                }
            }
        }
    }

    if (LISTS) {
        // no barrier: each wave posts its list and counts itself done; the last
        // wave of the work group merges (earlier waves just end)
        if (lgrp < NQ)
            wtop[lgrp][wave * kListLen + lslot] = lst;
        if (lane == 0)
            wrows[wave] = nrows;
        uint32_t prev = 0;
        if (lane == 0)
            prev = __hip_atomic_fetch_add(&wdone, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
        if (prev == NW - 1) {
            // per query row, the kListLen largest of the NW * kListLen entries, one
            // per lane (each wave's list sorted, descending), by a merge network in
            // registers
            constexpr int NE = NW * kListLen;
            static_assert(!LISTS || NE == kWave, "one entry per lane");
            uint32_t n = 0;
#pragma unroll
            for (int w = 0; w < NW; w++)
                n += wrows[w];
#pragma unroll
            for (int qi = 0; qi < NQ; qi++) {
                const uint64_t best = top8_of_64(wtop[qi][lane], lane);
                const int64_t li = (int64_t)qi * kListWgs + blockIdx.x;
                if (lane < kListLen)
                    cl.list[li * kListLen + lane] = best;
                if (lane == 0)
                    cl.rows[li] = n;
            }
        }
    }
}

// Work groups of the decode-step scan, besides the append's: with the append work
// group, three per CU (8 waves each, 78 registers: the append's fp64 RoPE angles set
// the count), so every work group starts in the first round.
constexpr int64_t kStepScanWgs = 767;
static_assert(kStepScanWgs < kListWgs, "one list per thread of the top-k selection");

template <int ROWC, int NQ>
hipError_t launch_step(const h16 *q, const h16 *pool, int32_t nb, float *scores, int32_t ld,
                       const AppendArgs &ap, const CandLists *cl, int32_t *n_lists, hipStream_t s,
                       KernelEvents ev)
{
    constexpr int U = ROWC >= 128 ? 2 : 4;
    constexpr int LPR = ROWC < kWave ? ROWC : kWave;
    constexpr int RPW = kWave / LPR;
    constexpr int NW = kStepThreads / kWave;
    const int64_t groups = ((int64_t)nb + RPW - 1) / RPW;
    // one scan work group per 8 row groups (so every wave starts with a group), at
    // most kStepScanWgs of them
    int64_t grid = (groups + NW - 1) / NW;
    if (grid > kStepScanWgs)
        grid = kStepScanWgs;
    if (grid < 1)
        grid = 1;
    const size_t lds = sizeof(f32x2) * (size_t)(ap.d / 2) + sizeof(h16) * (size_t)ROWC * 8;
    if (cl) {
        launch_ev(score_decode_kernel<ROWC, U, kStepThreads, NQ, true, true>,
                  dim3((uint32_t)grid + 1), dim3(kStepThreads), lds, s, ev, q, pool, nb, scores,
                  ld, ap, *cl);
        *n_lists = (int32_t)grid + 1;
    } else {
        const CandLists nol{};
        launch_ev(score_decode_kernel<ROWC, U, kStepThreads, NQ, true, false>,
                  dim3((uint32_t)grid + 1), dim3(kStepThreads), lds, s, ev, q, pool, nb, scores,
                  ld, ap, nol);
    }
    return hipGetLastError();
}

template <int ROWC>
hipError_t launch_rowc(const h16 *q, int32_t n_q, const h16 *pool, int32_t nb, float *scores,
                       int32_t ld, const AppendArgs *ap, const CandLists *cl, int32_t *n_lists,
                       hipStream_t s, KernelEvents ev)
{
    if (!ap) {
        constexpr int U = ROWC >= 128 ? 2 : 4;
        constexpr int LPR = ROWC < kWave ? ROWC : kWave;
        constexpr int RPW = kWave / LPR;
        constexpr int NW = kThreads / kWave;
        const int64_t groups = ((int64_t)nb + RPW - 1) / RPW;
        // about 8 row groups per wave, 256 to 1,024 work groups of 8 waves (fewer when
        // there are fewer row groups than waves): measured at 31,898 to 255,181
        // tokens, the fewest beat the most by 1-2% on the short caches and lose
        // 0.5-1% on the long; 8-wave groups beat twice as many 4-wave ones by 1.5-2%
        int64_t grid = (groups + (int64_t)NW * 8 - 1) / ((int64_t)NW * 8);
        grid = grid > 1024 ? 1024 : (grid < 256 ? 256 : grid);
        const int64_t gmax = (groups + (int64_t)NW - 1) / NW;
        if (grid > gmax)
            grid = gmax;
        if (grid < 1)
            grid = 1;
        const AppendArgs none{};
        const CandLists nol{};
        launch_ev(score_decode_kernel<ROWC, U, kThreads, 1, false, false>, dim3((uint32_t)grid),
                  dim3(kThreads), 0, s, ev, q, pool, nb, scores, ld, none, nol);
        return hipGetLastError();
    }
    switch (n_q) {
    case 1: return launch_step<ROWC, 1>(q, pool, nb, scores, ld, *ap, cl, n_lists, s, ev);
    case 2: return launch_step<ROWC, 2>(q, pool, nb, scores, ld, *ap, cl, n_lists, s, ev);
    case 3: return launch_step<ROWC, 3>(q, pool, nb, scores, ld, *ap, cl, n_lists, s, ev);
    case 4: return launch_step<ROWC, 4>(q, pool, nb, scores, ld, *ap, cl, n_lists, s, ev);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int32_t scan_rows_per_group(int32_t row_elems)
{
    const int32_t rowc = row_elems / 8;  // 16-byte chunks per row
    return rowc >= kWave ? 1 : kWave / rowc;
}

hipError_t launch_score_decode(const h16 *q, int32_t n_q, const h16 *pool, int32_t nb,
                               int32_t row_elems, float *scores, int32_t ld, const AppendArgs *ap,
                               const CandLists *cl, int32_t *n_lists, hipStream_t s,
                               KernelEvents ev)
{
    if (nb <= 0 && !ap)
        return hipSuccess;
    // the fused append builds at most one pooled row, of the block right after the
    // scanned ones, in the layout the scan reads; candidate lists need the append
    if (n_q < 1 || n_q > 4 || (!ap && n_q != 1) || (cl && (!ap || !n_lists)) ||
        (ap && (ap->n_blocks > 1 || (ap->n_blocks == 1 && ap->b_lo != nb) ||
                (int64_t)ap->H * ap->d != row_elems)))
        return hipErrorInvalidValue;
    switch (row_elems / 8) {
    case 16: return launch_rowc<16>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s, ev);
    case 32: return launch_rowc<32>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s, ev);
    case 64: return launch_rowc<64>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s, ev);
    case 128: return launch_rowc<128>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s, ev);
    case 256: return launch_rowc<256>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s, ev);
    case 512: return launch_rowc<512>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s, ev);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qsa
