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
// In the decode step every wave also keeps the kListLen best (score, id) pairs
// of the rows it scored, as wave-uniform 64-bit rank keys; the last wave of the
// work group to finish picks the kListLen best of their union (in any order)
// and writes them, so the top-k launch reads a few thousand candidates instead
// of the whole row.
#include "qsa_append.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;   // stand-alone scan
constexpr int kStepThreads = 512;  // decode-step scan: 8 waves, so one list per 8 waves

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
    return group_sum<LPR>(acc);
}

// Inserts x into the descending list top[0..kListLen).
__device__ __forceinline__ void list_insert(uint64_t (&top)[kListLen], uint64_t x)
{
    if (x > top[kListLen - 1]) {
        top[kListLen - 1] = x;
#pragma unroll
        for (int i = kListLen - 1; i > 0; i--) {
            const uint64_t a = top[i - 1], b = top[i];
            top[i - 1] = a > b ? a : b;
            top[i] = a > b ? b : a;
        }
    }
}

// NQ queries (rows of q, ROWC 16-byte chunks each) score every row read once;
// query i's scores go to scores[i * ld + b].  APPEND: work group 0 runs the
// append.  LISTS (one query): candidate lists in the epilogue.
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
    static_assert(!LISTS || (APPEND && NQ == 1), "candidate lists: the one-query decode step");
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
        if (LISTS) {
            // its list: the new block (if any), then empty slots
            if (wave == 0 && lane < kListLen)
                cl.list[lane] = lane == 0 ? mine : 0ull;
            if (threadIdx.x == 0)
                cl.rows[0] = (uint32_t)ap.n_blocks;
        }
        return;
    }

    __shared__ uint64_t wtop[LISTS ? NW * kListLen : 1];
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
    uint64_t top[kListLen];
#pragma unroll
    for (int i = 0; i < kListLen; i++)
        top[i] = 0ull;
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
            float acc = 0.f;
#pragma unroll
            for (int qi = 0; qi < NQ; qi++) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < CPL; j++)
                    a = dot8(qv[qi][j], kv[u][j], a);
                a = group_sum<LPR>(a);
                if (sub == 0 && r[u] < nb)
                    scores[(int64_t)qi * ld + r[u]] = a;
                acc = a;
            }
            if (LISTS) {
                // the RPW rows of this group, one at a time, as wave-uniform values
#pragma unroll
                for (int rs = 0; rs < RPW; rs++) {
                    const int64_t rr = (g0 + (int64_t)u * tw) * RPW + rs;
                    if (rr < nb) {
                        const float sc =
                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), rs * LPR));
                        list_insert(top, rank_key(sc, (uint32_t)rr));
                        nrows++;
                    }
                }
            }
        }
    }

    if (LISTS) {
        // no barrier: each wave posts its list and counts itself done; the last
        // wave of the work group merges (earlier waves just end)
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < kListLen; i++)
                wtop[wave * kListLen + i] = top[i];
            wrows[wave] = nrows;
        }
        uint32_t prev = 0;
        if (lane == 0)
            prev = __hip_atomic_fetch_add(&wdone, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
        if (prev == NW - 1) {
            // the kListLen largest of the NW * kListLen entries, one per lane,
            // found in registers: a bitwise search with ballots for the
            // kListLen-th largest score key, then (only if it is tied) for the
            // low word among the entries with that key
            constexpr int NE = NW * kListLen;
            const uint64_t me = lane < NE ? wtop[lane] : 0ull;
            const uint32_t hi = (uint32_t)(me >> 32), lo = (uint32_t)me;
            uint32_t th = 0;
            for (int bit = 31; bit >= 0; bit--) {
                const uint32_t c = th | (1u << bit);
                if (__popcll(__ballot(hi >= c)) >= kListLen)
                    th = c;
            }
            uint32_t tl = 0;
            const uint32_t n_above = (uint32_t)__popcll(__ballot(hi > th));
            if (__popcll(__ballot(hi >= th)) > kListLen) {
                const uint32_t want = kListLen - n_above;
                for (int bit = 31; bit >= 0; bit--) {
                    const uint32_t c = tl | (1u << bit);
                    if ((uint32_t)__popcll(__ballot(hi == th && lo >= c)) >= want)
                        tl = c;
                }
            }
            // chosen: > (th, tl); empty entries (0) never; the list keeps them in
            // lane order, the rest of its slots empty
            const uint64_t thr = ((uint64_t)th << 32) | tl;
            const bool pick = me != 0ull && me >= thr;
            const uint64_t pm = __ballot(pick);
            const uint32_t slot = (uint32_t)__popcll(pm & ((1ull << lane) - 1ull));
            const uint32_t npick = (uint32_t)__popcll(pm);
            uint64_t *dst = cl.list + (int64_t)blockIdx.x * kListLen;
            if (pick && slot < (uint32_t)kListLen)
                dst[slot] = me;
            if ((uint32_t)lane >= npick && lane < kListLen)
                dst[lane] = 0ull;
            if (lane == 0) {
                uint32_t n = 0;
#pragma unroll
                for (int w = 0; w < NW; w++)
                    n += wrows[w];
                cl.rows[blockIdx.x] = n;
            }
        }
    }
}

template <int ROWC, int NQ>
hipError_t launch_step(const h16 *q, const h16 *pool, int32_t nb, float *scores, int32_t ld,
                       const AppendArgs &ap, const CandLists *cl, int32_t *n_lists, hipStream_t s)
{
    constexpr int U = ROWC >= 128 ? 2 : 4;
    constexpr int LPR = ROWC < kWave ? ROWC : kWave;
    constexpr int RPW = kWave / LPR;
    constexpr int NW = kStepThreads / kWave;
    const int64_t groups = ((int64_t)nb + RPW - 1) / RPW;
    // one scan work group per 8 row groups (so every wave starts with a group), at
    // most kListWgs - 1 of them: the lists, the append work group's included, fit
    // one per thread of the top-k selection
    int64_t grid = (groups + NW - 1) / NW;
    if (grid > kListWgs - 1)
        grid = kListWgs - 1;
    if (grid < 1)
        grid = 1;
    const size_t lds = sizeof(f32x2) * (size_t)(ap.d / 2) + sizeof(h16) * (size_t)ROWC * 8;
    if (cl) {
        hipLaunchKernelGGL((score_decode_kernel<ROWC, U, kStepThreads, 1, true, true>),
                           dim3((uint32_t)grid + 1), dim3(kStepThreads), lds, s, q, pool, nb,
                           scores, ld, ap, *cl);
        *n_lists = (int32_t)grid + 1;
    } else {
        const CandLists nol{};
        hipLaunchKernelGGL((score_decode_kernel<ROWC, U, kStepThreads, NQ, true, false>),
                           dim3((uint32_t)grid + 1), dim3(kStepThreads), lds, s, q, pool, nb,
                           scores, ld, ap, nol);
    }
    return hipGetLastError();
}

template <int ROWC>
hipError_t launch_rowc(const h16 *q, int32_t n_q, const h16 *pool, int32_t nb, float *scores,
                       int32_t ld, const AppendArgs *ap, const CandLists *cl, int32_t *n_lists,
                       hipStream_t s)
{
    if (!ap) {
        constexpr int U = ROWC >= 128 ? 2 : 4;
        constexpr int LPR = ROWC < kWave ? ROWC : kWave;
        constexpr int RPW = kWave / LPR;
        constexpr int NW = kThreads / kWave;
        const int64_t groups = ((int64_t)nb + RPW - 1) / RPW;
        int64_t grid = (groups + (int64_t)NW * U - 1) / ((int64_t)NW * U);
        if (grid > 2048)
            grid = 2048;
        if (grid < 1)
            grid = 1;
        const AppendArgs none{};
        const CandLists nol{};
        hipLaunchKernelGGL((score_decode_kernel<ROWC, U, kThreads, 1, false, false>),
                           dim3((uint32_t)grid), dim3(kThreads), 0, s, q, pool, nb, scores, ld,
                           none, nol);
        return hipGetLastError();
    }
    switch (n_q) {
    case 1: return launch_step<ROWC, 1>(q, pool, nb, scores, ld, *ap, cl, n_lists, s);
    case 2: return launch_step<ROWC, 2>(q, pool, nb, scores, ld, *ap, nullptr, n_lists, s);
    case 3: return launch_step<ROWC, 3>(q, pool, nb, scores, ld, *ap, nullptr, n_lists, s);
    case 4: return launch_step<ROWC, 4>(q, pool, nb, scores, ld, *ap, nullptr, n_lists, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_score_decode(const h16 *q, int32_t n_q, const h16 *pool, int32_t nb,
                               int32_t row_elems, float *scores, int32_t ld, const AppendArgs *ap,
                               const CandLists *cl, int32_t *n_lists, hipStream_t s)
{
    if (nb <= 0 && !ap)
        return hipSuccess;
    // the fused append builds at most one pooled row, of the block right after the
    // scanned ones, in the layout the scan reads; candidate lists for one query only
    if (n_q < 1 || n_q > 4 || (!ap && n_q != 1) || (cl && (n_q != 1 || !n_lists)) ||
        (ap && (ap->n_blocks > 1 || (ap->n_blocks == 1 && ap->b_lo != nb) ||
                (int64_t)ap->H * ap->d != row_elems)))
        return hipErrorInvalidValue;
    switch (row_elems / 8) {
    case 16: return launch_rowc<16>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s);
    case 32: return launch_rowc<32>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s);
    case 64: return launch_rowc<64>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s);
    case 128: return launch_rowc<128>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s);
    case 256: return launch_rowc<256>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s);
    case 512: return launch_rowc<512>(q, n_q, pool, nb, scores, ld, ap, cl, n_lists, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qsa
