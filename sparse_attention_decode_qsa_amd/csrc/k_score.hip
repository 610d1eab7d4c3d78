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
// flight per CU.  Work groups stride the rows in round-robin order so
// consecutive waves read consecutive rows.
//
// The decode step runs its append in the same launch: one extra work group
// copies the new token's rows, builds the pooled row of the block the token
// completes (if any) and scores that row with the same lane arithmetic as the
// scan, so the score is bit-identical to scanning the appended cache.  The
// scan work groups only read rows of blocks that were complete before.
#include "qsa_append.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Score of one row held in LDS, by one wave, in the scan's lane order.
template <int ROWC>
__device__ __forceinline__ void score_row_lds(const h16 *q, const h16 *row, float *out)
{
    constexpr int LPR = ROWC < kWave ? ROWC : kWave;
    constexpr int CPL = ROWC / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane % LPR;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; j++)
        acc = dot8(((const h16x8 *)q)[sub + LPR * j], ((const h16x8 *)row)[sub + LPR * j], acc);
    acc = group_sum<LPR>(acc);
    if (lane == 0)
        *out = acc;
}

template <int ROWC, int U, bool APPEND>
__global__ __launch_bounds__(kThreads) void score_decode_kernel(const h16 *__restrict__ q,
                                                                const h16 *__restrict__ pool,
                                                                int32_t nb,
                                                                float *__restrict__ scores,
                                                                AppendArgs ap)
{
    constexpr int LPR = ROWC < kWave ? ROWC : kWave;  // lanes per row
    constexpr int CPL = ROWC / LPR;                   // chunks per lane per row
    constexpr int RPW = kWave / LPR;                  // rows per wave per group
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int sub = lane % LPR;
    const int rsub = lane / LPR;

    if (APPEND && blockIdx.x == 0) {
        // append work group (dispatched first): [d/2] (cos, sin) pairs, then the pooled row
        extern __shared__ __align__(16) unsigned char lds[];
        f32x2 *cs = (f32x2 *)lds;
        h16 *row = (h16 *)(lds + sizeof(f32x2) * (ap.d / 2));
        append_copy(ap, 0, 1);
        if (ap.n_blocks == 1) {
            append_pool(ap, ap.b_lo, 1, cs, row);
            __syncthreads();
            if (wave == 0)
                score_row_lds<ROWC>(q, row, scores + ap.b_lo);
        }
        return;
    }

    h16x8 qv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; j++)
        qv[j] = ((const h16x8 *)q)[sub + LPR * j];

    const int64_t groups = ((int64_t)nb + RPW - 1) / RPW;
    const int64_t gw = (int64_t)(blockIdx.x - (APPEND ? 1 : 0)) * kWaves + wave;  // scan waves
    const int64_t tw = (int64_t)(gridDim.x - (APPEND ? 1 : 0)) * kWaves;
    const h16x8 *rows = (const h16x8 *)pool;

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
            for (int j = 0; j < CPL; j++)
                acc = dot8(qv[j], kv[u][j], acc);
            acc = group_sum<LPR>(acc);
            if (sub == 0 && r[u] < nb)
                scores[r[u]] = acc;
        }
    }
}

template <int ROWC>
hipError_t launch_rowc(const h16 *q, const h16 *pool, int32_t nb, float *scores,
                       const AppendArgs *ap, hipStream_t s)
{
    constexpr int U = ROWC >= 128 ? 2 : 4;
    constexpr int LPR = ROWC < kWave ? ROWC : kWave;
    constexpr int RPW = kWave / LPR;
    const int64_t groups = ((int64_t)nb + RPW - 1) / RPW;
    int64_t grid = (groups + (int64_t)kWaves * U - 1) / ((int64_t)kWaves * U);
    if (grid > 2048)
        grid = 2048;
    if (grid < 1)
        grid = 1;
    if (!ap) {
        const AppendArgs none{};
        hipLaunchKernelGGL((score_decode_kernel<ROWC, U, false>), dim3((uint32_t)grid),
                           dim3(kThreads), 0, s, q, pool, nb, scores, none);
    } else {
        const size_t lds = sizeof(f32x2) * (size_t)(ap->d / 2) + sizeof(h16) * (size_t)ROWC * 8;
        hipLaunchKernelGGL((score_decode_kernel<ROWC, U, true>), dim3((uint32_t)grid + 1),
                           dim3(kThreads), lds, s, q, pool, nb, scores, *ap);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_score_decode(const h16 *q, const h16 *pool, int32_t nb, int32_t row_elems,
                               float *scores, const AppendArgs *ap, hipStream_t s)
{
    if (nb <= 0 && !ap)
        return hipSuccess;
    // the fused append builds at most one pooled row, of the block right after
    // the scanned ones, in the layout the scan reads
    if (ap && (ap->n_blocks > 1 || (ap->n_blocks == 1 && ap->b_lo != nb) ||
               (int64_t)ap->H * ap->d != row_elems))
        return hipErrorInvalidValue;
    switch (row_elems / 8) {
    case 16: return launch_rowc<16>(q, pool, nb, scores, ap, s);
    case 32: return launch_rowc<32>(q, pool, nb, scores, ap, s);
    case 64: return launch_rowc<64>(q, pool, nb, scores, ap, s);
    case 128: return launch_rowc<128>(q, pool, nb, scores, ap, s);
    case 256: return launch_rowc<256>(q, pool, nb, scores, ap, s);
    case 512: return launch_rowc<512>(q, pool, nb, scores, ap, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qsa
