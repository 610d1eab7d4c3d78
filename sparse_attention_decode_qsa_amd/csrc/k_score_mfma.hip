// Block scores for a prefill chunk: S = Q_idx * P^T, a dense contraction over
// the h_idx*d_idx features (Qiita part 10, "QSAとQSA indexerについて": each query
// scores every pooled summary it can see), run on the gfx950 matrix cores.
//
// Both operands are feature-contiguous (Q_idx rows and pooled rows), which is
// exactly the per-lane operand layout of v_mfma_f32_16x16x32_f16: a lane holds
// 8 consecutive features of one row of A and of one column of B.
//
// Tiling: a work group computes a 256 (queries) x 256 (blocks) tile; its 8
// waves each own 128 x 64 (8 x 4 MFMA tiles, 128 fp32 accumulators per lane).
// Every 64-feature step stages A (32 KiB) and B (32 KiB) in LDS with rows padded
// to 144 bytes (16-byte fragment reads); 8 threads copy one row's 128
// bytes, so each step fetches whole 128-byte lines (32-feature steps fetched half a
// line per step and the other half one step later, 6% slower).  Two LDS buffers and
// two register sets: while step s is multiplied (two MFMA substeps of 32 features),
// step s + 1 waits in registers to be stored into the other buffer and the global
// loads of step s + 2 are in flight, and a step needs one barrier.  Every load is
// issued unconditionally (indexes clamped into the operands), so the compiler waits
// only for the oldest register set: a load under a branch made it wait for all of
// them.  Blocks at or past the last row's causal bound are never written.
//
// On this shape (1,024 queries x 31,819 blocks x 2,048 features) the matrix cores
// are busy about 43% of the kernel's time.  What holds them back is the staging of
// the operands, not the fragment reads: at this pitch the reads run into two-way
// bank conflicts (128 bytes per clock per CU), yet a 160-byte pitch that removes
// every conflict (and a third of the LDS's busy cycles) left the time unchanged,
// while the same loop with the steps' global loads and LDS stores taken out ran
// in about 0.8 of it; the score tile's fp32 stores (130 MB per chunk) add ~10%.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 512;
constexpr int TM = 256, TN = 256, TK = 64;
constexpr int PITCH = TK + 8;  // halfs per LDS row (144 bytes)
constexpr int WM = 128, WN = 64;
constexpr int FI = WM / 16, FJ = WN / 16;

// Tile order: the 1-D grid is dealt to the 8 XCDs round-robin (work group i runs
// on XCD i mod 8), and each XCD takes its work groups in order.  Work group i is
// mapped so that an XCD's consecutive work groups are the row tiles of one
// block-column tile, c = 8 * (j / nrow) + (i mod 8) with j = i / 8: those tiles run
// side by side on one L2, which then fetches the column's pooled rows once.
constexpr int kXcds = 8;
constexpr int NS = 2;  // register sets: a step's loads are issued NS steps ahead

__global__ __launch_bounds__(kThreads, 1) void score_prefill_kernel(const h16 *__restrict__ Q,
                                                                 int32_t n_q, int32_t pos0,
                                                                 const h16 *__restrict__ P,
                                                                 int32_t K, float *__restrict__ S,
                                                                 int32_t ld, int32_t ncol,
                                                                 int32_t nrow)
{
    __shared__ __attribute__((aligned(16))) h16 As[2][TM * PITCH];
    __shared__ __attribute__((aligned(16))) h16 Bs[2][TN * PITCH];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int32_t j = (int32_t)blockIdx.x / kXcds;
    const int32_t col = kXcds * (j / nrow) + (int32_t)blockIdx.x % kXcds;
    if (col >= ncol)
        return;
    const int32_t r0 = (j % nrow) * TM;
    const int32_t c0 = col * TN;
    const int32_t nb_max = (pos0 + n_q) / kBlockTokens;

    // global -> register staging: each operand's 256 rows x 128 bytes as 4 x 16 bytes
    // per thread, 8 threads per row.  Rows past the last query / last block are
    // clamped to it (their products are never stored) and feature offsets past the
    // end to the last step (the loads issued ahead of the last steps are never used).
    constexpr int TPR = TK / 8;          // threads per row
    constexpr int RPP = kThreads / TPR;  // rows per pass
    constexpr int LPO = TM / RPP;        // loads per operand per thread
    const int lr = t / TPR, lk = (t % TPR) * 8;
    const h16 *qa[LPO], *pb[LPO];
#pragma unroll
    for (int i = 0; i < LPO; i++) {
        qa[i] = Q + (int64_t)min(r0 + lr + RPP * i, n_q - 1) * K + lk;
        pb[i] = P + (int64_t)min(c0 + lr + RPP * i, nb_max - 1) * K + lk;
    }
    h16x8 ga[NS][LPO], gb[NS][LPO];
    auto gload = [&](int u, int k0) {
        k0 = min(k0, K - TK);
#pragma unroll
        for (int i = 0; i < LPO; i++)
            ga[u][i] = *(const h16x8 *)(qa[i] + k0);
#pragma unroll
        for (int i = 0; i < LPO; i++)
            gb[u][i] = *(const h16x8 *)(pb[i] + k0);
    };
    auto sstore = [&](int u, h16 *as, h16 *bs) {
#pragma unroll
        for (int i = 0; i < LPO; i++)
            *(h16x8 *)&as[(lr + RPP * i) * PITCH + lk] = ga[u][i];
#pragma unroll
        for (int i = 0; i < LPO; i++)
            *(h16x8 *)&bs[(lr + RPP * i) * PITCH + lk] = gb[u][i];
    };

    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; i++)
#pragma unroll
        for (int jj = 0; jj < FJ; jj++)
            acc[i][jj] = f32x4{0, 0, 0, 0};

    const int fr = lane & 15, fk = (lane >> 4) * 8;
    auto mma = [&](const h16 *as, const h16 *bs) {
#pragma unroll
        for (int kk = 0; kk < TK; kk += 32) {
            h16x8 b[FJ];
#pragma unroll
            for (int jj = 0; jj < FJ; jj++)
                b[jj] = *(const h16x8 *)&bs[(wn * WN + jj * 16 + fr) * PITCH + kk + fk];
#pragma unroll
            for (int i = 0; i < FI; i++) {
                const h16x8 a = *(const h16x8 *)&as[(wm * WM + i * 16 + fr) * PITCH + kk + fk];
#pragma unroll
                for (int jj = 0; jj < FJ; jj++)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[jj], acc[i][jj], 0, 0, 0);
            }
        }
    };

    // step s is read from buffer s % 2 and travels in register set s % NS.  K is a
    // multiple of NS * TK (host check), so the loop runs over whole groups of NS
    // steps (every register index a constant) with no branch around a load.
    const int nsteps = K / TK;
#pragma unroll
    for (int u = 0; u < NS; u++)
        gload(u, u * TK);
    sstore(0, As[0], Bs[0]);
    __syncthreads();
    gload(0, NS * TK);
    for (int s0 = 0; s0 < nsteps; s0 += NS) {
#pragma unroll
        for (int u = 0; u < NS; u++) {
            mma(As[u % 2], Bs[u % 2]);                          // step s0 + u
            sstore((u + 1) % NS, As[(u + 1) % 2], Bs[(u + 1) % 2]);  // step s0 + u + 1
            __syncthreads();
            gload((u + 1) % NS, (s0 + u + 1 + NS) * TK);        // step s0 + u + 1 + NS
        }
    }

    // D layout: lane holds column (lane & 15), rows 4*(lane >> 4) + e
#pragma unroll
    for (int i = 0; i < FI; i++) {
#pragma unroll
        for (int jj = 0; jj < FJ; jj++) {
            const int32_t c = c0 + wn * WN + jj * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int32_t r = r0 + wm * WM + i * 16 + 4 * (lane >> 4) + e;
                if (r < n_q && c < nb_max)
                    S[(int64_t)r * ld + c] = acc[i][jj][e];
            }
        }
    }
}

}  // namespace

hipError_t launch_score_prefill(const h16 *q, int32_t n_q, int32_t pos0, const h16 *pool,
                                int32_t row_elems, float *scores, int32_t ld, hipStream_t s,
                                KernelEvents ev)
{
    const int32_t nb_max = (pos0 + n_q) / kBlockTokens;
    if (nb_max <= 0)
        return hipSuccess;
    if (row_elems % (NS * TK))
        return hipErrorInvalidValue;
    const int32_t ncol = (nb_max + TN - 1) / TN, nrow = (n_q + TM - 1) / TM;
    // every XCD gets whole columns (all their row tiles); columns past ncol exit
    const int64_t wgs = (int64_t)((ncol + kXcds - 1) / kXcds) * kXcds * nrow;
    launch_ev(score_prefill_kernel, dim3((uint32_t)wgs), dim3(kThreads), 0, s, ev, q, n_q, pos0,
              pool, row_elems, scores, ld, ncol, nrow);
    return hipGetLastError();
}

}  // namespace qsa
