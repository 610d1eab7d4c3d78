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
// Every 32-feature step stages A (16 KiB) and B (16 KiB) in LDS with rows padded
// to 80 bytes (conflict-free 16-byte fragment reads).  Two LDS buffers and two
// register sets: while step s is multiplied, step s + 1 waits in registers to be
// stored into the other buffer and step s + 2's global loads are in flight, so a
// load has two steps of MFMA work to arrive, and a step needs one barrier.
// Blocks at or past the last row's causal bound are neither read nor written.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 512;
constexpr int TM = 256, TN = 256, TK = 32;
constexpr int PITCH = TK + 8;  // halfs per LDS row (80 bytes)
constexpr int WM = 128, WN = 64;
constexpr int FI = WM / 16, FJ = WN / 16;

__global__ __launch_bounds__(kThreads, 1) void score_prefill_kernel(const h16 *__restrict__ Q,
                                                                 int32_t n_q, int32_t pos0,
                                                                 const h16 *__restrict__ P,
                                                                 int32_t K, float *__restrict__ S,
                                                                 int32_t ld)
{
    __shared__ __attribute__((aligned(16))) h16 As[2][TM * PITCH];
    __shared__ __attribute__((aligned(16))) h16 Bs[2][TN * PITCH];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int32_t r0 = blockIdx.y * TM;
    const int32_t c0 = blockIdx.x * TN;
    const int32_t nb_max = (pos0 + n_q) / kBlockTokens;

    // global -> register staging: A: 2 x 16B per thread, B: 2 x 16B per thread
    const int lr = t >> 2, lk = (t & 3) * 8;
    h16x8 ga0[2], gb0[2], ga1[2], gb1[2];
    auto gload = [&](h16x8 (&ga)[2], h16x8 (&gb)[2], int k0) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int32_t r = r0 + lr + 128 * j;
            ga[j] = (r < n_q) ? *(const h16x8 *)(Q + (int64_t)r * K + k0 + lk)
                              : h16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int32_t c = c0 + lr + 128 * j;
            gb[j] = (c < nb_max) ? *(const h16x8 *)(P + (int64_t)c * K + k0 + lk)
                                 : h16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    };
    auto sstore = [&](const h16x8 (&ga)[2], const h16x8 (&gb)[2], h16 *as, h16 *bs) {
#pragma unroll
        for (int j = 0; j < 2; j++)
            *(h16x8 *)&as[(lr + 128 * j) * PITCH + lk] = ga[j];
#pragma unroll
        for (int j = 0; j < 2; j++)
            *(h16x8 *)&bs[(lr + 128 * j) * PITCH + lk] = gb[j];
    };

    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; i++)
#pragma unroll
        for (int j = 0; j < FJ; j++)
            acc[i][j] = f32x4{0, 0, 0, 0};

    const int fr = lane & 15, fk = (lane >> 4) * 8;
    auto mma = [&](const h16 *as, const h16 *bs) {
        h16x8 b[FJ];
#pragma unroll
        for (int j = 0; j < FJ; j++)
            b[j] = *(const h16x8 *)&bs[(wn * WN + j * 16 + fr) * PITCH + fk];
#pragma unroll
        for (int i = 0; i < FI; i++) {
            const h16x8 a = *(const h16x8 *)&as[(wm * WM + i * 16 + fr) * PITCH + fk];
#pragma unroll
            for (int j = 0; j < FJ; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], acc[i][j], 0, 0, 0);
        }
    };

    // step s is read from buffer s % 2; register set s % 2 carries step s (and
    // later s + 2) from global memory to its buffer.  The loop runs over pairs of
    // steps so that each register set has a fixed name.
    const int nsteps = K / TK;
    gload(ga0, gb0, 0);
    if (nsteps > 1)
        gload(ga1, gb1, TK);
    sstore(ga0, gb0, As[0], Bs[0]);
    __syncthreads();
    if (nsteps > 2)
        gload(ga0, gb0, 2 * TK);
    int s0 = 0;
    for (; s0 + 1 < nsteps; s0 += 2) {
        mma(As[0], Bs[0]);
        sstore(ga1, gb1, As[1], Bs[1]);
        __syncthreads();
        if (s0 + 3 < nsteps)
            gload(ga1, gb1, (s0 + 3) * TK);
        mma(As[1], Bs[1]);
        if (s0 + 2 < nsteps)
            sstore(ga0, gb0, As[0], Bs[0]);
        __syncthreads();
        if (s0 + 4 < nsteps)
            gload(ga0, gb0, (s0 + 4) * TK);
    }
    if (s0 < nsteps)  // an odd last step, already in buffer 0
        mma(As[0], Bs[0]);

    // D layout: lane holds column (lane & 15), rows 4*(lane >> 4) + e
#pragma unroll
    for (int i = 0; i < FI; i++) {
#pragma unroll
        for (int j = 0; j < FJ; j++) {
            const int32_t c = c0 + wn * WN + j * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int32_t r = r0 + wm * WM + i * 16 + 4 * (lane >> 4) + e;
                if (r < n_q && c < nb_max)
                    S[(int64_t)r * ld + c] = acc[i][j][e];
            }
        }
    }
}

}  // namespace

hipError_t launch_score_prefill(const h16 *q, int32_t n_q, int32_t pos0, const h16 *pool,
                                int32_t row_elems, float *scores, int32_t ld, hipStream_t s)
{
    const int32_t nb_max = (pos0 + n_q) / kBlockTokens;
    if (nb_max <= 0)
        return hipSuccess;
    if (row_elems % TK)
        return hipErrorInvalidValue;
    const dim3 grid((uint32_t)((nb_max + TN - 1) / TN), (uint32_t)((n_q + TM - 1) / TM));
    hipLaunchKernelGGL(score_prefill_kernel, grid, dim3(kThreads), 0, s, q, n_q, pos0, pool,
                       row_elems, scores, ld);
    return hipGetLastError();
}

}  // namespace qsa
