// Attention over the chosen cells only (Qiita part 10, "selected QSA K/V
// gather（COMMON-005）": top-k cells -> K/V rows -> ordinary attention over them),
// and the compact K/V gather itself.
//
// attn_kernel<G, D, DV>: one work group per (split, kv head g, query row).  A
// split walks `chunks` chunks of 64 cells with an online softmax (log2 domain):
//   * the cell -> token map of the chunk goes to LDS (compact rows, chosen
//     blocks + tail read straight from the caches, or an explicit list);
//   * QK: each wave takes 16 cells; the 4 lane groups of a wave split the head
//     dim in quarters, read 16-byte pieces of the K row, dot them against the G
//     query heads held in LDS, and reduce across the quarters;
//   * PV: each wave owns G/4 query heads; a lane owns DV/64 value dims and walks
//     the chunk's cells, reading each V row once per wave, coalesced.
// With several splits, each writes (m, l, o) partials; the last work group of a
// (row, g) to finish (an atomic ticket) merges them and resets the ticket.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <int N>
struct VecH;
template <>
struct VecH<1> {
    typedef h16 T;
};
template <>
struct VecH<2> {
    typedef h16x2 T;
};
template <>
struct VecH<4> {
    typedef h16x4 T;
};
template <>
struct VecH<8> {
    typedef h16x8 T;
};

__device__ __forceinline__ float h2f(h16 x) { return (float)x; }

template <int G, int D, int DV>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a)
{
    constexpr int HPW = G >= 4 ? G / 4 : 1;  // query heads per wave in PV
    constexpr int DPL = DV / kWave;          // value dims per lane
    constexpr int QV = D / 32;               // 16-byte K pieces per lane (a quarter row)
    static_assert(D % 32 == 0 && DV % kWave == 0, "shape");
    typedef typename VecH<DPL>::T vtype;

    __shared__ __attribute__((aligned(16))) h16 qs[G * D];
    __shared__ float ps[G][kAttnChunk];
    __shared__ int32_t toks[kAttnChunk];
    __shared__ uint32_t flag;

    const int split = blockIdx.x, g = blockIdx.y, row = blockIdx.z;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;

    int32_t count = 0, nsel = 0, nbr = 0;
    bool overflow = false;
    if (a.mode == kCellsCompact) {
        count = a.n_cells;
    } else if (a.mode == kCellsBlocks) {
        const int32_t N = a.pos0 + row + 1;
        nbr = N / kBlockTokens;
        nsel = min(a.topk, nbr);
        count = kBlockTokens * nsel + (N - kBlockTokens * nbr);
    } else {
        const int32_t nl = *a.n_list;
        overflow = nl > a.list_cap;
        count = overflow ? 0 : nl;
    }
    const int32_t *blkr = a.blk ? a.blk + (int64_t)row * a.ldb : nullptr;

    const h16 *qrow = a.q + ((int64_t)row * a.hq + (int64_t)g * G) * D;
    for (int i = t; i < G * D / 8; i += kThreads)
        ((h16x8 *)qs)[i] = ((const h16x8 *)qrow)[i];

    float m_run[HPW], l_run[HPW], o[HPW][DPL];
#pragma unroll
    for (int hh = 0; hh < HPW; hh++) {
        m_run[hh] = -INFINITY;
        l_run[hh] = 0.f;
#pragma unroll
        for (int j = 0; j < DPL; j++)
            o[hh][j] = 0.f;
    }
    const float sl2 = a.scale * kLog2e;
    const int64_t kg = (int64_t)g * D, vg = (int64_t)g * DV;

    for (int ch = 0; ch < a.chunks; ch++) {
        const int32_t c0 = (split * a.chunks + ch) * kAttnChunk;
        if (t < kAttnChunk) {
            const int32_t c = c0 + t;
            int32_t tok = -1;
            if (c < count) {
                if (a.mode == kCellsCompact) {
                    tok = c;
                } else if (a.mode == kCellsBlocks) {
                    if (c < kBlockTokens * nsel) {
                        const int32_t b = blkr ? blkr[c / kBlockTokens] : c / kBlockTokens;
                        // an id outside [0, nb) can only come from a broken selection:
                        // drop the cell rather than read outside the cache
                        tok = ((uint32_t)b < (uint32_t)nbr) ? kBlockTokens * b + (c & 3) : -1;
                    } else {
                        tok = kBlockTokens * nbr + (c - kBlockTokens * nsel);
                    }
                } else {
                    const int32_t j = a.list[c];
                    tok = ((uint32_t)j < (uint32_t)a.tok_bound) ? j : -1;
                }
            }
            toks[t] = tok;
        }
        __syncthreads();

        // ---- QK
        {
            const int cl = wave * 16 + (lane & 15);
            const int pt = lane >> 4;
            const int32_t tok = toks[cl];
            float acc[G];
#pragma unroll
            for (int h = 0; h < G; h++)
                acc[h] = 0.f;
            if (tok >= 0) {
                const h16 *kr = a.kbase + (int64_t)tok * a.k_tok + kg + pt * (D / 4);
#pragma unroll 2
                for (int v = 0; v < QV; v++) {
                    const h16x8 kv = *(const h16x8 *)(kr + 8 * v);
#pragma unroll
                    for (int h = 0; h < G; h++)
                        acc[h] = dot8(*(const h16x8 *)&qs[h * D + pt * (D / 4) + 8 * v], kv, acc[h]);
                }
            }
            float bias = 0.f;
            if (a.bias && tok >= 0)
                bias = h2f(a.bias[tok]) * kLog2e;
#pragma unroll
            for (int h = 0; h < G; h++) {
                acc[h] += __shfl_xor(acc[h], 16, kWave);
                acc[h] += __shfl_xor(acc[h], 32, kWave);
            }
            if (pt == 0) {
#pragma unroll
                for (int h = 0; h < G; h++)
                    ps[h][cl] = (tok >= 0) ? acc[h] * sl2 + bias : -INFINITY;
            }
        }
        __syncthreads();

        // ---- online softmax update for this wave's heads
#pragma unroll
        for (int hh = 0; hh < HPW; hh++) {
            const int h = wave * HPW + hh;
            if (h < G) {
                const float s = ps[h][lane];
                const float cmax = group_max<kWave>(s);
                const float mnew = fmaxf(m_run[hh], cmax);
                const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m_run[hh] - mnew);
                const float p = (s == -INFINITY) ? 0.f : exp2f(s - mnew);
                ps[h][lane] = p;
                l_run[hh] = l_run[hh] * alpha + group_sum<kWave>(p);
                m_run[hh] = mnew;
#pragma unroll
                for (int j = 0; j < DPL; j++)
                    o[hh][j] *= alpha;
            }
        }
        __syncthreads();

        // ---- PV
        if (wave * HPW < G) {
            const int nvalid = max(0, min(kAttnChunk, count - c0));
            for (int c = 0; c < nvalid; c++) {
                const int32_t tok = toks[c];
                if (tok < 0)
                    continue;
                const vtype vv = *(const vtype *)(a.vbase + (int64_t)tok * a.v_tok + vg +
                                                  lane * DPL);
#pragma unroll
                for (int hh = 0; hh < HPW; hh++) {
                    const int h = wave * HPW + hh;
                    if (h < G) {
                        const float p = ps[h][c];
                        if constexpr (DPL == 1) {
                            o[hh][0] += p * h2f(vv);
                        } else {
#pragma unroll
                            for (int j = 0; j < DPL; j++)
                                o[hh][j] += p * h2f(vv[j]);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    const int64_t hq0 = (int64_t)row * a.hq + (int64_t)g * G;
    if (a.splits == 1) {
#pragma unroll
        for (int hh = 0; hh < HPW; hh++) {
            const int h = wave * HPW + hh;
            if (h < G) {
                const float inv = 1.f / l_run[hh];
#pragma unroll
                for (int j = 0; j < DPL; j++)
                    a.out[(hq0 + h) * DV + lane * DPL + j] = overflow ? NAN : o[hh][j] * inv;
            }
        }
        return;
    }

    const int S = a.splits;
#pragma unroll
    for (int hh = 0; hh < HPW; hh++) {
        const int h = wave * HPW + hh;
        if (h < G) {
            float *pb = a.part + ((hq0 + h) * S + split) * (DV + 2);
            if (lane == 0) {
                pb[0] = m_run[hh];
                pb[1] = l_run[hh];
            }
#pragma unroll
            for (int j = 0; j < DPL; j++)
                pb[2 + lane * DPL + j] = o[hh][j];
        }
    }
    __threadfence();
    __syncthreads();
    if (t == 0)
        flag = (atomicAdd(&a.tickets[(int64_t)row * a.hkv + g], 1u) == (uint32_t)(S - 1)) ? 1u : 0u;
    __syncthreads();
    if (!flag)
        return;
    __threadfence();
    for (int e = t; e < G * DV; e += kThreads) {
        const int h = e / DV, j = e - h * DV;
        const float *pb = a.part + (hq0 + h) * S * (DV + 2);
        float M = -INFINITY;
        for (int s = 0; s < S; s++)
            M = fmaxf(M, __builtin_nontemporal_load(&pb[s * (DV + 2)]));
        float L = 0.f, O = 0.f;
        for (int s = 0; s < S; s++) {
            const float ms = __builtin_nontemporal_load(&pb[s * (DV + 2)]);
            const float w = exp2f(ms - M);
            L += w * __builtin_nontemporal_load(&pb[s * (DV + 2) + 1]);
            O += w * __builtin_nontemporal_load(&pb[s * (DV + 2) + 2 + j]);
        }
        a.out[(hq0 + h) * DV + j] = overflow ? NAN : O / L;
    }
    if (t == 0)
        a.tickets[(int64_t)row * a.hkv + g] = 0;
}

__global__ __launch_bounds__(kThreads) void gather_kernel(const int32_t *__restrict__ blk,
                                                          int32_t n_blk, int32_t n_tokens,
                                                          const uint4 *__restrict__ kc,
                                                          const uint4 *__restrict__ vc,
                                                          int32_t krow16, int32_t vrow16,
                                                          uint4 *__restrict__ ks,
                                                          uint4 *__restrict__ vs)
{
    const int32_t j = blockIdx.x;
    int64_t tok0, dst0;
    int32_t nrows;
    if (j < n_blk) {
        const int32_t b = blk[j];
        if ((uint32_t)b >= (uint32_t)(n_tokens / kBlockTokens))
            return;  // not a complete block: leave the destination rows untouched
        tok0 = (int64_t)kBlockTokens * b;
        dst0 = (int64_t)kBlockTokens * j;
        nrows = kBlockTokens;
    } else {
        tok0 = (int64_t)kBlockTokens * (n_tokens / kBlockTokens);
        dst0 = (int64_t)kBlockTokens * n_blk;
        nrows = n_tokens % kBlockTokens;
    }
    for (int32_t i = threadIdx.x; i < nrows * krow16; i += kThreads)
        ks[dst0 * krow16 + i] = kc[tok0 * krow16 + i];
    for (int32_t i = threadIdx.x; i < nrows * vrow16; i += kThreads)
        vs[dst0 * vrow16 + i] = vc[tok0 * vrow16 + i];
}

template <int D, int DV>
hipError_t launch_g(const AttnArgs &a, int G, hipStream_t s)
{
    const dim3 grid((uint32_t)a.splits, (uint32_t)a.hkv, (uint32_t)a.rows);
    switch (G) {
    case 1: hipLaunchKernelGGL((attn_kernel<1, D, DV>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<2, D, DV>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_kernel<4, D, DV>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_kernel<8, D, DV>), grid, dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((attn_kernel<16, D, DV>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs &a, int32_t D, int32_t DV, hipStream_t s)
{
    const int G = a.hq / a.hkv;
    if (D == 128 && DV == 128)
        return launch_g<128, 128>(a, G, s);
    if (D == 64 && DV == 64)
        return launch_g<64, 64>(a, G, s);
    if (D == 576 && DV == 512)
        return launch_g<576, 512>(a, G, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gather(const int32_t *blk, int32_t n_blk, int32_t n_tokens, const h16 *k_cache,
                         const h16 *v_cache, int32_t k_row16, int32_t v_row16, h16 *k_sel,
                         h16 *v_sel, hipStream_t s)
{
    hipLaunchKernelGGL(gather_kernel, dim3((uint32_t)n_blk + 1), dim3(kThreads), 0, s, blk, n_blk,
                       n_tokens, (const uint4 *)k_cache, (const uint4 *)v_cache, k_row16, v_row16,
                       (uint4 *)k_sel, (uint4 *)v_sel);
    return hipGetLastError();
}

}  // namespace qsa
