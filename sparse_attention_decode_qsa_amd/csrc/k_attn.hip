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
// Every K piece of a chunk is loaded before its QK (one memory round trip, the
// next chunk's loads in flight during this chunk's softmax and PV).  With VK (V
// rows are the first DV elements of the K rows, as in the MLA latent view) the V
// rows go to LDS from those K registers, so V is not loaded at all; otherwise up
// to 4 V pieces per thread ride along with the K loads and the rest follow.
// With several splits, each writes (m, l, o) partials and attn_combine_kernel (a
// second launch; the kernel boundary makes the partials visible) merges them.
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

// Cell c of row `row` -> token, or -1 (past the row's cells, or a dropped id).
struct CellMap {
    int32_t mode, count, nsel, nbr, tok_bound, cap;
    const int32_t *blkr;
    const int32_t *list;

    __device__ __forceinline__ int32_t operator()(int32_t c) const
    {
        if (mode == kCellsList) {
            // the entry is read whether or not c is below the device count (c < cap
            // keeps the read inside the list), so its load overlaps the count's
            const int32_t j = c < cap ? list[c] : -1;
            return (c < count && (uint32_t)j < (uint32_t)tok_bound) ? j : -1;
        }
        if (c >= count)
            return -1;
        if (mode == kCellsCompact)
            return c;
        if (mode == kCellsBlocks) {
            if (c < kBlockTokens * nsel) {
                const int32_t b = blkr ? blkr[c / kBlockTokens] : c / kBlockTokens;
                // an id outside [0, nb) can only come from a broken selection: drop
                // the cell rather than read outside the cache
                return ((uint32_t)b < (uint32_t)nbr) ? kBlockTokens * b + (c & 3) : -1;
            }
            return kBlockTokens * nbr + (c - kBlockTokens * nsel);
        }
        return -1;
    }
};

template <int G, int D, int DV, bool VK>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a)
{
    constexpr int HPW = G >= 4 ? G / 4 : 1;          // query heads per wave (softmax, PV)
    // with fewer than 4 heads, WPH waves share a head in PV, each on DV / WPH of
    // its value dims (at least 64), so that no wave idles; the head's first wave
    // runs its softmax and passes the rescale and the final sum through LDS
    constexpr int WPH0 = G >= 4 ? 1 : 4 / G;
    constexpr int WPH = WPH0 < DV / kWave ? WPH0 : DV / kWave;
    constexpr int DPL = DV / WPH / kWave;            // value dims per lane in PV
    constexpr int QV = D / 32;                       // 16-byte K pieces per lane (a quarter row)
    constexpr int VPR = DV / 8;                      // 16-byte pieces per V row
    constexpr int VV = kAttnChunk * VPR / kThreads;  // V pieces per thread per chunk
    constexpr int KP = QV;                           // K pieces loaded a chunk ahead (all)
    constexpr int VP = VK ? 0 : (VV < 4 ? VV : 4);   // V pieces loaded a chunk ahead
    // LDS row pitch of V: padded when the rows are written from K registers
    // (16 cells of a wave write the same column; a 1 KB pitch would put them all
    // in one bank group)
    constexpr int VPITCH = VK ? DV + 8 : DV;
    static_assert(D % 32 == 0 && DV % kWave == 0 && VV >= 1, "shape");
    static_assert(!VK || DV <= D, "V is a prefix of the K row");
    typedef typename VecH<DPL>::T vtype;

    __shared__ __attribute__((aligned(16))) h16 qs[G * D];
    __shared__ __attribute__((aligned(16))) h16 vs[kAttnChunk * VPITCH];
    __shared__ __attribute__((aligned(16))) float ps[G][kAttnChunk];
    __shared__ int32_t toks[2][kAttnChunk];
    __shared__ float alpha_sh[G], lsum_sh[G];  // WPH > 1: the head's rescale, final sum

    const int split = blockIdx.x, g = blockIdx.y, row = blockIdx.z;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    // head hh of this wave, the first value dim of its PV slice, and whether it
    // runs the head's softmax
    auto head = [&](int hh) { return WPH > 1 ? wave / WPH : wave * HPW + hh; };
    const int d0 = (wave % WPH) * (DV / WPH);
    const bool lead = wave % WPH == 0;

    CellMap cm;
    cm.mode = a.mode;
    cm.nsel = 0;
    cm.nbr = 0;
    cm.tok_bound = a.tok_bound;
    cm.cap = a.list_cap;
    cm.list = a.list;
    cm.blkr = a.blk ? a.blk + (int64_t)row * a.ldb : nullptr;
    bool overflow = false;
    if (a.mode == kCellsCompact) {
        cm.count = a.n_cells;
    } else if (a.mode == kCellsBlocks) {
        const int32_t N = a.pos0 + row + 1;
        cm.nbr = N / kBlockTokens;
        cm.nsel = min(a.topk, cm.nbr);
        cm.count = kBlockTokens * cm.nsel + (N - kBlockTokens * cm.nbr);
    } else {
        const int32_t nl = *a.n_list;
        overflow = nl > a.list_cap;
        cm.count = overflow ? 0 : nl;
    }

    // the query rows of this head group: all loads issued at once (indexes clamped;
    // a loop of load-then-store would wait for each), stored to LDS with the cell map
    constexpr int QN = G * D / 8, QPT = (QN + kThreads - 1) / kThreads;
    const h16x8 *qrow8 = (const h16x8 *)(a.q + ((int64_t)row * a.hq + (int64_t)g * G) * D);
    h16x8 qv[QPT];
#pragma unroll
    for (int i = 0; i < QPT; i++)
        qv[i] = qrow8[min(t + i * kThreads, QN - 1)];
    auto store_q = [&]() {
#pragma unroll
        for (int i = 0; i < QPT; i++)
            if (t + i * kThreads < QN)
                ((h16x8 *)qs)[t + i * kThreads] = qv[i];
    };

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
    const int64_t kg = a.kv_shared ? 0 : (int64_t)g * D, vg = a.kv_shared ? 0 : (int64_t)g * DV;
    // QK: wave w takes cells 16w .. 16w+15 of the chunk; the 4 lanes of a quad
    // split one cell's head dim in quarters, so their partial dots meet in-quad
    const int cl = wave * 16 + (lane >> 2);
    const int pt = lane & 3;
    const int32_t cbase = split * a.chunks * kAttnChunk;

    h16x8 kreg[KP], vreg[VP > 0 ? VP : 1];
    auto kaddr = [&](int32_t tok) {
        return a.kbase + (int64_t)max(tok, 0) * a.k_tok + kg + pt * (D / 4);
    };
    auto vload = [&](const int32_t *tk, int i) {
        const int p = t + kThreads * i, c = p / VPR, pc = p - c * VPR;
        const int32_t tv = tk[c];
        return (tv >= 0) ? *(const h16x8 *)(a.vbase + (int64_t)tv * a.v_tok + vg + pc * 8)
                         : h16x8{0, 0, 0, 0, 0, 0, 0, 0};
    };
    auto issue_loads = [&](const int32_t *tk) {
        const int32_t tok = tk[cl];
        const h16 *kr = kaddr(tok);
#pragma unroll
        for (int v = 0; v < KP; v++)
            kreg[v] = (tok >= 0) ? *(const h16x8 *)(kr + 8 * v) : h16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < VP; i++)
            vreg[i] = vload(tk, i);
    };

    if (t < kAttnChunk)
        toks[0][t] = cm(cbase + t);
    store_q();
    __syncthreads();
    issue_loads(toks[0]);

    for (int ch = 0; ch < a.chunks; ch++) {
        const int cur = ch & 1;
        const int32_t c0 = cbase + ch * kAttnChunk;
        // ids of the next chunk: the load is issued now, the LDS store after QK
        int32_t next_tok = -1;
        const bool has_next = ch + 1 < a.chunks;
        if (has_next && t < kAttnChunk)
            next_tok = cm(c0 + kAttnChunk + t);

        // ---- QK
        {
            const int32_t tok = toks[cur][cl];
            float acc[G];
#pragma unroll
            for (int h = 0; h < G; h++)
                acc[h] = 0.f;
            // fully unrolled, so that kreg stays in registers; with long rows the
            // scheduler is kept from hoisting every piece's query reads at once
#pragma unroll
            for (int v = 0; v < QV; v++) {
#pragma unroll
                for (int h = 0; h < G; h++)
                    acc[h] = dot8(*(const h16x8 *)&qs[h * D + pt * (D / 4) + 8 * v], kreg[v], acc[h]);
                if constexpr (QV > 4)
                    __builtin_amdgcn_sched_barrier(0);
            }
            float bias = 0.f;
            if (a.bias && tok >= 0)
                bias = h2f(a.bias[tok]) * kLog2e;
#pragma unroll
            for (int h = 0; h < G; h++)
                acc[h] = quad_sum(acc[h]);
            if (pt == 0) {
#pragma unroll
                for (int h = 0; h < G; h++)
                    ps[h][cl] = (tok >= 0) ? acc[h] * sl2 + bias : -INFINITY;
            }
        }
        if constexpr (VK) {
            // the cell's V row = the first DV elements of the K row this lane holds a
            // quarter of (zeros for a dropped cell)
#pragma unroll
            for (int v = 0; v < QV; v++) {
                const int d0 = pt * (D / 4) + 8 * v;
                if (d0 < DV)
                    *(h16x8 *)&vs[cl * VPITCH + d0] = kreg[v];
            }
        } else {
#pragma unroll
            for (int i = 0; i < VP; i++)
                *(h16x8 *)&vs[(t + kThreads * i) * 8] = vreg[i];
            for (int i0 = VP; i0 < VV; i0 += 4) {  // large value dims: the rest, 4 at a time
                h16x8 tmp[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (i0 + i < VV)
                        tmp[i] = vload(toks[cur], i0 + i);
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (i0 + i < VV)
                        *(h16x8 *)&vs[(t + kThreads * (i0 + i)) * 8] = tmp[i];
            }
        }
        if (has_next && t < kAttnChunk)
            toks[cur ^ 1][t] = next_tok;
        __syncthreads();
        if (has_next)
            issue_loads(toks[cur ^ 1]);

        // ---- online softmax update for this wave's heads (lane = cell)
#pragma unroll
        for (int hh = 0; hh < HPW; hh++) {
            const int h = head(hh);
            if (h < G && lead) {
                const float s = ps[h][lane];
                const float mnew = fmaxf(m_run[hh], wave_max(s));
                const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m_run[hh] - mnew);
                const float p = (s == -INFINITY) ? 0.f : exp2f(s - mnew);
                ps[h][lane] = p;
                l_run[hh] = l_run[hh] * alpha + wave_sum(p);
                m_run[hh] = mnew;
                if constexpr (WPH > 1) {
                    if (lane == 0)
                        alpha_sh[h] = alpha;
                } else {
#pragma unroll
                    for (int j = 0; j < DPL; j++)
                        o[hh][j] *= alpha;
                }
            }
        }
        __syncthreads();
        if constexpr (WPH > 1) {
            if (head(0) < G) {
                const float alpha = alpha_sh[head(0)];
#pragma unroll
                for (int j = 0; j < DPL; j++)
                    o[0][j] *= alpha;
            }
        }

        // ---- PV from the LDS copy of the chunk's V rows.  Cells past the end or
        // dropped have p = 0 and zeroed V rows, so all 64 are walked unguarded.
        if (head(0) < G) {
#pragma unroll 4
            for (int c4 = 0; c4 < kAttnChunk; c4 += 4) {
                f32x4 p4[HPW];
#pragma unroll
                for (int hh = 0; hh < HPW; hh++)
                    p4[hh] = *(const f32x4 *)&ps[min(head(hh), G - 1)][c4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const vtype vv = *(const vtype *)&vs[(c4 + u) * VPITCH + d0 + lane * DPL];
#pragma unroll
                    for (int hh = 0; hh < HPW; hh++) {
                        const float p = p4[hh][u];
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
    if constexpr (WPH > 1) {
        if (lead && lane == 0 && head(0) < G)
            lsum_sh[head(0)] = l_run[0];
        __syncthreads();
    }
#pragma unroll
    for (int hh = 0; hh < HPW; hh++) {
        const int h = head(hh);
        if (h < G) {
            if (a.splits == 1) {
                const float inv = 1.f / (WPH > 1 ? lsum_sh[h] : l_run[hh]);
#pragma unroll
                for (int j = 0; j < DPL; j++)
                    a.out[(hq0 + h) * DV + d0 + lane * DPL + j] = overflow ? NAN : o[hh][j] * inv;
            } else {
                // split-K partial (m, l, o); attn_combine_kernel merges them
                float *pb = a.part + ((hq0 + h) * a.splits + split) * (DV + 2);
                if (lead && lane == 0) {
                    pb[0] = m_run[hh];
                    pb[1] = l_run[hh];
                }
#pragma unroll
                for (int j = 0; j < DPL; j++)
                    pb[2 + d0 + lane * DPL + j] = o[hh][j];
            }
        }
    }
}

// Merge of split-K partials: one work group per (query head, row).  Wave 0
// turns the S (m, l) pairs into weights w_s = exp2(m_s - M) and
// L = sum_s w_s l_s (one split per lane) while every thread already loads its
// share of the o_s rows: output dim j, splits s = grp, grp + G, ... (G groups of
// DV threads when DV < 256).  out_j = sum_s w_s o_sj / L, the group sums added
// in group order.
constexpr int kCombThreads = 256;
static_assert(kAttnMaxSplits <= kWave, "one split per lane of wave 0");

template <int DV>
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(const float *__restrict__ part,
                                                                   int32_t hq, int32_t S,
                                                                   const int32_t *n_list,
                                                                   int32_t list_cap,
                                                                   float *__restrict__ out)
{
    constexpr int DPT = DV > kCombThreads ? DV / kCombThreads : 1;  // dims per thread
    constexpr int G = DV < kCombThreads ? kCombThreads / DV : 1;    // split groups
    // splits per thread per round: G * 32 splits (32 at 512 value dims, 64 at 128)
    // are merged in one round, i.e. one memory round trip
    constexpr int CH = 32;
    static_assert(DPT * CH <= 64, "partials held per thread");
    __shared__ float w_sh[kAttnMaxSplits];
    __shared__ float l_sh;
    __shared__ float red[G][DV];

    const int h = blockIdx.x, row = blockIdx.y, t = threadIdx.x;
    const int grp = t / (DV / DPT), jt = t % (DV / DPT);
    const int64_t stride = DV + 2;
    const float *pb = part + ((int64_t)row * hq + h) * S * stride;

    float m = -INFINITY, l = 0.f;
    if (t < kWave && t < S) {
        m = pb[t * stride];
        l = pb[t * stride + 1];
    }
    float acc[DPT];
#pragma unroll
    for (int p = 0; p < DPT; p++)
        acc[p] = 0.f;
    int32_t nl = 0;
    for (int s0 = 0; s0 < S; s0 += G * CH) {
        float o[CH][DPT];
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int sl = s0 + grp + G * i;
            const int sc = sl < S ? sl : S - 1;
#pragma unroll
            for (int p = 0; p < DPT; p++)
                o[i][p] = pb[sc * stride + 2 + jt + p * (DV / DPT)];
        }
        if (s0 == 0) {
            // the list count (a scalar load) goes out with this round's partials
            nl = n_list ? *n_list : 0;
            if (t < kWave) {
                const float M = wave_max(m);
                const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
                const float L = wave_sum(w * l);
                w_sh[t] = w;
                if (t == 0)
                    l_sh = L;
            }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int sl = s0 + grp + G * i;
            const float w = sl < S ? w_sh[sl < kAttnMaxSplits ? sl : 0] : 0.f;
#pragma unroll
            for (int p = 0; p < DPT; p++)
                acc[p] = sl < S ? fmaf(w, o[i][p], acc[p]) : acc[p];
        }
    }
    const bool overflow = n_list && nl > list_cap;
    if (G > 1) {
        red[grp][jt] = acc[0];
        __syncthreads();
        if (grp == 0) {
            float O = red[0][jt];
#pragma unroll
            for (int g = 1; g < G; g++)
                O += red[g][jt];
            out[((int64_t)row * hq + h) * DV + jt] = overflow ? NAN : O / l_sh;
        }
    } else {
#pragma unroll
        for (int p = 0; p < DPT; p++)
            out[((int64_t)row * hq + h) * DV + jt + p * (DV / DPT)] =
                overflow ? NAN : acc[p] / l_sh;
    }
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

template <int D, int DV, bool VK>
hipError_t launch_g(const AttnArgs &a, int G, hipStream_t s)
{
    const dim3 grid((uint32_t)a.splits, (uint32_t)a.hkv, (uint32_t)a.rows);
    // the 576-wide latent rows are attended in head groups of at most 2
    constexpr int kMaxG = D > 128 ? 2 : 16;
    if (G > kMaxG)
        return hipErrorInvalidValue;
    switch (G) {
    case 1: hipLaunchKernelGGL((attn_kernel<1, D, DV, VK>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<2, D, DV, VK>), grid, dim3(kThreads), 0, s, a); break;
    case 4:
        if constexpr (kMaxG >= 4)
            hipLaunchKernelGGL((attn_kernel<4, D, DV, VK>), grid, dim3(kThreads), 0, s, a);
        break;
    case 8:
        if constexpr (kMaxG >= 8)
            hipLaunchKernelGGL((attn_kernel<8, D, DV, VK>), grid, dim3(kThreads), 0, s, a);
        break;
    case 16:
        if constexpr (kMaxG >= 16)
            hipLaunchKernelGGL((attn_kernel<16, D, DV, VK>), grid, dim3(kThreads), 0, s, a);
        break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1)
        return e;
    hipLaunchKernelGGL((attn_combine_kernel<DV>), dim3((uint32_t)a.hq, (uint32_t)a.rows),
                       dim3(kCombThreads), 0, s, a.part, a.hq, a.splits,
                       a.mode == kCellsList ? a.n_list : nullptr, a.list_cap, a.out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs &a, int32_t D, int32_t DV, hipStream_t s)
{
    const int G = a.hq / a.hkv;
    if (a.splits > kAttnMaxSplits)
        return hipErrorInvalidValue;
    if (a.v_in_k && (a.vbase != a.kbase || a.v_tok != a.k_tok))
        return hipErrorInvalidValue;
    if (D == 128 && DV == 128 && !a.v_in_k)
        return launch_g<128, 128, false>(a, G, s);
    if (D == 64 && DV == 64 && !a.v_in_k)
        return launch_g<64, 64, false>(a, G, s);
    if (D == 576 && DV == 512)
        return a.v_in_k ? launch_g<576, 512, true>(a, G, s) : launch_g<576, 512, false>(a, G, s);
    return hipErrorInvalidValue;
}

hipError_t launch_combine(const float *part, int32_t hq, int32_t splits, int32_t dv, int32_t rows,
                          float *out, hipStream_t s)
{
    if (splits < 1 || splits > kAttnMaxSplits || rows < 1)
        return hipErrorInvalidValue;
    const dim3 grid((uint32_t)hq, (uint32_t)rows);
    switch (dv) {
    case 64:
        hipLaunchKernelGGL((attn_combine_kernel<64>), grid, dim3(kCombThreads), 0, s, part, hq,
                           splits, nullptr, 0, out);
        break;
    case 128:
        hipLaunchKernelGGL((attn_combine_kernel<128>), grid, dim3(kCombThreads), 0, s, part, hq,
                           splits, nullptr, 0, out);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
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
