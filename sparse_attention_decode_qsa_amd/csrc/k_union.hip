// Grouped-union attention for a prefill chunk.
//
// The pages report that their "QSA grouped-union" switch speeds up prompt
// processing and leaves token generation unchanged (Qiita part 10: the opening
// paragraphs, the union ON/OFF table of 「Vulkan版のプロファイリングでTGが遅くなった
// 原因を調べる」 and the r2-versus-r3 table of 「COMMON-004実装結果」).  They do not
// spell out its steps.  The reading taken here keeps the method's result:
// consecutive query rows form groups; a group streams the union of its rows'
// chosen blocks (and the span of its rows' tails) once, and a per-row mask keeps
// every row on exactly its own cells: its chosen blocks plus its tail
// [4 * floor(N_r / 4), N_r).  The output therefore equals the per-row prefill
// attention up to fp32 summation order; what changes is that K/V rows shared by
// several rows of a group are read once, and that QK^T and PV become dense
// contractions over 128 queries (group rows x query heads of one KV head) that
// run on the matrix cores.
//
// union_build_kernel: one work group per group.  The chosen ids of the group's
// rows set bits of an LDS bitmap (windows of 2^18 blocks); a scan of the word
// popcounts turns the bitmap into the ascending union list, and a second pass
// ORs each row's bit into the mask of its blocks' union slots.
//
// union_attn_kernel: grid (groups, KV heads, splits), 4 waves, 32 queries per
// wave.  Per tile of 16 blocks (64 cells): K is staged in LDS row-major and V
// transposed (dv-major), the next tile's loads are in flight during the current
// tile's math.  S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_f16, so a
// lane's scores, softmax state and outputs all belong to its own two queries;
// the k slots of the PV product are the score lanes' cells in the order the
// score product leaves them (each lane holds whole 4-cell blocks).  Online
// softmax in the log2 domain; P is rounded to binary16 for the PV product.
#include "qsa_internal.h"
#include "qsa_select.h"

namespace qsa {
namespace {

constexpr int kUBThreads = 1024;
constexpr int kWinBlocks = 1 << 18;  // bitmap window of the union build
constexpr int kWinWords = kWinBlocks / 32;

constexpr int kUAThreads = 256;   // 4 waves
constexpr int kTB = 16;           // blocks per tile
constexpr int kTC = kTB * kBlockTokens;  // cells per tile
constexpr int kDim = 128;         // D = DV
constexpr int KP = kDim + 8;      // K tile pitch (halfs)
constexpr int VP = kTC + 4;       // V^T tile pitch (halfs)
constexpr float kLog2e = 1.4426950408889634f;

struct UnionBuildLds {
    uint32_t bits[kWinWords];
    uint32_t pre[kWinWords];
    uint32_t msk[kUnionCap];
    Scratch<kUBThreads> S;
    uint32_t total;
};

__global__ __launch_bounds__(kUBThreads) void union_build_kernel(
    const int32_t *__restrict__ blk, int32_t ldb, int32_t pos0, int32_t n_q, int32_t k, int32_t G,
    int32_t cap_u, int32_t *__restrict__ uid, uint32_t *__restrict__ umask,
    int32_t *__restrict__ n_u)
{
    __shared__ UnionBuildLds sm;
    const int t = threadIdx.x;
    const int32_t g = blockIdx.x, r0 = g * G;
    const int32_t nr = min(G, n_q - r0);
    const int32_t nb_hi = (pos0 + r0 + nr) / kBlockTokens;  // blocks the last row sees
    const int32_t n_ent = nr * k;
    int32_t *ug = uid + (int64_t)g * cap_u;

    for (int32_t i = t; i < n_ent; i += kUBThreads)
        sm.msk[i] = 0u;
    uint32_t base = 0;
    for (int32_t w0 = 0; w0 < nb_hi; w0 += kWinBlocks) {
        const int32_t nwb = min(kWinBlocks, nb_hi - w0);
        const int32_t nw = (nwb + 31) / 32;
        for (int32_t i = t; i < nw; i += kUBThreads)
            sm.bits[i] = 0u;
        __syncthreads();
        for (int32_t e = t; e < n_ent; e += kUBThreads) {
            const int32_t i = e / k, j = e - i * k;
            const int32_t ns = min(k, (pos0 + r0 + i + 1) / kBlockTokens);
            if (j < ns) {
                const uint32_t id = (uint32_t)(blk[(int64_t)(r0 + i) * ldb + j] - w0);
                if (id < (uint32_t)nwb)
                    atomicOr(&sm.bits[id >> 5], 1u << (id & 31));
            }
        }
        __syncthreads();
        const int32_t per = (nw + kUBThreads - 1) / kUBThreads;
        const int32_t wa = t * per, wb = min(nw, wa + per);
        uint32_t c = 0;
        for (int32_t w = wa; w < wb; w++)
            c += __popc(sm.bits[w]);
        uint32_t pos = base + wg_exclusive_scan<kUBThreads>(c, sm.S);
        for (int32_t w = wa; w < wb; w++) {
            sm.pre[w] = pos;
            uint32_t m = sm.bits[w];
            while (m) {
                const uint32_t b = (uint32_t)__ffs((int)m) - 1u;
                ug[pos++] = w0 + w * 32 + (int32_t)b;
                m &= m - 1u;
            }
        }
        if (t == kUBThreads - 1)
            sm.total = pos;
        __syncthreads();
        for (int32_t e = t; e < n_ent; e += kUBThreads) {
            const int32_t i = e / k, j = e - i * k;
            const int32_t ns = min(k, (pos0 + r0 + i + 1) / kBlockTokens);
            if (j < ns) {
                const uint32_t id = (uint32_t)(blk[(int64_t)(r0 + i) * ldb + j] - w0);
                if (id < (uint32_t)nwb) {
                    const uint32_t w = id >> 5;
                    const uint32_t p = sm.pre[w] + __popc(sm.bits[w] & ((1u << (id & 31)) - 1u));
                    atomicOr(&sm.msk[p], 1u << i);
                }
            }
        }
        base = sm.total;
        __syncthreads();
    }
    for (uint32_t i = t; i < base; i += kUBThreads)
        umask[(int64_t)g * cap_u + i] = sm.msk[i];
    if (t == 0)
        n_u[g] = (int32_t)base;
}

struct alignas(16) UnionAttnLds {
    alignas(16) h16 ks[kTC * KP];    // K tile, [cell][d]
    alignas(16) h16 vt[kDim * VP];   // V tile transposed, [dv][cell]
    int32_t bid[kTB];                // block id of each tile block, -1 past the end
    uint32_t bmask[kTB];             // union block: rows that chose it
    int32_t btail[kTB];              // 1 for a block of the tail span
};

struct UnionAttnArgs {
    const h16 *q;           // [n_q][hq][128]
    const h16 *kc, *vc;     // token-major caches
    const int32_t *uid;     // [groups][cap_u]
    const uint32_t *umask;  // [groups][cap_u]
    const int32_t *n_u;     // [groups]
    int32_t cap_u;
    int32_t n_q, pos0, hq, hkv;
    float scale;
    int32_t splits;
    float *part;            // [n_q][hq][splits][130] when splits > 1
    float *out;             // [n_q][hq][128]
};

template <int GQA>
__global__ __launch_bounds__(kUAThreads, 2) void union_attn_kernel(UnionAttnArgs a)
{
    constexpr int G = 128 / GQA;  // rows per group
    __shared__ UnionAttnLds sm;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n = lane & 15, g4 = lane >> 4;
    const int32_t g = blockIdx.x, h = blockIdx.y, split = blockIdx.z;
    const int32_t r0 = g * G;
    const int32_t nr = min(G, a.n_q - r0);
    const int64_t kt = (int64_t)a.hkv * kDim;  // elements per token row

    // virtual block list: the union, then the blocks of the tail span [t0, t1)
    const int32_t nu = a.n_u[g];
    const int32_t t0 = ((a.pos0 + r0 + 1) / kBlockTokens) * kBlockTokens;
    const int32_t t1 = a.pos0 + r0 + nr;
    const int32_t ntb = t1 > t0 ? (t1 - 1) / kBlockTokens - t0 / kBlockTokens + 1 : 0;
    const int32_t n_virt = nu + ntb;
    const int32_t n_tiles = (n_virt + kTB - 1) / kTB;
    const int32_t tps = (n_tiles + a.splits - 1) / a.splits;
    const int32_t tb = min(n_tiles, split * tps), te = min(n_tiles, tb + tps);
    const int32_t *ug = a.uid + (int64_t)g * a.cap_u;
    const uint32_t *mg = a.umask + (int64_t)g * a.cap_u;

    auto block_of = [&](int32_t v, uint32_t &mask, int32_t &tail) -> int32_t {
        mask = 0u;
        tail = 0;
        if (v < nu) {
            mask = mg[v];
            return ug[v];
        }
        if (v < n_virt) {
            tail = 1;
            return t0 / kBlockTokens + (v - nu);
        }
        return -1;
    };

    // this lane's two queries (nb = 0, 1): m = 32 wave + 16 nb + n
    int32_t qrow[2];
    h16x8 qf[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; nb++) {
        const int m = 32 * wave + 16 * nb + n;
        qrow[nb] = m / GQA;
        const int32_t r = r0 + qrow[nb];
        const int hh = h * GQA + m % GQA;
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            qf[nb][ks] = (qrow[nb] < nr)
                             ? *(const h16x8 *)(a.q + ((int64_t)r * a.hq + hh) * kDim + 32 * ks + 8 * g4)
                             : h16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    int32_t p_last[2], tail_lo[2];
#pragma unroll
    for (int nb = 0; nb < 2; nb++) {
        p_last[nb] = a.pos0 + r0 + qrow[nb];
        tail_lo[nb] = ((p_last[nb] + 1) / kBlockTokens) * kBlockTokens;
    }

    // staging registers: K (cell t/4, 32 dims), V (block t/16, 8 dims x 4 cells)
    const int kcell = t >> 2, kpart = (t & 3) * 32;
    const int vblk = t >> 4, vch = (t & 15) * 8;
    h16x8 kr[4], vr[4];
    uint32_t meta_mask = 0u;
    int32_t meta_id = -1, meta_tail = 0;
    auto gload = [&](int32_t tile) {
        const int32_t vbase = tile * kTB;
        uint32_t mk;
        int32_t tl;
        {
            const int32_t id = block_of(vbase + (kcell >> 2), mk, tl);
            const int32_t c = id * kBlockTokens + (kcell & 3);
            const bool ok = id >= 0 && c < t1;
#pragma unroll
            for (int j = 0; j < 4; j++)
                kr[j] = ok ? *(const h16x8 *)(a.kc + (int64_t)c * kt + (int64_t)h * kDim + kpart + 8 * j)
                           : h16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        {
            const int32_t id = block_of(vbase + vblk, mk, tl);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int32_t c = id * kBlockTokens + e;
                vr[e] = (id >= 0 && c < t1)
                            ? *(const h16x8 *)(a.vc + (int64_t)c * kt + (int64_t)h * kDim + vch)
                            : h16x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        if (t < kTB)
            meta_id = block_of(vbase + t, meta_mask, meta_tail);
    };
    auto sstore = [&]() {
#pragma unroll
        for (int j = 0; j < 4; j++)
            *(h16x8 *)&sm.ks[kcell * KP + kpart + 8 * j] = kr[j];
#pragma unroll
        for (int i = 0; i < 8; i++)
            *(h16x4 *)&sm.vt[(vch + i) * VP + vblk * 4] = h16x4{vr[0][i], vr[1][i], vr[2][i], vr[3][i]};
        if (t < kTB) {
            sm.bid[t] = meta_id;
            sm.bmask[t] = meta_mask;
            sm.btail[t] = meta_tail;
        }
    };

    f32x4 oacc[2][8];
#pragma unroll
    for (int nb = 0; nb < 2; nb++)
#pragma unroll
        for (int i = 0; i < 8; i++)
            oacc[nb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    const float sl2 = a.scale * kLog2e;

    if (tb < te)
        gload(tb);
    for (int32_t tile = tb; tile < te; tile++) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (tile + 1 < te)
            gload(tile + 1);

        // S^T = K Q^T: lane holds cells 16 mb + 4 g4 + e of queries n (+16 nb)
        f32x4 sacc[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; nb++)
#pragma unroll
            for (int mb = 0; mb < 4; mb++)
                sacc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                const h16x8 kf = *(const h16x8 *)&sm.ks[(16 * mb + n) * KP + 32 * ks + 8 * g4];
#pragma unroll
                for (int nb = 0; nb < 2; nb++)
                    sacc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[nb][ks], sacc[nb][mb],
                                                                         0, 0, 0);
            }
        }

        // mask, online softmax, P in the k-slot order of the PV product
        int32_t bid[4], btl[4];
        uint32_t bmk[4];
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            bid[mb] = sm.bid[4 * mb + g4];
            bmk[mb] = sm.bmask[4 * mb + g4];
            btl[mb] = sm.btail[4 * mb + g4];
        }
        h16x8 pf[2][2];
#pragma unroll
        for (int nb = 0; nb < 2; nb++) {
            float s[4][4];
            float tmax = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int32_t c = bid[mb] * kBlockTokens + e;
                    const bool vis = bid[mb] >= 0 &&
                                     (btl[mb] ? (c >= tail_lo[nb] && c <= p_last[nb])
                                              : ((bmk[mb] >> qrow[nb]) & 1u) != 0u);
                    s[mb][e] = vis ? sacc[nb][mb][e] * sl2 : -INFINITY;
                    tmax = fmaxf(tmax, s[mb][e]);
                }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
            const float mnew = fmaxf(m_run[nb], tmax);
            const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m_run[nb] - mnew);
            float psum = 0.f;
#pragma unroll
            for (int mb = 0; mb < 4; mb++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float p = (s[mb][e] == -INFINITY) ? 0.f : exp2f(s[mb][e] - mnew);
                    s[mb][e] = p;
                    psum += p;
                }
            l_run[nb] = l_run[nb] * alpha + psum;
            m_run[nb] = mnew;
#pragma unroll
            for (int i = 0; i < 8; i++)
                oacc[nb][i] *= alpha;
#pragma unroll
            for (int kc = 0; kc < 2; kc++)
                pf[nb][kc] = h16x8{(h16)s[2 * kc][0],     (h16)s[2 * kc][1],
                                   (h16)s[2 * kc][2],     (h16)s[2 * kc][3],
                                   (h16)s[2 * kc + 1][0], (h16)s[2 * kc + 1][1],
                                   (h16)s[2 * kc + 1][2], (h16)s[2 * kc + 1][3]};
        }

        // O^T += V^T P^T: lane holds dv 16 i + 4 g4 + e of queries n (+16 nb)
#pragma unroll
        for (int i = 0; i < 8; i++) {
#pragma unroll
            for (int kc = 0; kc < 2; kc++) {
                const h16 *vp = &sm.vt[(16 * i + n) * VP + 32 * kc + 4 * g4];
                const h16x4 lo = *(const h16x4 *)vp;
                const h16x4 hi = *(const h16x4 *)(vp + 16);
                const h16x8 vf = h16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int nb = 0; nb < 2; nb++)
                    oacc[nb][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[nb][kc], oacc[nb][i],
                                                                        0, 0, 0);
            }
        }
    }

    // the four lane groups hold different cells of the same queries
#pragma unroll
    for (int nb = 0; nb < 2; nb++) {
        float l = l_run[nb];
        l += __shfl_xor(l, 16, kWave);
        l += __shfl_xor(l, 32, kWave);
        if (qrow[nb] >= nr)
            continue;
        const int m = 32 * wave + 16 * nb + n;
        const int64_t qh = (int64_t)(r0 + qrow[nb]) * a.hq + h * GQA + m % GQA;
        if (a.splits == 1) {
            const float inv = 1.f / l;
#pragma unroll
            for (int i = 0; i < 8; i++)
                *(f32x4 *)(a.out + qh * kDim + 16 * i + 4 * g4) = oacc[nb][i] * inv;
        } else {
            float *pb = a.part + (qh * a.splits + split) * (kDim + 2);
            if (g4 == 0) {
                pb[0] = m_run[nb];
                pb[1] = l;
            }
#pragma unroll
            for (int i = 0; i < 8; i++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    pb[2 + 16 * i + 4 * g4 + e] = oacc[nb][i][e];
        }
    }
}

}  // namespace

bool union_supported(int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t k)
{
    if (hkv < 1 || hq % hkv || d != kDim || dv != kDim)
        return false;
    const int32_t gqa = hq / hkv;
    if (gqa != 4 && gqa != 8 && gqa != 16)
        return false;
    return (int64_t)(128 / gqa) * k <= kUnionCap;
}

int32_t union_group_rows(int32_t hq, int32_t hkv) { return 128 / (hq / hkv); }

int32_t union_splits(int32_t n_q, int32_t hq, int32_t hkv)
{
    const int32_t groups = (n_q + union_group_rows(hq, hkv) - 1) / union_group_rows(hq, hkv);
    const int32_t wgs = groups * hkv;
    int32_t s = (kUnionTargetWgs + wgs - 1) / wgs;
    return s < 1 ? 1 : (s > kUnionMaxSplits ? kUnionMaxSplits : s);
}

hipError_t launch_union_attn(const UnionArgs &u, hipStream_t s)
{
    const int32_t G = union_group_rows(u.hq, u.hkv);
    const int32_t groups = (u.n_q + G - 1) / G;
    const int32_t cap_u = G * u.k;
    hipLaunchKernelGGL(union_build_kernel, dim3((uint32_t)groups), dim3(kUBThreads), 0, s, u.blk,
                       u.ldb, u.pos0, u.n_q, u.k, G, cap_u, u.uid, u.umask, u.n_u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    UnionAttnArgs a;
    a.q = u.q;
    a.kc = u.k_cache;
    a.vc = u.v_cache;
    a.uid = u.uid;
    a.umask = u.umask;
    a.n_u = u.n_u;
    a.cap_u = cap_u;
    a.n_q = u.n_q;
    a.pos0 = u.pos0;
    a.hq = u.hq;
    a.hkv = u.hkv;
    a.scale = u.scale;
    a.splits = u.splits;
    a.part = u.part;
    a.out = u.out;
    const dim3 grid((uint32_t)groups, (uint32_t)u.hkv, (uint32_t)u.splits);
    switch (u.hq / u.hkv) {
    case 4: hipLaunchKernelGGL(union_attn_kernel<4>, grid, dim3(kUAThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL(union_attn_kernel<8>, grid, dim3(kUAThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL(union_attn_kernel<16>, grid, dim3(kUAThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess || u.splits == 1)
        return e;
    return launch_combine(u.part, u.hq, u.splits, kDim, u.n_q, u.out, s);
}

}  // namespace qsa
