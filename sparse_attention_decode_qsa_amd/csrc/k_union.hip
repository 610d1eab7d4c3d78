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

constexpr int kSetThreads = 256;  // 4 waves: one set of 128 queries
constexpr int kTB = 16;           // blocks per tile
constexpr int kTC = kTB * kBlockTokens;  // cells per tile
constexpr int kDim = 128;         // D = DV
constexpr int KP = kDim + 8;      // K tile pitch (halfs)
constexpr int VP = kTC + 4;       // V^T tile pitch (halfs)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.f;  // log2 headroom of the softmax reference (see below)

struct UnionBuildLds {
    uint32_t bits[kWinWords];
    uint32_t pre[kWinWords];
    uint32_t msk[kUnionCap];
    Scratch<kUBThreads> S;
    uint32_t total;
};

__global__ __launch_bounds__(kUBThreads) void union_build_kernel(
    const int32_t *__restrict__ blk, int32_t ldb, int32_t pos0, int32_t n_q, int32_t k, int32_t G,
    int32_t cap_u, int32_t u_limit, int32_t *__restrict__ uid, uint32_t *__restrict__ umask,
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
    // this thread's chosen ids (entry e = t + j * kUBThreads is row e / k, slot
    // e % k), loaded once; -1 where the entry is past the row's choices, and for an
    // id outside the row's [0, nb_r) (only a broken selection has one: dropped, as
    // the per-row attention drops it, so no row reaches past its own prefix)
    constexpr int kPer = kUnionCap / kUBThreads;
    int32_t myid[kPer];
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const int32_t e = t + j * kUBThreads;
        const int32_t i = e / k, sl = e - i * k;
        const int32_t nb_r = (pos0 + r0 + i + 1) / kBlockTokens;
        const bool ok = e < n_ent && sl < min(k, nb_r);
        const int32_t id = ok ? blk[(int64_t)(r0 + i) * ldb + sl] : -1;
        myid[j] = (id >= 0 && id < nb_r) ? id : -1;
    }
    uint32_t base = 0;
    for (int32_t w0 = 0; w0 < nb_hi; w0 += kWinBlocks) {
        const int32_t nwb = min(kWinBlocks, nb_hi - w0);
        const int32_t nw = (nwb + 31) / 32;
        for (int32_t i = t; i < nw; i += kUBThreads)
            sm.bits[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPer; j++) {
            const uint32_t id = (uint32_t)(myid[j] - w0);
            if (myid[j] >= 0 && id < (uint32_t)nwb)
                atomicOr(&sm.bits[id >> 5], 1u << (id & 31));
        }
        __syncthreads();
        const int32_t per = (nw + kUBThreads - 1) / kUBThreads;
        const int32_t wa = t * per, wb = min(nw, wa + per);
        uint32_t c = 0;
        for (int32_t w = wa; w < wb; w++)
            c += __popc(sm.bits[w]);
        uint32_t pos = base + wg_exclusive_scan<kUBThreads>(c, sm.S);
        if (t == kUBThreads - 1)
            sm.total = pos + c;
        __syncthreads();
        if (sm.total > (uint32_t)u_limit) {
            // past the limit: the group goes per row, only its count is needed
            if (t == 0)
                n_u[g] = (int32_t)sm.total;
            return;
        }
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
#pragma unroll
        for (int j = 0; j < kPer; j++) {
            const uint32_t id = (uint32_t)(myid[j] - w0);
            if (myid[j] >= 0 && id < (uint32_t)nwb) {
                const int32_t row = (t + j * kUBThreads) / k;
                const uint32_t w = id >> 5;
                const uint32_t p = sm.pre[w] + __popc(sm.bits[w] & ((1u << (id & 31)) - 1u));
                atomicOr(&sm.msk[p], 1u << row);
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

struct alignas(16) UnionTile {
    alignas(16) h16 ks[kTC * KP];    // K tile, [cell][d]
    alignas(16) h16 vt[kDim * VP];   // V tile transposed, [dv][cell]
    int32_t bid[kTB];                // block id of each tile block, -1 past the end
    uint32_t bmask[kTB];             // union block: rows that chose it; 0 otherwise
    int32_t btail[kTB];              // 1 for a block of the tail span
};
template <int SETS>
struct alignas(16) UnionTiles {
    UnionTile buf[SETS][2];          // per set: the tile being read and the next one
};
struct alignas(16) UnionMerge {      // set 1's state, for set 0 to merge
    f32x4 o[4][16][kWave];
    float m[4][2][kWave];
    float l[4][2][kWave];
};
template <int SETS>
union UnionAttnLds {
    UnionTiles<SETS> tiles;
    UnionMerge merge;
};

constexpr int kPartStride = kUnionPartStride;  // (m, l, -, -) then o: 16-byte aligned
static_assert(kPartStride == 4 + kDim, "partial row layout");

struct UnionAttnArgs {
    const h16 *q;           // [n_q][hq][128]
    const h16 *kc, *vc;     // token-major caches
    const int32_t *uid;     // [groups][cap_u]
    const uint32_t *umask;  // [groups][cap_u]
    const int32_t *n_u;     // [groups]
    int32_t cap_u;
    int32_t u_limit;        // groups with more union blocks are the per-row kernel's
    int32_t n_q, pos0, hq, hkv;
    float scale;
    int32_t splits;
    float *part;            // [n_q][hq][splits][kPartStride] when splits > 1
    float *out;             // [n_q][hq][128]
};

// SETS wave sets of 4 waves per work group take alternate tiles and merge through
// LDS at the end (SETS = 2), or each work group is one set (SETS = 1).
template <int GQA, int SETS>
__global__ __launch_bounds__(kSetThreads * SETS, 3 - SETS) void union_attn_kernel(UnionAttnArgs a)
{
    constexpr int G = 128 / GQA;  // rows per group
    constexpr int kUASets = SETS;
    __shared__ UnionAttnLds<SETS> sm;
    const int lane = threadIdx.x & 63;
    const int set = threadIdx.x >> 8, t = threadIdx.x & 255, wave = t >> 6;  // within the set
    const int n = lane & 15, g4 = lane >> 4;
    const int32_t g = blockIdx.x, h = blockIdx.y, split = blockIdx.z;
    const int32_t r0 = g * G;
    const int32_t nr = min(G, a.n_q - r0);
    const int64_t kt = (int64_t)a.hkv * kDim;  // elements per token row

    // virtual block list: the union, then the blocks of the tail span [t0, t1)
    const int32_t nu = a.n_u[g];
    if (nu > a.u_limit)
        return;  // the per-row kernel takes this group (uniform over the work group)
    const int32_t t0 = ((a.pos0 + r0 + 1) / kBlockTokens) * kBlockTokens;
    const int32_t t1 = a.pos0 + r0 + nr;
    const int32_t ntb = t1 > t0 ? (t1 - 1) / kBlockTokens - t0 / kBlockTokens + 1 : 0;
    const int32_t n_virt = nu + ntb;
    const int32_t n_tiles = (n_virt + kTB - 1) / kTB;
    const int32_t tps = (n_tiles + a.splits - 1) / a.splits;
    const int32_t tb = min(n_tiles, split * tps), te = min(n_tiles, tb + tps);
    const int32_t *ug = a.uid + (int64_t)g * a.cap_u;
    const uint32_t *mg = a.umask + (int64_t)g * a.cap_u;

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

    // Thread t stages block t / 16 of a tile: K cell t / 4 (32 dims) and V dims
    // 8 (t % 16) .. + 8 of the block's 4 cells; (t % 16) == 0 writes the block's
    // entry.  The block's id and mask are fetched two tiles ahead, its K/V one
    // tile ahead.
    const int vb = t >> 4;
    const int kpart = (t & 15) * 8;  // K and V: 16 lanes cover one 256-byte cell row
    const int vch = (t & 15) * 8;
    struct Meta {
        int32_t id;
        uint32_t mask;
        int32_t tail;
    };
    auto meta_of = [&](int32_t tile) -> Meta {
        const int32_t v = tile * kTB + vb;
        if (v < nu)
            return Meta{ug[v], mg[v], 0};
        if (v < n_virt)
            return Meta{t0 / kBlockTokens + (v - nu), 0u, 1};
        return Meta{-1, 0u, 0};
    };
    h16x8 kr[4], vr[4];
    Meta staged{-1, 0u, 0};
    const h16 *kbase = a.kc + (int64_t)h * kDim + kpart;
    const h16 *vbase = a.vc + (int64_t)h * kDim + vch;
    // Every load is unconditional: a cell that is not there (no block, or past t1)
    // reads token 0's row, a real, finite row whose weight the masks make 0 (a
    // missing block has an empty mask; cells past t1 lie in tail blocks, masked per
    // cell).  Conditional loads made the compiler branch around each one (3% slower).
    auto kv_load = [&](const Meta &m) {
        staged = m;
        const int32_t cb = m.id >= 0 ? m.id * kBlockTokens : 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int64_t off = (int64_t)((m.id >= 0 && cb + e < t1) ? cb + e : 0) * kt;
            kr[e] = *(const h16x8 *)(kbase + off);
            vr[e] = *(const h16x8 *)(vbase + off);
        }
    };
    auto sstore = [&](UnionTile &T) {
#pragma unroll
        for (int e = 0; e < 4; e++)
            *(h16x8 *)&T.ks[(vb * 4 + e) * KP + kpart] = kr[e];
#pragma unroll
        for (int i = 0; i < 8; i++)
            *(h16x4 *)&T.vt[(vch + i) * VP + vb * 4] = h16x4{vr[0][i], vr[1][i], vr[2][i], vr[3][i]};
        if ((t & 15) == 0) {
            T.bid[vb] = staged.id;
            T.bmask[vb] = staged.mask;
            T.btail[vb] = staged.tail;
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

    // set s takes tiles tb + s, tb + s + 2, ...; both sets pass the same barriers
    UnionTile *buf = sm.tiles.buf[set];
    const int32_t first = tb + set;
    Meta ahead{-1, 0u, 0};
    if (first < te) {
        kv_load(meta_of(first));
        if (first + kUASets < te)
            ahead = meta_of(first + kUASets);
        sstore(buf[0]);
    }
    __syncthreads();
    if (first + kUASets < te) {
        kv_load(ahead);
        if (first + 2 * kUASets < te)
            ahead = meta_of(first + 2 * kUASets);
    }
    const int32_t n_iter = (te - tb + kUASets - 1) / kUASets;
    for (int32_t j = 0; j < n_iter; j++) {
        const int32_t tile = first + kUASets * j;
        if (tile < te) {
        const UnionTile &T = buf[j & 1];
        const bool has_tail = (tile + 1) * kTB > nu && ntb > 0;  // uniform

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
                const h16x8 kf = *(const h16x8 *)&T.ks[(16 * mb + n) * KP + 32 * ks + 8 * g4];
#pragma unroll
                for (int nb = 0; nb < 2; nb++)
                    sacc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[nb][ks], sacc[nb][mb],
                                                                         0, 0, 0);
            }
        }

        // mask (per block; per cell only in a tile holding the tail span), online
        // softmax, P in the k-slot order of the PV product
        uint32_t bmk[4];
#pragma unroll
        for (int mb = 0; mb < 4; mb++)
            bmk[mb] = T.bmask[4 * mb + g4];
        h16x8 pf[2][2];
        bool rescale = false;
        float alpha[2];
#pragma unroll
        for (int nb = 0; nb < 2; nb++) {
            float s[4][4];
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                const bool vis = ((bmk[mb] >> qrow[nb]) & 1u) != 0u;
#pragma unroll
                for (int e = 0; e < 4; e++)
                    s[mb][e] = vis ? sacc[nb][mb][e] : -INFINITY;
            }
            if (has_tail) {
#pragma unroll
                for (int mb = 0; mb < 4; mb++) {
                    if (T.btail[4 * mb + g4]) {
                        const int32_t c0 = T.bid[4 * mb + g4] * kBlockTokens;
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            s[mb][e] = (c0 + e >= tail_lo[nb] && c0 + e <= p_last[nb])
                                           ? sacc[nb][mb][e]
                                           : -INFINITY;
                    }
                }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 4; mb++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    tmax = fmaxf(tmax, s[mb][e]);
            tmax = max_across_rows(tmax);
            // scores are scaled inside the exponent: p = 2^(s * sl2 - m).  The
            // reference m moves only when the tile's maximum passes it by more than
            // kLazyMax (p then stays below 2^kLazyMax; o and l share the reference,
            // so o / l is unchanged up to rounding), which spares most tiles the
            // rescale of the outputs
            const float tm = tmax * sl2;
            const float mnew = tm > m_run[nb] + kLazyMax ? tm : m_run[nb];
            const float mref = (mnew == -INFINITY) ? 0.f : mnew;
            alpha[nb] = __builtin_amdgcn_exp2f(m_run[nb] - mref);
            rescale |= mnew != m_run[nb];
            float psum = 0.f;
#pragma unroll
            for (int mb = 0; mb < 4; mb++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][e], sl2, -mref));
                    s[mb][e] = p;
                    psum += p;
                }
            l_run[nb] = l_run[nb] * alpha[nb] + psum;
            m_run[nb] = mnew;
#pragma unroll
            for (int kc = 0; kc < 2; kc++)
                pf[nb][kc] = h16x8{(h16)s[2 * kc][0],     (h16)s[2 * kc][1],
                                   (h16)s[2 * kc][2],     (h16)s[2 * kc][3],
                                   (h16)s[2 * kc + 1][0], (h16)s[2 * kc + 1][1],
                                   (h16)s[2 * kc + 1][2], (h16)s[2 * kc + 1][3]};
        }
        // O is rescaled only when some lane's running maximum moved
        if (__any(rescale)) {
#pragma unroll
            for (int nb = 0; nb < 2; nb++)
#pragma unroll
                for (int i = 0; i < 8; i++)
                    oacc[nb][i] *= alpha[nb];
        }

        // O^T += V^T P^T: lane holds dv 16 i + 4 g4 + e of queries n (+16 nb)
#pragma unroll
        for (int i = 0; i < 8; i++) {
#pragma unroll
            for (int kc = 0; kc < 2; kc++) {
                const h16 *vp = &T.vt[(16 * i + n) * VP + 32 * kc + 4 * g4];
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
        // this set's next tile into its other buffer, then one barrier; then the
        // loads of the tile after it
        if (tile + kUASets < te)
            sstore(buf[(j + 1) & 1]);
        __syncthreads();
        if (tile + 2 * kUASets < te) {
            kv_load(ahead);
            if (tile + 3 * kUASets < te)
                ahead = meta_of(tile + 3 * kUASets);
        }
    }

    // the four lane groups hold different cells of the same queries
    float l_tot[2];
#pragma unroll
    for (int nb = 0; nb < 2; nb++) {
        float l = l_run[nb];
        l += __shfl_xor(l, 16, kWave);
        l += __shfl_xor(l, 32, kWave);
        l_tot[nb] = l;
    }
    // set 1 hands its state to set 0 through LDS (the tiles are no longer read)
    if (SETS == 2 && set == 1) {
#pragma unroll
        for (int nb = 0; nb < 2; nb++) {
            sm.merge.m[wave][nb][lane] = m_run[nb];
            sm.merge.l[wave][nb][lane] = l_tot[nb];
#pragma unroll
            for (int i = 0; i < 8; i++)
                sm.merge.o[wave][nb * 8 + i][lane] = oacc[nb][i];
        }
    }
    if (SETS == 2) {
        __syncthreads();
        if (set == 1)
            return;
    }
#pragma unroll
    for (int nb = 0; nb < 2 && SETS == 2; nb++) {
        const float m1 = sm.merge.m[wave][nb][lane];
        const float mm = fmaxf(m_run[nb], m1);
        const float mref = (mm == -INFINITY) ? 0.f : mm;
        const float a0 = __builtin_amdgcn_exp2f(m_run[nb] - mref);
        const float a1 = __builtin_amdgcn_exp2f(m1 - mref);
        l_tot[nb] = a0 * l_tot[nb] + a1 * sm.merge.l[wave][nb][lane];
        m_run[nb] = mm;
#pragma unroll
        for (int i = 0; i < 8; i++)
            oacc[nb][i] = a0 * oacc[nb][i] + a1 * sm.merge.o[wave][nb * 8 + i][lane];
    }
#pragma unroll
    for (int nb = 0; nb < 2; nb++) {
        const float l = l_tot[nb];
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
            float *pb = a.part + (qh * a.splits + split) * kPartStride;
            if (g4 == 0)
                *(f32x4 *)pb = f32x4{m_run[nb], l, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 8; i++)
                *(f32x4 *)(pb + 4 + 16 * i + 4 * g4) = oacc[nb][i];
        }
    }
}

// Merge of the split partials of a prefill chunk: one work group per row, a
// thread per (query head, 4 output dims); weights w_s = 2^(m_s - M).
constexpr int kUCombThreads = 256;
__global__ __launch_bounds__(kUCombThreads) void union_combine_kernel(const float *__restrict__ part,
                                                                     int32_t hq, int32_t S,
                                                                     const int32_t *__restrict__ n_u,
                                                                     int32_t group_rows,
                                                                     int32_t u_limit,
                                                                     float *__restrict__ out)
{
    const int64_t row = blockIdx.x;
    if (n_u[row / group_rows] > u_limit)
        return;  // a per-row group: its output is the per-row kernel's
    for (int idx = threadIdx.x; idx < hq * (kDim / 4); idx += kUCombThreads) {
        const int h = idx / (kDim / 4), c = idx % (kDim / 4);
        const float *pb = part + (row * hq + h) * S * kPartStride;
        float M = -INFINITY;
        for (int sp = 0; sp < S; sp++)
            M = fmaxf(M, pb[sp * kPartStride]);
        const float mref = (M == -INFINITY) ? 0.f : M;
        float L = 0.f;
        f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < S; sp++) {
            const f32x4 ml = *(const f32x4 *)(pb + sp * kPartStride);
            const float w = __builtin_amdgcn_exp2f(ml[0] - mref);
            L += w * ml[1];
            o += w * *(const f32x4 *)(pb + sp * kPartStride + 4 + 4 * c);
        }
        *(f32x4 *)(out + (row * hq + h) * kDim + 4 * c) = o * (1.f / L);
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
    const int64_t G = union_group_rows(hq, hkv);
    const int64_t wgs = (((int64_t)n_q + G - 1) / G) * hkv;
    const int64_t s = (kUnionTargetWgs + wgs - 1) / wgs;
    return s < 1 ? 1 : (s > kUnionMaxSplits ? kUnionMaxSplits : (int32_t)s);
}

hipError_t launch_union_attn(const UnionArgs &u, hipStream_t s)
{
    const int32_t G = union_group_rows(u.hq, u.hkv);
    const int32_t groups = (u.n_q + G - 1) / G;
    const int32_t cap_u = G * u.k;
    hipLaunchKernelGGL(union_build_kernel, dim3((uint32_t)groups), dim3(kUBThreads), 0, s, u.blk,
                       u.ldb, u.pos0, u.n_q, u.k, G, cap_u, u.u_limit, u.uid, u.umask, u.n_u);
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
    a.u_limit = u.u_limit;
    a.n_q = u.n_q;
    a.pos0 = u.pos0;
    a.hq = u.hq;
    a.hkv = u.hkv;
    a.scale = u.scale;
    a.splits = u.splits;
    a.part = u.part;
    a.out = u.out;
    const dim3 grid((uint32_t)groups, (uint32_t)u.hkv, (uint32_t)u.splits);
    const dim3 block(kSetThreads * kUnionSets);
    switch (u.hq / u.hkv) {
    case 4: hipLaunchKernelGGL((union_attn_kernel<4, kUnionSets>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((union_attn_kernel<8, kUnionSets>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((union_attn_kernel<16, kUnionSets>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (u.u_limit >= cap_u) {
        // no group can exceed the limit: the union kernel's partials, if split
        if (u.splits == 1)
            return hipSuccess;
        hipLaunchKernelGGL(union_combine_kernel, dim3((uint32_t)u.n_q), dim3(kUCombThreads), 0, s,
                           u.part, u.hq, u.splits, u.n_u, G, u.u_limit, u.out);
        return hipGetLastError();
    }
    // the groups whose union is too large for the union form to pay go per row; the
    // same launch merges the other groups' split partials
    RowsArgs ra;
    ra.q = u.q;
    ra.blk = u.blk;
    ra.ldb = u.ldb;
    ra.k_cache = u.k_cache;
    ra.v_cache = u.v_cache;
    ra.n_q = u.n_q;
    ra.pos0 = u.pos0;
    ra.k = u.k;
    ra.hq = u.hq;
    ra.hkv = u.hkv;
    ra.scale = u.scale;
    ra.out = u.out;
    ra.n_u = u.n_u;
    ra.group_rows = G;
    ra.u_limit = u.u_limit;
    ra.part = u.part;
    ra.splits = u.splits;
    return launch_rows_attn(ra, s);
}

int32_t union_limit(int32_t hq, int32_t hkv, int32_t k)
{
    // A union block costs the union kernel about 8/3 of what one row's block costs
    // the per-row kernel (measured at depth 126,253: 1.7-2.2 ns against 0.76 ns per
    // block, whole chip), so the union pays while it holds at most 3/8 of the
    // group's rows x k blocks (6 k for groups of 16 rows).
    return (int32_t)(((int64_t)union_group_rows(hq, hkv) * k * 3) / 8);
}

}  // namespace qsa
