// Top-k over block scores in the block domain (Qiita part 10,
// "QSAとQSA indexerについて": keep the highest-scoring blocks; "block-domain
// top-k（COMMON-006）実装は見送り": select pools, then expand only the chosen ones).
//
// Forms:
//   * register form (prefill rows up to 65,536 blocks): one work group per row,
//     the row's keys held in registers;
//   * rows form (longer prefill rows): one work group per row, straight from
//     global memory (select_row_global);
//   * list form (one decode row): the row's candidate lists (written by the
//     decode scan, or built from a score array by score_lists_kernel) and one
//     1024-thread work group running lists_select, with select_row_global as
//     the exact fallback.
// Ids come out in ascending order; equal scores go to the lower id.
#include <mutex>

#include "qsa_select.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- register form
// One 1024-thread work group per row; the row's keys stay in registers (KPT per
// thread, element (j, e) of thread t is id 4*(j*1024 + t) + e), so the scores are
// read once and nothing leaves the work group.  Used for rows of up to 1024*KPT
// blocks (65,536 at KPT = 64, i.e. contexts up to 262,147 tokens).
constexpr int kRegThreads = 1024;
constexpr int kListCap = 4096;  // keys in bins >= the lower bound, kept in LDS

// Two work groups per CU (8 waves per SIMD, at most 64 registers, a few spilled
// outside the key loops): one work group's row loads overlap the other's histogram
// and ranking passes.  At one work group per CU (79-103 registers) the 1,024 rows
// of a chunk took 42 / 66 / 105 us at 15,000 / 31,800 / 62,800 blocks per row,
// against 31 / 48 / 84 us.
template <int KPT>
__global__ __launch_bounds__(kRegThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void topk_reg_kernel(const float *__restrict__ scores,
                                                               int32_t ld, int32_t pos0,
                                                               int32_t k, int32_t *__restrict__ blk,
                                                               int32_t *__restrict__ n_sel)
{
    constexpr int NT = kRegThreads;
    constexpr int V4 = KPT / 4;
    __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
    __shared__ uint64_t cand[kCandCap];
    __shared__ uint32_t lst[kListCap];
    __shared__ uint32_t bitmap[NT * KPT / 32];
    __shared__ Scratch<NT> S;

    const int t = threadIdx.x;
    const int32_t r = blockIdx.x;
    const float *row = scores + (int64_t)r * ld;
    const uint32_t nb = (uint32_t)((pos0 + r + 1) / kBlockTokens);
    int32_t *outr = blk + (int64_t)r * k;
    if (nb <= (uint32_t)k) {
        for (uint32_t i = t; i < nb; i += NT)
            outr[i] = (int32_t)i;
        if (t == 0)
            n_sel[r] = (int32_t)nb;
        return;
    }
    auto id_of = [&](int j, int e) { return (uint32_t)(4 * (j * NT + t) + e); };
    // a fresh copy of t per loop keeps the compiler from holding 64 precomputed
    // addresses live across loops (they would spill)
    auto fresh_t = [&]() {
        int tt = t;
        asm volatile("" : "+v"(tt));
        return tt;
    };

    // top 16 key bits, two per register (the histogram and the bin test need 12)
    // Every load is issued unconditionally from an address inside the row, so the
    // loads of a group overlap (a load under a branch makes the compiler wait for
    // it where the branches merge).  Groups of 4 wholly below nb are 16-byte loads;
    // the row's last partial group is read once per thread with clamped scalar
    // loads; groups at or past nb give key 0.  A misaligned or very short row
    // takes clamped scalar loads throughout.
    uint32_t kp[KPT / 2];
    if ((((uintptr_t)row) & 15) == 0 && nb >= 4) {
        const uint32_t ip = nb & ~3u;  // first id of the partial group (if nb % 4)
        float pv[3];
#pragma unroll
        for (int e = 0; e < 3; e++)
            pv[e] = row[min(ip + e, nb - 1)];
#pragma unroll
        for (int j = 0; j < V4; j++) {
            const uint32_t i0 = id_of(j, 0);
            const bool full = i0 + 3 < nb;
            const f32x4 v = *(const f32x4 *)(row + (full ? i0 : 0u));
            const bool part = i0 == ip;
            uint32_t kk[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float x = part ? pv[e < 3 ? e : 0] : v[e];
                const bool on = full || (part && i0 + e < nb);
                kk[e] = score_key(x) & (0u - (uint32_t)on);  // no branch: 0 when off
            }
            kp[2 * j] = (kk[0] >> 16) | (kk[1] & 0xffff0000u);
            kp[2 * j + 1] = (kk[2] >> 16) | (kk[3] & 0xffff0000u);
            if ((j & 7) == 7)
                __builtin_amdgcn_sched_barrier(0);  // at most 8 row loads in flight per lane
        }
    } else {
#pragma unroll
        for (int j = 0; j < V4; j++) {
            const uint32_t i0 = id_of(j, 0);
            uint32_t kk[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float x = row[min(i0 + e, nb - 1)];
                kk[e] = score_key(x) & (0u - (uint32_t)(i0 + e < nb));
            }
            kp[2 * j] = (kk[0] >> 16) | (kk[1] & 0xffff0000u);
            kp[2 * j + 1] = (kk[2] >> 16) | (kk[3] & 0xffff0000u);
            if ((j & 7) == 7)
                __builtin_amdgcn_sched_barrier(0);
        }
    }
    auto bin_of = [&](int j) -> uint32_t {  // j-th key of this thread, top 12 bits
        const uint32_t w = kp[j >> 1];
        const uint32_t k16 = (j & 1) ? (w >> 16) : (w & 0xffffu);
        return k16 >> (16 - kHistBits);
    };
    // 1. A lower bound L on the threshold bin: the k-th largest of the per-thread
    //    maximum bins.  The k threads at or above it each hold a key in a bin
    //    >= L, so at least k keys lie in bins >= L (k <= 1024 = NT).
    uint32_t mybin = 0;
    {
        const int tt = fresh_t();
#pragma unroll
        for (int j = 0; j < KPT; j++)
            if ((uint32_t)(4 * ((j / 4) * NT + tt) + j % 4) < nb)
                mybin = max(mybin, bin_of(j));
    }
    for (int i = t; i < kHistBins; i += NT)
        hist[i] = 0;
    if (t == 0) {
        S.cnt = 0;
        S.cnt2 = 0;
    }
    __syncthreads();
    atomicAdd(&hist[mybin], 1u);
    __syncthreads();
    find_from_top<NT, kHistBins>(hist, (uint32_t)k, S);
    const uint32_t L = S.res[0];
    __syncthreads();
    // 2. The keys in bins >= L (a few per cent of the row) go to a short LDS list
    //    (16 key bits, 16 id bits).  Each thread counts its own first, so a wave
    //    reserves its slots with one LDS atomic instead of one per key.
    uint32_t mine = 0;
    {
#pragma unroll
        for (int j = 0; j < KPT / 2; j++)
            asm volatile("" : "+v"(kp[j]));
        const int tt = fresh_t();
#pragma unroll
        for (int j = 0; j < KPT; j++)
            mine += ((uint32_t)(4 * ((j / 4) * NT + tt) + j % 4) < nb && bin_of(j) >= L) ? 1u : 0u;
    }
    {
        const uint32_t incl = wave_incl_scan(mine);  // inclusive scan over the wave (DPP)
        uint32_t base = 0;
        if ((t & (kWave - 1)) == kWave - 1 && incl)
            base = atomicAdd(&S.cnt, incl);
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, kWave - 1) + incl - mine;
        if (mine) {
#pragma unroll
            for (int j = 0; j < KPT / 2; j++)
                asm volatile("" : "+v"(kp[j]));
            const int tt = fresh_t();
#pragma unroll
            for (int j = 0; j < KPT; j++) {
                const uint32_t id = (uint32_t)(4 * ((j / 4) * NT + tt) + j % 4);
                if (id < nb && bin_of(j) >= L) {
                    if (base < (uint32_t)kListCap) {
                        const uint32_t w = kp[j >> 1];
                        const uint32_t k16 = (j & 1) ? (w >> 16) : (w & 0xffffu);
                        lst[base] = (k16 << 16) | id;
                    }
                    base++;
                }
            }
        }
    }
    for (int i = t; i < kHistBins; i += NT)
        hist[i] = 0;
    __syncthreads();
    const uint32_t n_list = S.cnt;
    const bool short_list = n_list <= (uint32_t)kListCap;
    if (short_list) {
        for (uint32_t i = t; i < n_list; i += NT)
            atomicAdd(&hist[lst[i] >> (32 - kHistBits)], 1u);
    } else {
        // long list (flat score distributions): histogram of every key >= L
#pragma unroll
        for (int j = 0; j < KPT / 2; j++)
            asm volatile("" : "+v"(kp[j]));
        const int tt = fresh_t();
#pragma unroll
        for (int j = 0; j < KPT; j++) {
            const uint32_t bin = bin_of(j);
            if ((uint32_t)(4 * ((j / 4) * NT + tt) + j % 4) < nb && bin >= L)
                atomicAdd(&hist[bin], 1u);
        }
    }
    __syncthreads();
    find_from_top<NT, kHistBins>(hist, (uint32_t)k, S);
    const uint32_t B = S.res[0];
    uint32_t need = (uint32_t)k - S.res[1];
    const uint32_t W = (nb + 31) / 32;
    for (uint32_t i = t; i < W; i += NT)
        bitmap[i] = 0;
    for (int i = t; i < 16; i += NT)  // hist[0..15] becomes a digit histogram
        hist[i] = 0;
    if (t == 0)
        S.cnt2 = 0;
    __syncthreads();
    if (short_list) {
        // 3. Bins above B are in.  Bin B's entries are split once more by the next
        //    4 key bits, which the list already holds.
        for (uint32_t i = t; i < n_list; i += NT) {
            const uint32_t e = lst[i];
            const uint32_t bin = e >> (32 - kHistBits);
            if (bin > B) {
                set_bit(bitmap, e & 0xffffu);
            } else if (bin == B) {
                atomicAdd(&hist[(e >> 16) & 15u], 1u);
            }
        }
        __syncthreads();
        // digit d where the count from the top reaches need (16 bins: one lane scan)
        if (t == 0) {
            uint32_t acc = 0, d = 0;
            for (int b = 15; b >= 0; b--) {
                if (acc + hist[b] >= need) {
                    d = (uint32_t)b;
                    break;
                }
                acc += hist[b];
            }
            S.res[0] = d;
            S.res[1] = acc;
            S.cnt = 0;
        }
        __syncthreads();
        const uint32_t d = S.res[0];
        need -= S.res[1];
        for (uint32_t i = t; i < n_list; i += NT) {
            const uint32_t e = lst[i];
            if ((e >> (32 - kHistBits)) != B)
                continue;
            const uint32_t dig = (e >> 16) & 15u;
            if (dig > d) {
                set_bit(bitmap, e & 0xffffu);
            } else if (dig == d) {
                const uint32_t slot = atomicAdd(&S.cnt, 1u);
                if (slot < kCandCap)
                    cand[slot] = e & 0xffffu;
            }
        }
    } else {
        // long list: walk every register-held key
        if (t == 0)
            S.cnt = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KPT / 2; j++)
            asm volatile("" : "+v"(kp[j]));
        const int tt = fresh_t();
#pragma unroll
        for (int j = 0; j < KPT; j++) {
            const uint32_t id = (uint32_t)(4 * ((j / 4) * NT + tt) + j % 4);
            const uint32_t bin = bin_of(j);
            if (id < nb) {
                if (bin > B) {
                    set_bit(bitmap, id);
                } else if (bin == B) {
                    const uint32_t slot = atomicAdd(&S.cnt, 1u);
                    if (slot < kCandCap)
                        cand[slot] = id;
                }
            }
        }
    }
    __syncthreads();
    const uint32_t c = S.cnt;
    // full keys of the candidates, fetched together (the row was just read: L2)
    for (uint32_t i = t; i < min(c, (uint32_t)kCandCap); i += NT) {
        const uint32_t id = (uint32_t)cand[i];
        cand[i] = ((uint64_t)score_key(row[id]) << 32) | id;
    }
    __syncthreads();
    if (c <= (uint32_t)NT) {
        // 4a. rank by counting: order (key desc, id asc) is strict, so candidate i
        //     is chosen iff fewer than `need` candidates rank before it
        const uint32_t c16 = (c + 15) & ~15u;
        if ((uint32_t)t >= c && (uint32_t)t < c16)
            cand[t] = 0x00000000ffffffffull;  // never ranks before anyone
        __syncthreads();
        if ((uint32_t)t < c) {
            const uint64_t me = cand[t];
            const uint32_t mk = (uint32_t)(me >> 32), mid = (uint32_t)me;
            uint32_t before = 0;
            for (uint32_t j0 = 0; j0 < c16; j0 += 16) {
                uint64_t o[16];
#pragma unroll
                for (int u = 0; u < 16; u++)
                    o[u] = cand[j0 + u];
#pragma unroll
                for (int u = 0; u < 16; u++) {
                    const uint32_t ok = (uint32_t)(o[u] >> 32), oid = (uint32_t)o[u];
                    before += (ok > mk || (ok == mk && oid < mid)) ? 1u : 0u;
                }
            }
            if (before < need)
                set_bit(bitmap, mid);
        }
    } else {
        // 4b. digit passes over the candidates (in LDS, or re-read from L2)
        uint32_t *h256 = hist;
        if (c <= (uint32_t)kCandCap) {
            LdsCands<NT> src{cand, c};
            resolve<NT>(src, B, need, nb, h256, S);
            const uint32_t T = S.res[0], I = S.res[1];
            src.each([&](uint32_t kk, uint32_t id) {
                if (kk > T || (kk == T && id <= I))
                    set_bit(bitmap, id);
            });
        } else {
            RowCands<NT> src{row, nb, B};
            resolve<NT>(src, B, need, nb, h256, S);
            const uint32_t T = S.res[0], I = S.res[1];
            src.each([&](uint32_t kk, uint32_t id) {
                if (kk > T || (kk == T && id <= I))
                    set_bit(bitmap, id);
            });
        }
    }
    __syncthreads();
    compact_bitmap<NT>(bitmap, nb, outr, (uint32_t)k, S);
    if (t == 0)
        n_sel[r] = k;
}

// ---------------------------------------------------------------- rows form
// Dynamic LDS: cand[kCandCap] (u64) | hist[4096] | bitmap[ceil(nb_max/32)]
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(const float *__restrict__ scores,
                                                             int32_t ld, int32_t pos0, int32_t k,
                                                             int32_t *__restrict__ blk,
                                                             int32_t *__restrict__ n_sel)
{
    extern __shared__ uint64_t lds64[];
    uint64_t *cand = lds64;
    uint32_t *hist = (uint32_t *)(cand + kCandCap);
    uint32_t *bitmap = hist + kHistBins;
    __shared__ Scratch<kThreads> S;

    const int32_t r = blockIdx.x;
    const float *row = scores + (int64_t)r * ld;
    const uint32_t nb = (uint32_t)((pos0 + r + 1) / kBlockTokens);
    int32_t *outr = blk + (int64_t)r * k;
    if (nb <= (uint32_t)k) {
        for (uint32_t i = threadIdx.x; i < nb; i += kThreads)
            outr[i] = (int32_t)i;
        if (threadIdx.x == 0)
            n_sel[r] = (int32_t)nb;
        return;
    }
    select_row_global<kThreads>(row, nb, k, outr, hist, cand, bitmap, S);
    if (threadIdx.x == 0)
        n_sel[r] = k;
}
// ---------------------------------------------------------------- list form
// One 1024-thread work group: thread w holds list w, lists_select finds R*, the
// chosen ids go into an LDS bitmap, compacted in ascending id order.
__global__ __launch_bounds__(kSelThreads) void topk_lists_kernel(const float *__restrict__ scores,
                                                                 int32_t nb, int32_t k,
                                                                 CandLists cl, int32_t W,
                                                                 ListLayout lay,
                                                                 int32_t *__restrict__ blk,
                                                                 int32_t *__restrict__ n_sel)
{
    constexpr int NT = kSelThreads;
    __shared__ uint32_t bitmap[kMaxBlocks / 32];
    __shared__ uint64_t cand[kCandCap];
    __shared__ ListSelLds L;
    const int t = threadIdx.x;

    uint64_t R[kListLen];
    uint32_t nrows;
    load_list(cl, W, R, &nrows);
    zero_words<NT>(bitmap, ((uint32_t)nb + 31) / 32);
    uint64_t rs = 0;
    int sel;
    // at most two passes, the second after widening (one copy of the selection)
#pragma clang loop unroll(disable)
    for (int pass = 0;; pass++) {
        sel = lists_select(R, nrows, t < W, (uint32_t)k, L, &rs);
        if (sel != kListsHide || pass > 0 || !widen_lists(R, &nrows, W, rs, scores, lay, L))
            break;
        __syncthreads();
    }
    if (sel == kListsExact) {
#pragma unroll
        for (int j = 0; j < kListLen; j++)
            if (R[j] >= rs) {
                const uint32_t id = rank_id(R[j]);
                if (id < (uint32_t)nb)
                    set_bit(bitmap, id);
            }
        __syncthreads();
        compact_bitmap<NT>(bitmap, (uint32_t)nb, blk, (uint32_t)k, L.S);
    } else {
        __syncthreads();
        select_row_global<NT>(scores, (uint32_t)nb, k, blk, L.hist[0], cand, bitmap, L.S);
    }
    if (t == 0)
        n_sel[0] = k;
}

// Candidate lists from a score row, laid out as the decode scan lays them out:
// work group w owns the runs of 4 rows 4(w + nwg m) .. 4(w + nwg m) + 3; its
// rank keys go to LDS, and wave 0 takes the kListLen largest one at a time.
constexpr int kListBuildThreads = 512;
constexpr int kListBuildMaxRows = 4 * ((kMaxBlocks / 4 + kListWgs - 1) / kListWgs) + 4;

// Row r = blockIdx.y of the score array (stride ld) sees nb_r = (pos0 + r + 1) / 4
// blocks; its lists go to cl.list + r * kListWgs * kListLen, cl.rows + r * kListWgs.
__global__ __launch_bounds__(kListBuildThreads) void score_lists_kernel(
    const float *__restrict__ scores, int32_t ld, int32_t pos0, CandLists cl)
{
    __shared__ uint64_t rk[kListBuildMaxRows];
    __shared__ uint32_t n_own;
    const int t = threadIdx.x;
    const int64_t nwg = gridDim.x, w = blockIdx.x;
    const int32_t row = blockIdx.y;
    const int32_t nb = (pos0 + row + 1) / kBlockTokens;
    scores += (int64_t)row * ld;
    cl.list += (int64_t)row * kListWgs * kListLen;
    cl.rows += (int64_t)row * kListWgs;
    const int64_t runs = ((int64_t)nb + 3) / 4;
    const int64_t my_runs = runs > w ? (runs - w + nwg - 1) / nwg : 0;
    const int64_t n = min(my_runs * 4, (int64_t)kListBuildMaxRows);
    for (int64_t i = t; i < n; i += kListBuildThreads) {
        const int64_t r = 4 * (w + nwg * (i / 4)) + (i & 3);
        rk[i] = r < nb ? rank_key(scores[r], (uint32_t)r) : 0ull;
    }
    if (t == 0) {
        const int64_t last = 4 * (w + nwg * (my_runs - 1));  // first row of the last run
        n_own = my_runs == 0 ? 0u : (uint32_t)(4 * (my_runs - 1) + min((int64_t)4, nb - last));
    }
    __syncthreads();
    if (t < kWave) {
        for (int j = 0; j < kListLen; j++) {
            uint64_t best = 0ull;
            int at = -1;
            for (int64_t i = t; i < n; i += kWave)
                if (rk[i] > best) {
                    best = rk[i];
                    at = (int)i;
                }
            const uint64_t m = wave_max_u64(best);
            if (m != 0ull && best == m)
                rk[at] = 0ull;  // the one lane holding it (rank keys are distinct)
            if (t == 0)
                cl.list[w * kListLen + j] = m;
        }
        if (t == 0)
            cl.rows[w] = n_own;
    }
}

__global__ void iota_kernel(int32_t *blk, int32_t n, int32_t *n_sel)
{
    for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        blk[i] = i;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        n_sel[0] = n;
}

// Register form for rows whose longest prefix fits 1024 * KPT blocks.  For the
// decode form (one row), pos0 is chosen so the row sees exactly nb blocks.
hipError_t launch_reg(const float *scores, int32_t n_q, int32_t ld_or_nb, int32_t pos0, int32_t k,
                      int32_t *blk, int32_t *n_sel, hipStream_t s, bool decode)
{
    int32_t ld = ld_or_nb, p0 = pos0, nb_max;
    if (decode) {
        nb_max = ld_or_nb;
        ld = nb_max;
        p0 = kBlockTokens * nb_max - 1;  // the row sees floor((p0 + 1) / 4) = nb blocks
    } else {
        nb_max = (pos0 + n_q) / kBlockTokens;
    }
    const dim3 grid((uint32_t)n_q), block(kRegThreads);
    if (nb_max <= kRegThreads * 16)
        hipLaunchKernelGGL((topk_reg_kernel<16>), grid, block, 0, s, scores, ld, p0, k, blk, n_sel);
    else if (nb_max <= kRegThreads * 32)
        hipLaunchKernelGGL((topk_reg_kernel<32>), grid, block, 0, s, scores, ld, p0, k, blk, n_sel);
    else
        hipLaunchKernelGGL((topk_reg_kernel<64>), grid, block, 0, s, scores, ld, p0, k, blk, n_sel);
    return hipGetLastError();
}

}  // namespace

int32_t topk_max_blocks() { return kMaxBlocks; }

hipError_t launch_topk_decode(const float *scores, int32_t nb, int32_t k, int32_t *blk,
                              int32_t *n_sel, CandLists cl, hipStream_t s)
{
    if (nb > kMaxBlocks)
        return hipErrorInvalidValue;
    if (nb <= k) {
        const int32_t grid = nb > 0 ? (nb + kThreads - 1) / kThreads : 1;
        hipLaunchKernelGGL(iota_kernel, dim3(grid), dim3(kThreads), 0, s, blk, nb, n_sel);
        return hipGetLastError();
    }
    int32_t nwg = 0;
    hipError_t e = launch_score_lists(scores, 1, nb, kBlockTokens * nb - 1, cl, &nwg, s);
    if (e != hipSuccess)
        return e;
    return launch_topk_lists(scores, nb, k, cl, nwg, blk, n_sel, s);
}

hipError_t launch_score_lists(const float *scores, int32_t rows, int32_t ld, int32_t pos0,
                              CandLists cl, int32_t *n_lists, hipStream_t s)
{
    const int32_t nb_max = (pos0 + rows) / kBlockTokens;
    if (rows < 1 || nb_max > kMaxBlocks)
        return hipErrorInvalidValue;
    const int32_t runs = (nb_max + 3) / 4;
    const int32_t nwg = runs < 1 ? 1 : (runs < kListWgs ? runs : kListWgs);
    hipLaunchKernelGGL(score_lists_kernel, dim3((uint32_t)nwg, (uint32_t)rows),
                       dim3(kListBuildThreads), 0, s, scores, ld, pos0, cl);
    *n_lists = nwg;
    return hipGetLastError();
}

hipError_t launch_topk_lists(const float *scores, int32_t nb, int32_t k, CandLists cl,
                             int32_t n_lists, int32_t *blk, int32_t *n_sel, hipStream_t s,
                             int32_t scan_rpw, int32_t n_scan)
{
    if (nb > kMaxBlocks || n_lists < 1 || n_lists > kListWgs)
        return hipErrorInvalidValue;
    if (nb <= k) {
        const int32_t grid = nb > 0 ? (nb + kThreads - 1) / kThreads : 1;
        hipLaunchKernelGGL(iota_kernel, dim3(grid), dim3(kThreads), 0, s, blk, nb, n_sel);
        return hipGetLastError();
    }
    // the rows behind the lists: the decode scan's layout, or launch_score_lists'
    // (list w owns runs of 4 rows at stride 4 n_lists: row groups of one row)
    const ListLayout lay = scan_rpw > 0 ? ListLayout{1, n_lists - 1, scan_rpw, (uint32_t)n_scan}
                                        : ListLayout{0, n_lists, 1, (uint32_t)nb};
    hipLaunchKernelGGL(topk_lists_kernel, dim3(1), dim3(kSelThreads), 0, s, scores, nb, k, cl,
                       n_lists, lay, blk, n_sel);
    return hipGetLastError();
}

hipError_t launch_topk_rows(const float *scores, int32_t n_q, int32_t ld, int32_t pos0, int32_t k,
                            int32_t *blk, int32_t *n_sel, hipStream_t s)
{
    const int32_t nb_max = (pos0 + n_q) / kBlockTokens;
    if (nb_max > kMaxBlocks)
        return hipErrorInvalidValue;
    if (nb_max <= kRegThreads * 64)
        return launch_reg(scores, n_q, ld, pos0, k, blk, n_sel, s, false);
    const size_t lds = sizeof(uint64_t) * kCandCap + sizeof(uint32_t) * kHistBins +
                       sizeof(uint32_t) * (size_t)((nb_max + 31) / 32);
    static std::once_flag once;
    std::call_once(once, [] {
        (void)hipFuncSetAttribute((const void *)topk_rows_kernel,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    });
    hipLaunchKernelGGL(topk_rows_kernel, dim3(n_q), dim3(kThreads), lds, s, scores, ld, pos0, k,
                       blk, n_sel);
    return hipGetLastError();
}

}  // namespace qsa
