// Top-k over block scores in the block domain (Qiita part 10,
// "QSAとQSA indexerについて": keep the highest-scoring blocks; "block-domain
// top-k（COMMON-006）実装は見送り": select pools, then expand only the chosen ones).
//
// Selection is a radix select on the order-preserving 32-bit key of each fp32
// score (score_key), made exact and deterministic:
//   1. a 4096-bin histogram of the top 12 key bits finds the bin B that holds
//      the k-th largest key; every block in a higher bin is chosen;
//   2. the blocks of bin B are candidates; 8/8/4-bit digit passes over them find
//      the exact k-th key T, then passes over block ids find the largest id I
//      still chosen among keys equal to T (equal scores go to lower ids);
//   3. chosen = key > T, or key == T and id <= I.  The chosen ids are set in an
//      LDS bitmap and compacted in id order, so the output is ascending.
// Atomics only count (histograms, list slots); the result never depends on
// their order.
//
// Two forms:
//   * rows: one work group per score row (prefill chunks);
//   * decode: one long row spread over G work groups in two launches
//     (histogram, then candidate extraction); the last work group to finish each
//     launch (an atomic ticket) does the serial part, and restores the
//     workspace words it used to zero.
#include <mutex>

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr int kCandCap = 4096;
constexpr int kMaxBlocks = 1 << 19;  // bitmap of 64 KiB in LDS


template <int NT>
struct Scratch {
    uint32_t tmp[NT];
    uint32_t res[4];
    uint32_t cnt;
    uint32_t cnt2;
    uint32_t flag;
};

// Over NBINS (4096 or 256) LDS bins, finds the bin where the count taken from
// the top reaches need (need >= 1).  res[0] = bin (0xffffffff if the total is
// below need), res[1] = count in the bins above it, res[2] = total, res[3] =
// count in the bin.  All NT
// threads call it; wave 0 does the work: lane l sums bins [l*per, (l+1)*per), a
// wave scan finds the lane where the count from the top crosses need, and a
// second wave scan over that lane's bins finds the bin.  hist is 16-byte aligned;
// NBINS is 256 or 4096.
template <int NT, int NBINS>
__device__ void find_from_top(const uint32_t *hist, uint32_t need, Scratch<NT> &S)
{
    static_assert(NBINS == 256 || NBINS == 4096, "bins");
    if (threadIdx.x < kWave) {
        // opaque copy of the lane: keeps the compiler from hoisting the 64 bin
        // addresses out of a caller's loop (they would stay live and spill)
        uint32_t lane = threadIdx.x;
        asm volatile("" : "+v"(lane));
        constexpr int per = NBINS / kWave;  // 4 or 64
        uint32_t c = 0;
        if (per == 4) {
            const uint4 v = *(const uint4 *)(hist + lane * 4);
            c = v.x + v.y + v.z + v.w;
        } else {
            // rotated order: at step i the 64 lanes read 64 different banks; all
            // loads are issued before the sum
            uint32_t h[per];
#pragma unroll
            for (int i = 0; i < per; i++)
                h[i] = hist[lane * per + ((i + (int)lane) & (per - 1))];
#pragma unroll
            for (int i = 0; i < per; i++)
                c += h[i];
        }
        const uint32_t incl = wave_incl_scan(c);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
        const uint32_t above = total - incl;  // in the bins of the lanes above
        if (need > total) {
            if (lane == 0) {
                S.res[0] = 0xffffffffu;
                S.res[2] = total;
            }
        } else {
            const uint64_t m = __ballot(above < need && need <= above + c);
            const int L = __ffsll((unsigned long long)m) - 1;
            const uint32_t aboveL = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
            const uint32_t h = ((int)lane < per) ? hist[L * per + (int)lane] : 0u;
            const uint32_t incl2 = wave_incl_scan(h);
            const uint32_t tot2 = (uint32_t)__builtin_amdgcn_readlane((int)incl2, kWave - 1);
            const uint32_t above2 = aboveL + (tot2 - incl2);
            if ((int)lane < per && above2 < need && need <= above2 + h) {
                S.res[0] = (uint32_t)(L * per + (int)lane);
                S.res[1] = above2;
                S.res[3] = h;
            }
            if (lane == 0)
                S.res[2] = total;
        }
    }
    __syncthreads();
}

// As find_from_top for NBINS = 4 * NT, with every thread taking part: thread t
// owns bins 4t..4t+3, a work-group prefix sum (wave scans, then the NT/64 wave
// totals through wtot) gives the count in the bins of higher threads, and the
// one thread whose bins reach `need` finds the bin.  Sets res[0..3] as
// find_from_top does.
template <int NT>
__device__ void find_from_top_wg(const uint32_t *hist, uint32_t need, Scratch<NT> &S,
                                 uint32_t *wtot)
{
    constexpr int NW = NT / kWave;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const uint4 v = ((const uint4 *)hist)[t];
    const uint32_t c = v.x + v.y + v.z + v.w;
    const uint32_t incl = wave_incl_scan(c);
    if (lane == kWave - 1)
        wtot[w] = incl;
    __syncthreads();
    uint32_t total = 0, above = 0;
#pragma unroll
    for (int i = 0; i < NW; i++) {
        const uint32_t x = wtot[i];
        total += x;
        above += i > w ? x : 0u;
    }
    above += wtot[w] - incl;  // higher lanes of this wave
    if (need > total) {
        if (t == 0) {
            S.res[0] = 0xffffffffu;
            S.res[2] = total;
        }
    } else if (above < need && need <= above + c) {
        const uint32_t h[4] = {v.w, v.z, v.y, v.x};  // bins 4t+3 .. 4t
        uint32_t a = above;
        int i = 0;
        while (a + h[i] < need) {
            a += h[i];
            i++;
        }
        S.res[0] = (uint32_t)(4 * t + 3 - i);
        S.res[1] = a;
        S.res[2] = total;
        S.res[3] = h[i];
    }
    __syncthreads();
}

// Candidate sources: each calls f(key, id) for every block of bin B.
template <int NT>
struct LdsCands {
    const uint64_t *c;
    uint32_t n;
    template <class F>
    __device__ void each(F f) const
    {
        for (uint32_t i = threadIdx.x; i < n; i += NT)
            f((uint32_t)(c[i] >> 32), (uint32_t)c[i]);
    }
};

template <int NT>
struct GlobalCands {
    const uint64_t *c;
    uint32_t n;
    template <class F>
    __device__ void each(F f) const
    {
        for (uint32_t i = threadIdx.x; i < n; i += NT) {
            const uint64_t v = c[i];
            f((uint32_t)(v >> 32), (uint32_t)v);
        }
    }
};

template <int NT>
struct RowCands {
    const float *row;
    uint32_t nb;
    uint32_t bin;
    template <class F>
    __device__ void each(F f) const
    {
        for (uint32_t i = threadIdx.x; i < nb; i += NT) {
            const uint32_t key = score_key(row[i]);
            if ((key >> (32 - kHistBits)) == bin)
                f(key, i);
        }
    }
};

// Exact threshold among the candidates: on return S.res[0] = T (key), S.res[1]
// = I (largest chosen id among keys equal to T).
template <int NT, class Src>
__device__ void resolve(const Src &src, uint32_t bin, uint32_t need, uint32_t nb, uint32_t *h256,
                        Scratch<NT> &S)
{
    uint32_t prefix = bin;
    int shift = 32 - kHistBits;
    const int widths[3] = {8, 8, 4};
    uint32_t last_count = 0;
    for (int p = 0; p < 3; p++) {
        const int w = widths[p];
        shift -= w;
        if (threadIdx.x < 256)
            h256[threadIdx.x] = 0;
        __syncthreads();
        const uint32_t pf = prefix, sh = (uint32_t)shift, mask = (1u << w) - 1u;
        src.each([&](uint32_t key, uint32_t) {
            if ((key >> (sh + w)) == pf)
                atomicAdd(&h256[(key >> sh) & mask], 1u);
        });
        __syncthreads();
        find_from_top<NT, 256>(h256, need, S);
        const uint32_t d = S.res[0];
        need -= S.res[1];
        last_count = h256[d];
        prefix = (prefix << w) | d;
        __syncthreads();
    }
    const uint32_t T = prefix;
    uint32_t I = 0xffffffffu;
    if (need < last_count) {
        // the `need` lowest ids among keys equal to T
        const int nbits = 32 - __clz((int)(nb - 1));
        const int top = ((nbits + 7) / 8) * 8;
        uint32_t ip = 0;
        for (int sh = top - 8; sh >= 0; sh -= 8) {
            if (threadIdx.x < 256)
                h256[threadIdx.x] = 0;
            __syncthreads();
            const uint32_t ipf = ip, s2 = (uint32_t)sh;
            src.each([&](uint32_t key, uint32_t id) {
                if (key == T && (s2 + 8 >= 32 || (id >> (s2 + 8)) == ipf))
                    atomicAdd(&h256[255u - ((id >> s2) & 255u)], 1u);
            });
            __syncthreads();
            find_from_top<NT, 256>(h256, need, S);
            const uint32_t d = 255u - S.res[0];
            need -= S.res[1];
            ip = (ip << 8) | d;
            __syncthreads();
        }
        I = ip;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        S.res[0] = T;
        S.res[1] = I;
    }
    __syncthreads();
}

// Exclusive prefix sum over the work group; returns this thread's offset.
template <int NT>
__device__ uint32_t wg_exclusive_scan(uint32_t v, Scratch<NT> &S)
{
    constexpr int NW = NT / kWave;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const uint32_t s = wave_incl_scan(v);
    __syncthreads();
    if (lane == kWave - 1)
        S.tmp[w] = s;
    __syncthreads();
    const uint32_t wt = lane < NW ? S.tmp[lane] : 0u;
    const uint32_t ws = wave_incl_scan(wt);
    const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(ws - wt), w);  // waves below
    __syncthreads();
    return base + s - v;
}

// Writes the ids of the set bits of bitmap[0 .. ceil(nb/32)) in ascending order;
// never more than cap of them.
template <int NT>
__device__ void compact_bitmap(const uint32_t *bitmap, uint32_t nb, int32_t *out, uint32_t cap,
                               Scratch<NT> &S)
{
    const uint32_t W = (nb + 31) / 32;
    const uint32_t per = (W + NT - 1) / NT;
    const uint32_t w0 = threadIdx.x * per;
    const uint32_t w1 = min(W, w0 + per);
    uint32_t c = 0;
    for (uint32_t w = w0; w < w1; w++)
        c += __popc(bitmap[w]);
    uint32_t pos = wg_exclusive_scan<NT>(c, S);
    for (uint32_t w = w0; w < w1; w++) {
        uint32_t m = bitmap[w];
        while (m) {
            const uint32_t b = (uint32_t)__ffs((int)m) - 1u;
            if (pos < cap)
                out[pos] = (int32_t)(w * 32 + b);
            pos++;
            m &= m - 1u;
        }
    }
}

__device__ void set_bit(uint32_t *bitmap, uint32_t id) { atomicOr(&bitmap[id >> 5], 1u << (id & 31)); }

template <int NT>
__device__ void zero_words(uint32_t *p, uint32_t n)
{
    for (uint32_t i = threadIdx.x; i < n; i += NT)
        p[i] = 0;
}

// ---------------------------------------------------------------- register form
// One 1024-thread work group per row; the row's keys stay in registers (KPT per
// thread, element (j, e) of thread t is id 4*(j*1024 + t) + e), so the scores are
// read once and nothing leaves the work group.  Used for rows of up to 1024*KPT
// blocks (65,536 at KPT = 64, i.e. contexts up to 262,147 tokens).
constexpr int kRegThreads = 1024;
constexpr int kListCap = 4096;  // keys in bins >= the lower bound, kept in LDS

template <int KPT>
__global__ __launch_bounds__(kRegThreads) void topk_reg_kernel(const float *__restrict__ scores,
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
    uint32_t kp[KPT / 2];
    const bool vec_ok = (((uintptr_t)row) & 15) == 0;
#pragma unroll
    for (int j = 0; j < V4; j++) {
        const uint32_t i0 = id_of(j, 0);
        uint32_t kk[4];
        if (vec_ok && i0 + 3 < nb) {
            const f32x4 v = *(const f32x4 *)(row + i0);
#pragma unroll
            for (int e = 0; e < 4; e++)
                kk[e] = score_key(v[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++)
                kk[e] = (i0 + e < nb) ? score_key(row[i0 + e]) : 0u;
        }
        kp[2 * j] = (kk[0] >> 16) | (kk[1] & 0xffff0000u);
        kp[2 * j + 1] = (kk[2] >> 16) | (kk[3] & 0xffff0000u);
        if ((j & 7) == 7)
            __builtin_amdgcn_sched_barrier(0);  // at most 8 row loads in flight per lane
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
        uint32_t incl = mine;  // inclusive scan over the wave
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t u = __shfl_up(incl, o, kWave);
            if ((t & (kWave - 1)) >= o)
                incl += u;
        }
        uint32_t base = 0;
        if ((t & (kWave - 1)) == kWave - 1 && incl)
            base = atomicAdd(&S.cnt, incl);
        base = __shfl(base, kWave - 1, kWave) + incl - mine;
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
// Generic exact selection of one row straight from global memory (any nb up to
// kMaxBlocks): histogram pass, candidates of the threshold bin to LDS (or
// re-read from L2 when there are too many), digit passes, bitmap compaction.
template <int NT>
__device__ void select_row_global(const float *row, uint32_t nb, int32_t k, int32_t *outr,
                                  uint32_t *hist, uint64_t *cand, uint32_t *bitmap,
                                  Scratch<NT> &S)
{
    zero_words<NT>(hist, kHistBins);
    if (threadIdx.x == 0)
        S.cnt = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nb; i += NT)
        atomicAdd(&hist[score_key(row[i]) >> (32 - kHistBits)], 1u);
    __syncthreads();
    find_from_top<NT, kHistBins>(hist, (uint32_t)k, S);
    const uint32_t B = S.res[0];
    const uint32_t need = (uint32_t)k - S.res[1];
    zero_words<NT>(bitmap, (nb + 31) / 32);
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nb; i += NT) {
        const uint32_t key = score_key(row[i]);
        const uint32_t bin = key >> (32 - kHistBits);
        if (bin > B) {
            set_bit(bitmap, i);
        } else if (bin == B) {
            const uint32_t slot = atomicAdd(&S.cnt, 1u);
            if (slot < kCandCap)
                cand[slot] = ((uint64_t)key << 32) | i;
        }
    }
    __syncthreads();
    const uint32_t c = S.cnt;
    uint32_t *h256 = hist;  // the 12-bit histogram is no longer needed
    if (c <= (uint32_t)kCandCap) {
        LdsCands<NT> src{cand, c};
        resolve<NT>(src, B, need, nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    } else {
        RowCands<NT> src{row, nb, B};
        resolve<NT>(src, B, need, nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    }
    __syncthreads();
    compact_bitmap<NT>(bitmap, nb, outr, (uint32_t)k, S);
}

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

// ---------------------------------------------------------------- decode form
// One long row spread over many CUs, two launches that meet only at the kernel
// boundary.  Neither uses a fence or a global atomic: on this part a device-scope
// fence or a contended atomic costs more than the kernel boundary itself.
//   filter  work group g takes scores [1024 g, 1024 g + 1024) and the same
//           deterministic sample of the row (every stride-th score), finds the
//           bin of the r-th largest sampled key (r about 3x the sample's expected
//           share of k) and writes its own keys in that bin or above, in id
//           order, to region g of ws.cand, and their count to ws.rcnt[g];
//   final   one work group reads all region counts and the first `head` entries
//           of every region in one round (regions longer than that in a second
//           round), so it holds the list in ascending id order.  It selects
//           exactly: a 12-bit histogram gives the threshold bin, an 8-bit digit
//           histogram splits it, rank counting settles the threshold digit (or
//           further digit passes, when it is crowded), and a prefix sum over the
//           list writes the chosen ids in ascending order.
//           If the list holds fewer than k keys (the sample misled the bound) or
//           more than fit in LDS (flat scores), it selects from the whole row.
constexpr int kFilterPerWg = 1024;  // scores per filter work group (4 per thread)
constexpr int kSample = 1024;       // sampled scores (4 per thread)
constexpr int kFinalThreads = 1024;
constexpr int kListMax = 4096;      // list entries the final step keeps in LDS
constexpr int kMaxRegions = kMaxBlocks / kFilterPerWg;
static_assert(kMaxRegions % kWave == 0, "whole regions per lane of wave 0");
static_assert(kListMax == 4 * kFinalThreads, "four list entries per final thread");

__global__ __launch_bounds__(kThreads) void topk_filter_kernel(const float *__restrict__ scores,
                                                               int32_t nb, int32_t k, TopkWs ws,
                                                               uint32_t head)
{
    __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
    __shared__ Scratch<kThreads> S;
    const int t = threadIdx.x;
    const uint32_t stride = max(64u, ((uint32_t)nb + kSample - 1) / kSample);
    const uint32_t ns = ((uint32_t)nb + stride - 1) / stride;
    // this work group's own 4 scores per thread and 4 sampled scores per thread
    const int32_t i0 = blockIdx.x * kFilterPerWg + 4 * t;
    float own[4], smp[4];
    if (i0 + 3 < nb && ((((uintptr_t)scores) & 15) == 0)) {
        const f32x4 v = *(const f32x4 *)(scores + i0);
        own[0] = v[0], own[1] = v[1], own[2] = v[2], own[3] = v[3];
    } else {
#pragma unroll
        for (int e = 0; e < 4; e++)
            own[e] = (i0 + e < nb) ? scores[i0 + e] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const uint32_t j = (uint32_t)(t + kThreads * e);
        smp[e] = (j < ns) ? scores[(size_t)j * stride] : 0.f;
    }
    zero_words<kThreads>(hist, kHistBins);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; e++)
        if ((uint32_t)(t + kThreads * e) < ns)
            atomicAdd(&hist[score_key(smp[e]) >> (32 - kHistBits)], 1u);
    __syncthreads();
    // r-th largest sampled key: about 3x the sample's expected count of top-k
    // keys, so the bound keeps ~3k keys of the row; exactness is checked later
    const uint32_t want = (uint32_t)(((uint64_t)3 * k * ns + nb - 1) / nb) + 8;
    find_from_top<kThreads, kHistBins>(hist, min(want, ns), S);
    const uint32_t Lb = (S.res[0] == 0xffffffffu) ? 0u : S.res[0];
    uint32_t key[4], mine = 0;
    bool keep[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        key[e] = score_key(own[e]);
        keep[e] = i0 + e < nb && (key[e] >> (32 - kHistBits)) >= Lb;
        mine += keep[e] ? 1u : 0u;
    }
    uint32_t off = wg_exclusive_scan<kThreads>(mine, S);
    uint64_t *region = ws.cand + (size_t)blockIdx.x * kFilterPerWg;
#pragma unroll
    for (int e = 0; e < 4; e++)
        if (keep[e])
            region[off++] = ((uint64_t)key[e] << 32) | (uint32_t)(i0 + e);
    if (t == kThreads - 1) {
        ws.rcnt[blockIdx.x] = off;  // exclusive offset + own count = region total
        S.res[3] = off;
    }
    __syncthreads();
    // pad the region up to the head the final step reads in its first round, so
    // that read only touches lines written by this launch
    for (uint32_t i = S.res[3] + t; i < head; i += kThreads)
        region[i] = 0ull;
}

// head: entries read from every region in the first round (a power of two,
// head * regions <= kListMax, head <= kFilterPerWg).
__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(const float *__restrict__ scores,
                                                                   int32_t nb, int32_t k,
                                                                   int32_t *__restrict__ blk,
                                                                   int32_t *__restrict__ n_sel,
                                                                   TopkWs ws, int32_t head_log2)
{
    constexpr int NT = kFinalThreads;
    __shared__ uint64_t cand[kListMax];
    __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
    __shared__ uint32_t bitmap[kMaxBlocks / 32];
    __shared__ uint32_t rbase[kMaxRegions], rlen[kMaxRegions];
    __shared__ __attribute__((aligned(16))) uint8_t sel[kListMax];
    __shared__ __attribute__((aligned(16))) uint32_t h256[256];
    __shared__ Scratch<NT> S;
    const int t = threadIdx.x;
    const int32_t G = (nb + kFilterPerWg - 1) / kFilterPerWg;
    const uint32_t head = 1u << head_log2;

    // one round of loads: every region count and the head of every region
    uint64_t e[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t sl = (uint32_t)(t + NT * j);
        const uint32_t g = sl >> head_log2, i = sl & (head - 1u);
        e[j] = (g < (uint32_t)G) ? ws.cand[(size_t)g * kFilterPerWg + i] : 0ull;
    }
    // wave 0: the region counts (8 consecutive regions per lane) and their
    // exclusive prefix, i.e. where each region starts in the list
    constexpr int RPL = kMaxRegions / kWave;
    if (t < kWave) {
        uint32_t rc[RPL], tot = 0;
#pragma unroll
        for (int q = 0; q < RPL; q++) {
            const int32_t g = RPL * t + q;
            rc[q] = (g < G) ? ws.rcnt[g] : 0u;
            tot += rc[q];
        }
        const uint32_t incl = wave_incl_scan(tot);
        uint32_t b = incl - tot;
        bool over = false;
#pragma unroll
        for (int q = 0; q < RPL; q++) {
            const int32_t g = RPL * t + q;
            if (g < G) {
                rbase[g] = b;
                rlen[g] = rc[q];
                over |= rc[q] > head;  // longer than its head: a second round
            }
            b += rc[q];
        }
        const uint64_t anyover = __ballot(over);
        if (t == 0) {
            S.cnt = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
            S.flag = anyover ? 1u : 0u;
        }
    }
    ((uint32_t *)sel)[t] = 0u;
    __syncthreads();
    const uint32_t c = S.cnt;
    if (c < (uint32_t)k || c > (uint32_t)kListMax) {
        // the list cannot be used: select from the whole row
        select_row_global<NT>(scores, (uint32_t)nb, k, blk, hist, cand, bitmap, S);
    } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t sl = (uint32_t)(t + NT * j);
            const uint32_t g = sl >> head_log2, i = sl & (head - 1u);
            if (g < (uint32_t)G && i < rlen[g])
                cand[rbase[g] + i] = e[j];
        }
        if (S.flag) {
            // rare: the tails of long regions, one region at a time
            for (int32_t g = 0; g < G; g++) {
                const uint32_t n = rlen[g];
                for (uint32_t i = head + t; i < n; i += NT)
                    cand[rbase[g] + i] = ws.cand[(size_t)g * kFilterPerWg + i];
            }
        }
        zero_words<NT>(hist, kHistBins);
        if (t < 256)
            h256[t] = 0;
        if (t == 0)
            S.cnt2 = 0;
        __syncthreads();
        for (uint32_t i = t; i < c; i += NT)
            atomicAdd(&hist[(uint32_t)(cand[i] >> (64 - kHistBits))], 1u);
        __syncthreads();
        find_from_top<NT, kHistBins>(hist, (uint32_t)k, S);
        const uint32_t B = S.res[0];
        const uint32_t need = (uint32_t)k - S.res[1];
        for (uint32_t i = t; i < c; i += NT) {
            const uint64_t v = cand[i];
            const uint32_t bin = (uint32_t)(v >> (64 - kHistBits));
            if (bin > B)
                sel[i] = 1;
            else if (bin == B)
                atomicAdd(&h256[(uint32_t)(v >> 44) & 255u], 1u);
        }
        __syncthreads();
        find_from_top<NT, 256>(h256, need, S);
        const uint32_t d = S.res[0];
        const uint32_t need2 = need - S.res[1];
        const uint32_t cd = h256[d];
        uint32_t *dl = hist;  // list indices of digit d
        for (uint32_t i = t; i < c; i += NT) {
            const uint64_t v = cand[i];
            if ((uint32_t)(v >> (64 - kHistBits)) != B)
                continue;
            const uint32_t dig = (uint32_t)(v >> 44) & 255u;
            if (dig > d)
                sel[i] = 1;
            else if (dig == d && cd <= (uint32_t)kWave)
                dl[atomicAdd(&S.cnt2, 1u)] = i;
        }
        __syncthreads();
        if (cd <= (uint32_t)kWave) {
            if ((uint32_t)t < cd) {
                const uint32_t me = dl[t];
                const uint64_t v = cand[me];
                const uint32_t mk = (uint32_t)(v >> 32), mid = (uint32_t)v;
                uint32_t before = 0;
                for (uint32_t j = 0; j < cd; j++) {
                    const uint64_t o = cand[dl[j]];
                    const uint32_t ok = (uint32_t)(o >> 32), oid = (uint32_t)o;
                    before += (ok > mk || (ok == mk && oid < mid)) ? 1u : 0u;
                }
                if (before < need2)
                    sel[me] = 1;
            }
        } else {
            LdsCands<NT> all{cand, c};
            resolve<NT>(all, B, need, (uint32_t)nb, h256, S);
            const uint32_t T = S.res[0], I = S.res[1];
            for (uint32_t i = t; i < c; i += NT) {
                const uint64_t v = cand[i];
                const uint32_t kk = (uint32_t)(v >> 32), id = (uint32_t)v;
                if ((kk >> (32 - kHistBits)) == B && (kk > T || (kk == T && id <= I)))
                    sel[i] = 1;
            }
        }
        __syncthreads();
        // chosen ids in list order = ascending ids; thread t owns entries 4t..4t+3
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < 4; j++)
            cnt += (4u * t + j < c) ? sel[4 * t + j] : 0u;
        uint32_t pos = wg_exclusive_scan<NT>(cnt, S);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t i = 4u * t + j;
            if (i < c && sel[i]) {
                if (pos < (uint32_t)k)
                    blk[pos] = (int32_t)(uint32_t)cand[i];
                pos++;
            }
        }
    }
    if (t == 0)
        n_sel[0] = k;
}

// ---------------------------------------------------------------- list form
// The decode step's scan leaves, per work group w, its kListLen best rank keys
// (in any order, 0 for an empty slot) and its row count.  One 1024-thread work group, thread w holding
// list w in registers:
//   1. selection of R*, the k-th largest rank key of the lists: 4096-bucket
//      histograms over the range of the live score keys (the whole range of the
//      lists' keys first, then the chosen bucket; equal-width buckets over the
//      actual range keep the LDS atomics spread out, where fixed float-bit
//      digits would pile the candidates into a few bins), then digits of the
//      block id when one key is shared by many entries, until at most 64
//      entries are live; those are ranked by counting.  Rank keys are distinct
//      (ids are), so R* is exact and the chosen set is {R >= R*};
//   2. if a list is full (its work group scored more than kListLen rows) and
//      its smallest key is >= R* (checked on the per-wave maxima of those
//      smallest keys, by the wave that finds R*), rows of that work group missing from the list
//      could outrank R*: the whole score row is selected from instead
//      (select_row_global).  Otherwise every row outside the lists ranks below
//      the smallest key of its own list, hence below R*, and the lists hold the
//      top-k exactly;
//   3. chosen ids go into an LDS bitmap, compacted in ascending id order.
constexpr int kSmallRank = 64;  // keys ranked by counting (one per lane of wave 0)

__global__ __launch_bounds__(kFinalThreads) void topk_lists_kernel(const float *__restrict__ scores,
                                                                   int32_t nb, int32_t k,
                                                                   CandLists cl, int32_t W,
                                                                   int32_t *__restrict__ blk,
                                                                   int32_t *__restrict__ n_sel)
{
    constexpr int NT = kFinalThreads;
    static_assert(kListWgs <= NT, "one list per thread");
    __shared__ uint32_t bitmap[kMaxBlocks / 32];
    __shared__ __attribute__((aligned(16))) uint32_t hist[2][kHistBins];
    __shared__ uint64_t cand[kCandCap];
    __shared__ Scratch<NT> S;
    __shared__ uint32_t wtot[NT / kWave];
    __shared__ uint64_t wlast[NT / kWave];
    __shared__ uint32_t wkey[2][NT / kWave];
    __shared__ uint64_t rstar;
    __shared__ uint32_t hidden;
    const int t = threadIdx.x;

    // one round of loads: this thread's list and row count
    uint64_t R[kListLen];
    uint32_t nrows = 0;
    if (t < W) {
        const uint4 *src = (const uint4 *)(cl.list + (int64_t)t * kListLen);
#pragma unroll
        for (int j = 0; j < kListLen / 2; j++) {
            const uint4 v = src[j];
            R[2 * j] = ((uint64_t)v.y << 32) | v.x;
            R[2 * j + 1] = ((uint64_t)v.w << 32) | v.z;
        }
        nrows = cl.rows[t];
    } else {
#pragma unroll
        for (int j = 0; j < kListLen; j++)
            R[j] = 0ull;
    }
    // while they are in flight: clear both histograms and the bitmap
    ((uint4 *)hist[0])[t] = uint4{0, 0, 0, 0};
    ((uint4 *)hist[1])[t] = uint4{0, 0, 0, 0};
    zero_words<NT>(bitmap, ((uint32_t)nb + 31) / 32);
    if (t == 0)
        S.cnt = 0;
    // per wave: the smallest and largest score key of the nonempty entries, and
    // the largest smallest entry of a full list (for step 2)
    {
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        uint64_t last = ~0ull;
#pragma unroll
        for (int j = 0; j < kListLen; j++) {
            const uint32_t key = (uint32_t)(R[j] >> 32);
            if (R[j] != 0ull) {
                kmin = min(kmin, key);
                kmax = max(kmax, key);
            }
            last = R[j] < last ? R[j] : last;
        }
        if (!(t < W && nrows > (uint32_t)kListLen))
            last = 0ull;
        last = wave_max_u64(last);
        kmin = wave_min_u32(kmin);
        kmax = wave_max_u32(kmax);
        if ((t & (kWave - 1)) == 0) {
            wlast[t / kWave] = last;
            wkey[0][t / kWave] = kmin;
            wkey[1][t / kWave] = kmax;
        }
    }
    __syncthreads();

    // 1. select R*.  Key passes: the live keys [lo, lo + span] go into 4096
    // equal buckets ((key - lo) >> s); the bucket holding the need-th key from
    // the top becomes the new range, until one key is left or few entries.  If
    // that key is shared by many entries, id passes follow: the id bits 18..0
    // (bits 31..19 of ~id are 1 for every id below kMaxBlocks = 2^19) in 8, 8
    // and 3 bits, with (imask, ival) the low-word bits fixed so far.
    static_assert(kMaxBlocks == 1 << 19, "id digits cover 19 bits");
    uint32_t lo = 0xffffffffu, hi_key = 0u;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) {
        lo = min(lo, wkey[0][i]);
        hi_key = max(hi_key, wkey[1][i]);
    }
    uint32_t span = hi_key - lo;
    uint32_t imask = 0u, ival = 0u;
    auto live = [&](uint64_t r) {
        const uint32_t key = (uint32_t)(r >> 32);
        return r != 0ull && key >= lo && key - lo <= span && ((uint32_t)r & imask) == ival;
    };
    uint32_t need = (uint32_t)k, cnt = 0;
    bool ok = hi_key >= lo;  // some entry at all
    int p = 0;
    while (ok) {
        const int s = span >= (uint32_t)kHistBins ? 32 - __clz((int)span) - kHistBits : 0;
        uint32_t *h = hist[p & 1];
#pragma unroll
        for (int j = 0; j < kListLen; j++)
            if (live(R[j]))
                atomicAdd(&h[((uint32_t)(R[j] >> 32) - lo) >> s], 1u);
        __syncthreads();
        find_from_top_wg<NT>(h, need, S, wtot);
        const uint32_t d = S.res[0];
        if (d == 0xffffffffu) {  // fewer than k keys in the lists
            ok = false;
            break;
        }
        need -= S.res[1];
        cnt = S.res[3];
        // nobody reads h again in this pass; the next pass uses the other one
        ((uint4 *)h)[t] = uint4{0, 0, 0, 0};
        p++;
        lo += d << s;
        span = s == 0 ? 0u : min(span - (d << s), (1u << s) - 1u);
        if (span == 0 || cnt <= (uint32_t)kSmallRank)
            break;
    }
    if (ok && cnt > (uint32_t)kSmallRank) {
        // one key, many entries: id digits
        imask = 0xfff80000u;
        ival = 0xfff80000u;
        const int shifts[3] = {11, 3, 0};
        const int widths[3] = {8, 8, 3};
        for (int q = 0; q < 3; q++) {
            const int w = widths[q], sh = shifts[q];
            uint32_t *h = hist[p & 1];
#pragma unroll
            for (int j = 0; j < kListLen; j++)
                if (live(R[j]))
                    atomicAdd(&h[((uint32_t)R[j] >> sh) & ((1u << w) - 1u)], 1u);
            __syncthreads();
            find_from_top<NT, 256>(h, need, S);
            const uint32_t d = S.res[0];
            need -= S.res[1];
            cnt = S.res[3];
            if (t < 64)
                ((uint4 *)h)[t] = uint4{0, 0, 0, 0};
            p++;
            imask |= ((1u << w) - 1u) << sh;
            ival |= d << sh;
            if (cnt <= (uint32_t)kSmallRank)
                break;
        }
    }
    if (ok) {
        // the <= 64 live entries; R* is the one with `need - 1` of them above it
#pragma unroll
        for (int j = 0; j < kListLen; j++) {
            if (live(R[j])) {
                const uint32_t slot = atomicAdd(&S.cnt, 1u);
                if (slot < (uint32_t)kSmallRank)
                    cand[slot] = R[j];
            }
        }
        __syncthreads();
        if (t < kWave) {
            const uint64_t me = (uint32_t)t < cnt ? cand[t] : 0ull;
            uint32_t above = 0;
            for (uint32_t j = 0; j < cnt; j++)
                above += cand[j] > me ? 1u : 0u;
            const bool is_rs = (uint32_t)t < cnt && above == need - 1u;
            if (is_rs)
                rstar = me;
            // 2. a full list whose last key is chosen may hide chosen rows
            const uint64_t last = t < NT / kWave ? wlast[t] : 0ull;
            const uint64_t rs = __shfl(me, __ffsll((unsigned long long)__ballot(is_rs)) - 1, kWave);
            const bool hid = __ballot(last >= rs) != 0ull;
            if (t == 0)
                hidden = hid ? 1u : 0u;
        }
        __syncthreads();
        const uint64_t rs = rstar;
        ok = hidden == 0u;
        if (ok) {
#pragma unroll
            for (int j = 0; j < kListLen; j++)
                if (R[j] >= rs) {
                    const uint32_t id = rank_id(R[j]);
                    if (id < (uint32_t)nb)
                        set_bit(bitmap, id);
                }
            __syncthreads();
            compact_bitmap<NT>(bitmap, (uint32_t)nb, blk, (uint32_t)k, S);
        }
    }
    if (!ok) {
        __syncthreads();
        select_row_global<NT>(scores, (uint32_t)nb, k, blk, hist[0], cand, bitmap, S);
    }
    if (t == 0)
        n_sel[0] = k;
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
                              int32_t *n_sel, TopkWs ws, hipStream_t s)
{
    if (nb > kMaxBlocks)
        return hipErrorInvalidValue;
    if (nb <= k) {
        const int32_t grid = nb > 0 ? (nb + kThreads - 1) / kThreads : 1;
        hipLaunchKernelGGL(iota_kernel, dim3(grid), dim3(kThreads), 0, s, blk, nb, n_sel);
        return hipGetLastError();
    }
    const int32_t G = (nb + kFilterPerWg - 1) / kFilterPerWg;
    int32_t head_log2 = 0;  // largest power of two with head * G <= kListMax
    while (head_log2 < 10 && ((int64_t)2 << head_log2) * G <= kListMax)
        head_log2++;
    hipLaunchKernelGGL(topk_filter_kernel, dim3(G), dim3(kThreads), 0, s, scores, nb, k, ws,
                       1u << head_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(topk_final_kernel, dim3(1), dim3(kFinalThreads), 0, s, scores, nb, k, blk,
                       n_sel, ws, head_log2);
    return hipGetLastError();
}

hipError_t launch_topk_lists(const float *scores, int32_t nb, int32_t k, CandLists cl,
                             int32_t n_lists, int32_t *blk, int32_t *n_sel, hipStream_t s)
{
    if (nb > kMaxBlocks || n_lists < 1 || n_lists > kListWgs)
        return hipErrorInvalidValue;
    if (nb <= k) {
        const int32_t grid = nb > 0 ? (nb + kThreads - 1) / kThreads : 1;
        hipLaunchKernelGGL(iota_kernel, dim3(grid), dim3(kThreads), 0, s, blk, nb, n_sel);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(topk_lists_kernel, dim3(1), dim3(kFinalThreads), 0, s, scores, nb, k, cl,
                       n_lists, blk, n_sel);
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
