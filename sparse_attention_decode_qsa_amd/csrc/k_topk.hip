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
constexpr int kDecodePerWg = 512;

// control words in TopkWs::ctrl
enum : int { kTicketA = 0, kTicketB = 1, kSureCnt = 2, kCandCnt = 3, kBin = 4, kAbove = 5 };

template <int NT>
struct Scratch {
    uint32_t tmp[NT];
    uint32_t res[4];
    uint32_t cnt;
    uint32_t flag;
};

// Over nbins (4096 or 256) LDS bins, finds the bin where the count taken from
// the top reaches need.  res[0] = bin (0xffffffff if the total is below need),
// res[1] = count in the bins above it, res[2] = total.  All NT threads call it.
template <int NT>
__device__ void find_from_top(const uint32_t *hist, int nbins, uint32_t need, Scratch<NT> &S)
{
    // Per-thread bin sums, a suffix scan within each wave, then across the wave
    // totals; every step is a parallel shuffle scan (no single-lane LDS walks).
    constexpr int NW = NT / kWave;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int per = nbins >= NT ? nbins / NT : 1;
    const int nthr = nbins >= NT ? NT : nbins;
    uint32_t c = 0;
    if (t < nthr)
        for (int i = 0; i < per; i++)
            c += hist[t * per + i];
    // inclusive suffix sum over the lanes of this wave (bins of higher threads)
    uint32_t sfx = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t v = __shfl_down(sfx, o, kWave);
        if (lane + o < kWave)
            sfx += v;
    }
    if (lane == 0)
        S.tmp[w] = sfx;  // wave total
    __syncthreads();
    // count in the waves above this one
    uint32_t wt = lane < NW ? S.tmp[lane] : 0u;
    uint32_t wsfx = wt;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
        const uint32_t v = __shfl_down(wsfx, o, kWave);
        if (lane + o < NW)
            wsfx += v;
    }
    const uint32_t above_wave = __shfl(wsfx - wt, w, kWave) ;
    const uint32_t total = __shfl(wsfx, 0, kWave);
    const uint32_t above = above_wave + sfx - c;  // count in all higher threads
    __syncthreads();
    if (t == 0) {
        S.res[2] = total;
        if (need > total)
            S.res[0] = 0xffffffffu;  // not reached
    }
    if (above < need && need <= above + c) {
        uint32_t acc = above;
        int sel = t * per;
        for (int i = per - 1; i >= 0; i--) {
            const uint32_t h = hist[t * per + i];
            if (acc + h >= need) {
                sel = t * per + i;
                break;
            }
            acc += h;
        }
        S.res[0] = (uint32_t)sel;
        S.res[1] = acc;
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
        find_from_top<NT>(h256, 256, need, S);
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
            find_from_top<NT>(h256, 256, need, S);
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
    uint32_t s = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t u = __shfl_up(s, o, kWave);
        if (lane >= o)
            s += u;
    }
    __syncthreads();
    if (lane == kWave - 1)
        S.tmp[w] = s;
    __syncthreads();
    uint32_t wt = lane < NW ? S.tmp[lane] : 0u;
    uint32_t ws = wt;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
        const uint32_t u = __shfl_up(ws, o, kWave);
        if (lane >= o)
            ws += u;
    }
    const uint32_t base = __shfl(ws - wt, w, kWave);  // sum of the waves below
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

template <int KPT>
__global__ __launch_bounds__(kRegThreads) void topk_reg_kernel(const float *__restrict__ scores,
                                                               int32_t ld, int32_t pos0,
                                                               int32_t k, int32_t *__restrict__ blk,
                                                               int32_t *__restrict__ n_sel)
{
    constexpr int NT = kRegThreads;
    constexpr int V4 = KPT / 4;
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint64_t cand[kCandCap];
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
    // 1. a lower bound L on the threshold bin from every 16th key: the bin where
    //    the sample reaches about twice its expected share of k
    for (int i = t; i < kHistBins; i += NT)
        hist[i] = 0;
    if (t == 0)
        S.cnt = 0;
    __syncthreads();
    {
        const int tt = fresh_t();
#pragma unroll
        for (int j = 0; j < KPT; j += 16)
            if ((uint32_t)(4 * ((j / 4) * NT + tt)) < nb)
                atomicAdd(&hist[bin_of(j)], 1u);
    }
    __syncthreads();
    find_from_top<NT>(hist, kHistBins, (uint32_t)(k / 8 + 16), S);
    uint32_t L = S.res[0] == 0xffffffffu ? 0u : S.res[0];
    __syncthreads();
    // 2. exact histogram of the keys in bins >= L; if they are fewer than k, the
    //    bound was too high: redo it over every key
    for (int pass = 0; pass < 2; pass++) {
        // opaque keys: keeps the 64 bin values from being hoisted out of the
        // loop into registers of their own
#pragma unroll
        for (int j = 0; j < KPT / 2; j++)
            asm volatile("" : "+v"(kp[j]));
        for (int i = t; i < kHistBins; i += NT)
            hist[i] = 0;
        __syncthreads();
        const int tt = fresh_t();
#pragma unroll
        for (int j = 0; j < KPT; j++) {
            const uint32_t bin = bin_of(j);
            if ((uint32_t)(4 * ((j / 4) * NT + tt) + j % 4) < nb && bin >= L)
                atomicAdd(&hist[bin], 1u);
        }
        __syncthreads();
        find_from_top<NT>(hist, kHistBins, (uint32_t)k, S);
        if (S.res[0] != 0xffffffffu || L == 0)
            break;
        L = 0;
        __syncthreads();
    }
    const uint32_t B = S.res[0];
    const uint32_t need = (uint32_t)k - S.res[1];
    const uint32_t W = (nb + 31) / 32;
    for (uint32_t i = t; i < W; i += NT)
        bitmap[i] = 0;
    __syncthreads();
    // 3. bins above B are in; ids of bin B become candidates
    {
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
        // pad to a multiple of 16 with entries that never rank before anyone
        const uint32_t c16 = (c + 15) & ~15u;
        if ((uint32_t)t >= c && (uint32_t)t < c16)
            cand[t] = 0x00000000ffffffffull;
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
// Dynamic LDS: hist[4096] | cand[kCandCap] (u64) | bitmap[ceil(nb_max/32)]
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
    zero_words<kThreads>(hist, kHistBins);
    if (threadIdx.x == 0)
        S.cnt = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nb; i += kThreads)
        atomicAdd(&hist[score_key(row[i]) >> (32 - kHistBits)], 1u);
    __syncthreads();
    find_from_top<kThreads>(hist, kHistBins, (uint32_t)k, S);
    const uint32_t B = S.res[0];
    const uint32_t need = (uint32_t)k - S.res[1];
    zero_words<kThreads>(bitmap, (nb + 31) / 32);
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nb; i += kThreads) {
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
        LdsCands<kThreads> src{cand, c};
        resolve<kThreads>(src, B, need, nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    } else {
        RowCands<kThreads> src{row, nb, B};
        resolve<kThreads>(src, B, need, nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    }
    __syncthreads();
    compact_bitmap<kThreads>(bitmap, nb, outr, (uint32_t)k, S);
    if (threadIdx.x == 0)
        n_sel[r] = k;
}

// ---------------------------------------------------------------- decode form
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float *__restrict__ scores,
                                                             int32_t nb, int32_t k, TopkWs ws)
{
    __shared__ uint32_t hist[kHistBins];
    __shared__ Scratch<kThreads> S;
    zero_words<kThreads>(hist, kHistBins);
    __syncthreads();
    const int32_t lo = blockIdx.x * kDecodePerWg;
    const int32_t hi = min(nb, lo + kDecodePerWg);
    for (int32_t i = lo + threadIdx.x; i < hi; i += kThreads)
        atomicAdd(&hist[score_key(scores[i]) >> (32 - kHistBits)], 1u);
    __syncthreads();
    for (int i = threadIdx.x; i < kHistBins; i += kThreads)
        if (hist[i])
            atomicAdd(&ws.hist[i], hist[i]);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        S.flag = (atomicAdd(&ws.ctrl[kTicketA], 1u) == gridDim.x - 1) ? 1u : 0u;
    __syncthreads();
    if (!S.flag)
        return;
    __threadfence();
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) {
        hist[i] = __hip_atomic_load(&ws.hist[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ws.hist[i] = 0;
    }
    __syncthreads();
    find_from_top<kThreads>(hist, kHistBins, (uint32_t)k, S);
    if (threadIdx.x == 0) {
        ws.ctrl[kBin] = S.res[0];
        ws.ctrl[kAbove] = S.res[1];
        ws.ctrl[kTicketA] = 0;
    }
}

// Dynamic LDS: cand[kCandCap] (u64) | h256[256] | bitmap[ceil(nb/32)]
__global__ __launch_bounds__(kThreads) void topk_select_kernel(const float *__restrict__ scores,
                                                               int32_t nb, int32_t k,
                                                               int32_t *__restrict__ blk,
                                                               int32_t *__restrict__ n_sel,
                                                               TopkWs ws)
{
    extern __shared__ uint64_t lds64[];
    uint64_t *cand = lds64;
    uint32_t *h256 = (uint32_t *)(cand + kCandCap);
    uint32_t *bitmap = h256 + kThreads;
    __shared__ Scratch<kThreads> S;

    const uint32_t B = ws.ctrl[kBin];
    const int32_t lo = blockIdx.x * kDecodePerWg;
    const int32_t hi = min(nb, lo + kDecodePerWg);
    for (int32_t i0 = lo; i0 < hi; i0 += kThreads) {
        const int32_t i = i0 + threadIdx.x;
        uint32_t key = 0, bin = 0;
        if (i < hi) {
            key = score_key(scores[i]);
            bin = key >> (32 - kHistBits);
        }
        const bool sure = i < hi && bin > B;
        const bool maybe = i < hi && bin == B;
        const uint32_t s1 = wave_append_slot(sure, &ws.ctrl[kSureCnt]);
        if (sure)
            ws.sure[s1] = i;
        const uint32_t s2 = wave_append_slot(maybe, &ws.ctrl[kCandCnt]);
        if (maybe)
            ws.cand[s2] = ((uint64_t)key << 32) | (uint32_t)i;
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        S.flag = (atomicAdd(&ws.ctrl[kTicketB], 1u) == gridDim.x - 1) ? 1u : 0u;
    __syncthreads();
    if (!S.flag)
        return;
    __threadfence();

    const uint32_t above = __hip_atomic_load(&ws.ctrl[kAbove], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t n_sure = __hip_atomic_load(&ws.ctrl[kSureCnt], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t c = __hip_atomic_load(&ws.ctrl[kCandCnt], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t need = (uint32_t)k - above;
    zero_words<kThreads>(bitmap, ((uint32_t)nb + 31) / 32);
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < min(n_sure, (uint32_t)k); i += kThreads)
        set_bit(bitmap, min((uint32_t)ws.sure[i], (uint32_t)nb - 1u));
    if (c <= (uint32_t)kCandCap) {
        for (uint32_t i = threadIdx.x; i < c; i += kThreads)
            cand[i] = ws.cand[i];
        __syncthreads();
        LdsCands<kThreads> src{cand, c};
        resolve<kThreads>(src, B, need, (uint32_t)nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    } else {
        GlobalCands<kThreads> src{ws.cand, c};
        resolve<kThreads>(src, B, need, (uint32_t)nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    }
    __syncthreads();
    compact_bitmap<kThreads>(bitmap, (uint32_t)nb, blk, (uint32_t)k, S);
    if (threadIdx.x == 0) {
        n_sel[0] = k;
        ws.ctrl[kSureCnt] = 0;
        ws.ctrl[kCandCnt] = 0;
        ws.ctrl[kBin] = 0;
        ws.ctrl[kAbove] = 0;
        ws.ctrl[kTicketB] = 0;
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
                              int32_t *n_sel, TopkWs ws, hipStream_t s)
{
    if (nb > kMaxBlocks)
        return hipErrorInvalidValue;
    if (nb <= k) {
        const int32_t grid = nb > 0 ? (nb + kThreads - 1) / kThreads : 1;
        hipLaunchKernelGGL(iota_kernel, dim3(grid), dim3(kThreads), 0, s, blk, nb, n_sel);
        return hipGetLastError();
    }
    if (nb <= kRegThreads * 64)
        return launch_reg(scores, 1, nb, 0, k, blk, n_sel, s, true);
    const int32_t G = (nb + kDecodePerWg - 1) / kDecodePerWg;
    hipLaunchKernelGGL(topk_hist_kernel, dim3(G), dim3(kThreads), 0, s, scores, nb, k, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const size_t lds = sizeof(uint64_t) * kCandCap + sizeof(uint32_t) * kThreads +
                       sizeof(uint32_t) * (size_t)((nb + 31) / 32);
    static std::once_flag once;
    std::call_once(once, [] {
        (void)hipFuncSetAttribute((const void *)topk_select_kernel,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 112 * 1024);
    });
    hipLaunchKernelGGL(topk_select_kernel, dim3(G), dim3(kThreads), lds, s, scores, nb, k, blk,
                       n_sel, ws);
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
