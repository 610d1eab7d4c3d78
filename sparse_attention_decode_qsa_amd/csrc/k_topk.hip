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

struct Scratch {
    uint32_t tmp[kThreads];
    uint32_t res[4];
    uint32_t cnt;
    uint32_t flag;
};

// Over nbins (4096 or 256) LDS bins, finds the bin where the count taken from
// the top reaches need (1 <= need <= total).  res[0] = bin, res[1] = count in
// the bins above it.  All threads call it.
__device__ void find_from_top(const uint32_t *hist, int nbins, uint32_t need, Scratch &S)
{
    const int t = threadIdx.x;
    const int per = nbins / kThreads;
    uint32_t c = 0;
    for (int i = 0; i < per; i++)
        c += hist[t * per + i];
    S.tmp[t] = c;
    __syncthreads();
    if (t < kWave) {
        const uint32_t c4 = S.tmp[4 * t] + S.tmp[4 * t + 1] + S.tmp[4 * t + 2] + S.tmp[4 * t + 3];
        uint32_t s = c4;
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t v = __shfl_down(s, o, kWave);
            if (t + o < kWave)
                s += v;
        }
        const uint32_t above = s - c4;
        if (above < need && need <= s) {
            uint32_t acc = above;
            int thr = 4 * t;
            for (int j = 3; j >= 0; j--) {
                if (acc + S.tmp[4 * t + j] >= need) {
                    thr = 4 * t + j;
                    break;
                }
                acc += S.tmp[4 * t + j];
            }
            int sel = thr * per;
            for (int i = per - 1; i >= 0; i--) {
                const uint32_t h = hist[thr * per + i];
                if (acc + h >= need) {
                    sel = thr * per + i;
                    break;
                }
                acc += h;
            }
            S.res[0] = (uint32_t)sel;
            S.res[1] = acc;
        }
    }
    __syncthreads();
}

// Candidate sources: each calls f(key, id) for every block of bin B.
struct LdsCands {
    const uint64_t *c;
    uint32_t n;
    template <class F>
    __device__ void each(F f) const
    {
        for (uint32_t i = threadIdx.x; i < n; i += kThreads)
            f((uint32_t)(c[i] >> 32), (uint32_t)c[i]);
    }
};

struct GlobalCands {
    const uint64_t *c;
    uint32_t n;
    template <class F>
    __device__ void each(F f) const
    {
        for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
            const uint64_t v = c[i];
            f((uint32_t)(v >> 32), (uint32_t)v);
        }
    }
};

struct RowCands {
    const float *row;
    uint32_t nb;
    uint32_t bin;
    template <class F>
    __device__ void each(F f) const
    {
        for (uint32_t i = threadIdx.x; i < nb; i += kThreads) {
            const uint32_t key = score_key(row[i]);
            if ((key >> (32 - kHistBits)) == bin)
                f(key, i);
        }
    }
};

// Exact threshold among the candidates: on return S.res[0] = T (key), S.res[1]
// = I (largest chosen id among keys equal to T).
template <class Src>
__device__ void resolve(const Src &src, uint32_t bin, uint32_t need, uint32_t nb, uint32_t *h256,
                        Scratch &S)
{
    uint32_t prefix = bin;
    int shift = 32 - kHistBits;
    const int widths[3] = {8, 8, 4};
    uint32_t last_count = 0;
    for (int p = 0; p < 3; p++) {
        const int w = widths[p];
        shift -= w;
        h256[threadIdx.x] = 0;
        __syncthreads();
        const uint32_t pf = prefix, sh = (uint32_t)shift, mask = (1u << w) - 1u;
        src.each([&](uint32_t key, uint32_t) {
            if ((key >> (sh + w)) == pf)
                atomicAdd(&h256[(key >> sh) & mask], 1u);
        });
        __syncthreads();
        find_from_top(h256, kThreads, need, S);
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
            h256[threadIdx.x] = 0;
            __syncthreads();
            const uint32_t ipf = ip, s2 = (uint32_t)sh;
            src.each([&](uint32_t key, uint32_t id) {
                if (key == T && (s2 + 8 >= 32 || (id >> (s2 + 8)) == ipf))
                    atomicAdd(&h256[255u - ((id >> s2) & 255u)], 1u);
            });
            __syncthreads();
            find_from_top(h256, kThreads, need, S);
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
__device__ uint32_t wg_exclusive_scan(uint32_t v, Scratch &S)
{
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    uint32_t s = v;
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t u = __shfl_up(s, o, kWave);
        if (lane >= o)
            s += u;
    }
    __syncthreads();
    if (lane == kWave - 1)
        S.tmp[w] = s;
    __syncthreads();
    uint32_t base = 0;
    for (int i = 0; i < w; i++)
        base += S.tmp[i];
    __syncthreads();
    return base + s - v;
}

// Writes the ids of the set bits of bitmap[0 .. ceil(nb/32)) in ascending order;
// never more than cap of them.
__device__ void compact_bitmap(const uint32_t *bitmap, uint32_t nb, int32_t *out, uint32_t cap,
                               Scratch &S)
{
    const uint32_t W = (nb + 31) / 32;
    const uint32_t per = (W + kThreads - 1) / kThreads;
    const uint32_t w0 = threadIdx.x * per;
    const uint32_t w1 = min(W, w0 + per);
    uint32_t c = 0;
    for (uint32_t w = w0; w < w1; w++)
        c += __popc(bitmap[w]);
    uint32_t pos = wg_exclusive_scan(c, S);
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

__device__ void zero_words(uint32_t *p, uint32_t n)
{
    for (uint32_t i = threadIdx.x; i < n; i += kThreads)
        p[i] = 0;
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
    __shared__ Scratch S;

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
    zero_words(hist, kHistBins);
    if (threadIdx.x == 0)
        S.cnt = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nb; i += kThreads)
        atomicAdd(&hist[score_key(row[i]) >> (32 - kHistBits)], 1u);
    __syncthreads();
    find_from_top(hist, kHistBins, (uint32_t)k, S);
    const uint32_t B = S.res[0];
    const uint32_t need = (uint32_t)k - S.res[1];
    zero_words(bitmap, (nb + 31) / 32);
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
        LdsCands src{cand, c};
        resolve(src, B, need, nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    } else {
        RowCands src{row, nb, B};
        resolve(src, B, need, nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    }
    __syncthreads();
    compact_bitmap(bitmap, nb, outr, (uint32_t)k, S);
    if (threadIdx.x == 0)
        n_sel[r] = k;
}

// ---------------------------------------------------------------- decode form
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float *__restrict__ scores,
                                                             int32_t nb, int32_t k, TopkWs ws)
{
    __shared__ uint32_t hist[kHistBins];
    __shared__ Scratch S;
    zero_words(hist, kHistBins);
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
    find_from_top(hist, kHistBins, (uint32_t)k, S);
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
    __shared__ Scratch S;

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
    zero_words(bitmap, ((uint32_t)nb + 31) / 32);
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < min(n_sure, (uint32_t)k); i += kThreads)
        set_bit(bitmap, min((uint32_t)ws.sure[i], (uint32_t)nb - 1u));
    if (c <= (uint32_t)kCandCap) {
        for (uint32_t i = threadIdx.x; i < c; i += kThreads)
            cand[i] = ws.cand[i];
        __syncthreads();
        LdsCands src{cand, c};
        resolve(src, B, need, (uint32_t)nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    } else {
        GlobalCands src{ws.cand, c};
        resolve(src, B, need, (uint32_t)nb, h256, S);
        const uint32_t T = S.res[0], I = S.res[1];
        src.each([&](uint32_t key, uint32_t id) {
            if (key > T || (key == T && id <= I))
                set_bit(bitmap, id);
        });
    }
    __syncthreads();
    compact_bitmap(bitmap, (uint32_t)nb, blk, (uint32_t)k, S);
    if (threadIdx.x == 0) {
        n_sel[0] = k;
        ws.ctrl[kSureCnt] = 0;
        ws.ctrl[kCandCnt] = 0;
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
