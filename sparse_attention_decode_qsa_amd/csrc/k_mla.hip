// Mask -> ascending key list for the MLA-style list attention (devotd.net news on
// the llama.cpp CDNA sparse path, section 2: visible key positions are collected
// from the mask into a list; selection results are held as 64-bit masks, one
// bit per lane of a 64-lane wave, and counted to match).
//
// Two launches over segments of kListSeg positions:
//   count: per segment, one __ballot per 64 positions and __popcll of the mask;
//   write: each segment adds up the counts of the segments before it, then every
//          wave ranks its visible lanes with popcount(mask & lanes-below) and
//          writes the positions in order.  The last segment writes the total.
// Masks are always the full 64-bit ballot (no 32-lane assumption).
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPerWave = kListSeg / kWaves;  // 256 positions: 4 ballots per wave

// The load is unconditional (index clamped into the mask), so a wave's loads for
// several ballots are all in flight before the first ballot.
__device__ __forceinline__ bool visible(const h16 *mask, int32_t n, int64_t j)
{
    const uint16_t bits = *(const uint16_t *)(mask + (j < n ? j : (int64_t)n - 1));
    return j < n && bits != kF16NegInf;
}

// This wave's kPerWave positions from base: one ballot per 64 (all loads issued
// first); returns the visible count.
__device__ uint32_t wave_masks(const h16 *mask, int32_t n, int64_t base,
                               uint64_t (&mk)[kPerWave / kWave])
{
    bool v[kPerWave / kWave];
#pragma unroll
    for (int it = 0; it < kPerWave / kWave; it++)
        v[it] = visible(mask, n, base + it * kWave + lane_id());
    uint32_t c = 0;
#pragma unroll
    for (int it = 0; it < kPerWave / kWave; it++) {
        mk[it] = __ballot(v[it]);
        c += (uint32_t)__popcll(mk[it]);
    }
    return c;
}

__global__ __launch_bounds__(kThreads) void mask_count_kernel(const h16 *__restrict__ mask,
                                                              int32_t n,
                                                              uint32_t *__restrict__ seg_cnt)
{
    __shared__ uint32_t wc[kWaves];
    const int wave = threadIdx.x / kWave;
    const int64_t base = (int64_t)blockIdx.x * kListSeg + (int64_t)wave * kPerWave;
    uint64_t mk[kPerWave / kWave];
    const uint32_t c = wave_masks(mask, n, base, mk);
    if (lane_id() == 0)
        wc[wave] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int w = 0; w < kWaves; w++)
            s += wc[w];
        seg_cnt[blockIdx.x] = s;
    }
}

__global__ __launch_bounds__(kThreads) void mask_write_kernel(const h16 *__restrict__ mask,
                                                              int32_t n, int32_t list_cap,
                                                              const uint32_t *__restrict__ seg_cnt,
                                                              int32_t *__restrict__ list,
                                                              int32_t *__restrict__ n_list)
{
    __shared__ uint32_t pre[kWaves];
    __shared__ uint32_t wc[kWaves];
    const int t = threadIdx.x, wave = t / kWave;
    const uint32_t seg = blockIdx.x;
    // the counts of the segments before this one, summed per wave, and this
    // wave's ballots: one barrier publishes both.  The first count is loaded
    // unconditionally (index clamped) so that it is in flight with the mask loads
    const uint32_t first = seg_cnt[min((uint32_t)t, gridDim.x - 1)];
    const int64_t base = (int64_t)seg * kListSeg + (int64_t)wave * kPerWave;
    uint64_t mk[kPerWave / kWave];
    const uint32_t c = wave_masks(mask, n, base, mk);
    uint32_t s = (uint32_t)t < seg ? first : 0u;
    for (uint32_t i = t + kThreads; i < seg; i += kThreads)
        s += seg_cnt[i];
    const uint32_t ws = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(s), kWave - 1);
    if (lane_id() == 0) {
        pre[wave] = ws;
        wc[wave] = c;
    }
    __syncthreads();
    uint32_t seg_off = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++)
        seg_off += pre[w];
    uint32_t off = seg_off;
    for (int w = 0; w < wave; w++)
        off += wc[w];
#pragma unroll
    for (int it = 0; it < kPerWave / kWave; it++) {
        const uint64_t m = mk[it];  // the ballots of the count: the mask is read once
        if ((m >> lane_id()) & 1ull) {
            const uint32_t slot = off + rank_in_mask(m);
            if (slot < (uint32_t)list_cap)
                list[slot] = (int32_t)(base + it * kWave + lane_id());
        }
        off += (uint32_t)__popcll(m);
    }
    if (seg == gridDim.x - 1 && t == 0) {
        uint32_t total = seg_off;
        for (int w = 0; w < kWaves; w++)
            total += wc[w];
        *n_list = (int32_t)total;
    }
}

}  // namespace

hipError_t launch_mask_list(const h16 *mask, int32_t n, int32_t list_cap, uint32_t *seg_cnt,
                            int32_t *list, int32_t *n_list, hipStream_t s)
{
    const int32_t segs = (n + kListSeg - 1) / kListSeg;
    hipLaunchKernelGGL(mask_count_kernel, dim3(segs), dim3(kThreads), 0, s, mask, n, seg_cnt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(mask_write_kernel, dim3(segs), dim3(kThreads), 0, s, mask, n, list_cap,
                       seg_cnt, list, n_list);
    return hipGetLastError();
}

}  // namespace qsa
