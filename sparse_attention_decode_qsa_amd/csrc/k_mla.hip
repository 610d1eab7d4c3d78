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
constexpr uint16_t kNegInf = 0xFC00u;

__device__ __forceinline__ bool visible(const h16 *mask, int32_t n, int64_t j)
{
    if (j >= n)
        return false;
    const uint16_t bits = *(const uint16_t *)(mask + j);
    return bits != kNegInf;
}

__device__ uint32_t wave_count(const h16 *mask, int32_t n, int64_t base)
{
    uint32_t c = 0;
    for (int it = 0; it < kPerWave / kWave; it++) {
        const uint64_t m = __ballot(visible(mask, n, base + it * kWave + lane_id()));
        c += (uint32_t)__popcll(m);
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
    const uint32_t c = wave_count(mask, n, base);
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
    // wave's own count: one barrier publishes both
    uint32_t s = 0;
    for (uint32_t i = t; i < seg; i += kThreads)
        s += seg_cnt[i];
    const uint32_t ws = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(s), kWave - 1);
    const int64_t base = (int64_t)seg * kListSeg + (int64_t)wave * kPerWave;
    const uint32_t c = wave_count(mask, n, base);
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
    for (int it = 0; it < kPerWave / kWave; it++) {
        const int64_t j = base + it * kWave + lane_id();
        const bool v = visible(mask, n, j);
        const uint64_t m = __ballot(v);
        if (v) {
            const uint32_t slot = off + rank_in_mask(m);
            if (slot < (uint32_t)list_cap)
                list[slot] = (int32_t)j;
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
