// Pooled-key cache append: raw/K/V row copies plus the pooled summary of every
// 4-token block that completes (Qiita part 10, "QSAとQSA indexerについて":
// average pooling -> RMS norm -> RoPE; "incremental pooled-key cache（COMMON-004）":
// only newly completed blocks are computed).
//
// One launch, two kinds of work groups: the first `copy_wgs` copy the new rows
// with 16-byte loads/stores; the rest each produce the pooled rows of
// `blocks_per_wg` consecutive blocks.  A block's tokens below n_before come from
// k_raw and the others from k_new, so the two kinds never touch the same bytes.
#include "qsa_append.h"

namespace qsa {
namespace {

constexpr int kThreads = kAppendThreads;

struct PoolLaunch {
    AppendArgs a;
    int32_t copy_wgs;
    int32_t blocks_per_wg;
};

__global__ __launch_bounds__(kThreads) void append_kernel(PoolLaunch L)
{
    if ((int32_t)blockIdx.x < L.copy_wgs) {
        append_copy(L.a, blockIdx.x, L.copy_wgs);
        return;
    }
    extern __shared__ f32x2 cs[];  // [blocks_per_wg][d/2]: (cos, sin)
    const int32_t wg = (int32_t)blockIdx.x - L.copy_wgs;
    const int32_t b0 = L.a.b_lo + wg * L.blocks_per_wg;
    const int32_t nbk = min(L.blocks_per_wg, L.a.b_lo + L.a.n_blocks - b0);
    append_pool(L.a, b0, nbk, cs, nullptr);
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint4 *p, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
        p[i] = uint4{0, 0, 0, 0};
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s)
{
    PoolLaunch L;
    L.a = a;
    int64_t n16 = 0;
    for (int i = 0; i < 3; i++)
        n16 = (a.seg[i].n16 > n16) ? a.seg[i].n16 : n16;
    L.copy_wgs = (int32_t)((n16 + kThreads - 1) / kThreads);
    if (L.copy_wgs > 1024)
        L.copy_wgs = 1024;
    const int32_t units_per_block = a.H * (a.d / 8);
    L.blocks_per_wg = units_per_block >= kThreads ? 1 : kThreads / units_per_block;
    const int32_t pool_wgs = (a.n_blocks + L.blocks_per_wg - 1) / L.blocks_per_wg;
    const int32_t grid = L.copy_wgs + pool_wgs;
    if (grid == 0)
        return hipSuccess;
    const size_t lds = sizeof(f32x2) * (size_t)L.blocks_per_wg * (size_t)(a.d / 2);
    hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(kThreads), lds, s, L);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s)
{
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0)
        return hipSuccess;
    int64_t grid = (n16 + kThreads - 1) / kThreads;
    if (grid > 2048)
        grid = 2048;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, s, (uint4 *)p,
                       n16);
    return hipGetLastError();
}

}  // namespace qsa
