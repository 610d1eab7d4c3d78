// Pooled-key cache append: raw/K/V row copies plus the pooled summary of every
// 4-token block that completes (Qiita part 10, "QSAとQSA indexerについて":
// average pooling -> RMS norm -> RoPE; "incremental pooled-key cache（COMMON-004）":
// only newly completed blocks are computed).
//
// One launch, two kinds of work groups: the first `copy_wgs` copy the new rows
// with 16-byte loads/stores; the rest each produce the pooled rows of
// `blocks_per_wg` consecutive blocks.  A block's tokens below n_before come from
// k_raw and the others from k_new, so the two kinds never touch the same bytes.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;

struct PoolLaunch {
    AppendArgs a;
    int32_t copy_wgs;
    int32_t blocks_per_wg;
};

__global__ __launch_bounds__(kThreads) void append_kernel(PoolLaunch L)
{
    const AppendArgs &a = L.a;
    if ((int32_t)blockIdx.x < L.copy_wgs) {
        const int64_t stride = (int64_t)L.copy_wgs * kThreads;
#pragma unroll
        for (int s = 0; s < 3; s++) {
            const uint4 *src = (const uint4 *)a.seg[s].src;
            uint4 *dst = (uint4 *)a.seg[s].dst;
            for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < a.seg[s].n16;
                 i += stride)
                dst[i] = src[i];
        }
        return;
    }

    // ---- pooled rows of blocks [b0, b0 + nbk)
    extern __shared__ f32x2 cs[];  // [blocks_per_wg][d/2]: (cos, sin)
    const int32_t d = a.d, H = a.H, half = d / 2;
    const int64_t row = (int64_t)H * d;
    const int32_t wg = (int32_t)blockIdx.x - L.copy_wgs;
    const int32_t b0 = a.b_lo + wg * L.blocks_per_wg;
    const int32_t nbk = min(L.blocks_per_wg, a.b_lo + a.n_blocks - b0);

    // RoPE angles of pair i at block position 4b: 4b * base^(-2i/d), in fp64.
    for (int e = threadIdx.x; e < nbk * half; e += kThreads) {
        const int bl = e / half, i = e - bl * half;
        const double pos = (double)kBlockTokens * (double)(b0 + bl);
        const double inv = pow((double)a.base, -2.0 * (double)i / (double)d);
        double sn, cn;
        sincos(pos * inv, &sn, &cn);
        cs[e] = f32x2{(float)cn, (float)sn};
    }
    __syncthreads();

    // A unit is (block, head, quad): 4 RoPE pairs (i0..i0+3, i0+d/2..i0+d/2+3).
    // The d/8 units of one head sit in consecutive lanes of one wave.
    const int32_t qph = d / 8;
    const int32_t units = nbk * H * qph;
    for (int32_t ub = 0; ub < units; ub += kThreads) {
        const int32_t u = ub + threadIdx.x;
        const bool active = u < units;
        const int32_t uu = active ? u : 0;
        const int32_t bl = uu / (H * qph);
        const int32_t h = (uu / qph) % H;
        const int32_t i0 = (uu % qph) * 4;
        const int64_t b = b0 + bl;
        const int64_t lo = (int64_t)h * d + i0, hi = lo + half;

        f32x4 mlo = {0, 0, 0, 0}, mhi = {0, 0, 0, 0};
        if (active) {
#pragma unroll
            for (int t = 0; t < kBlockTokens; t++) {
                const int64_t tok = b * kBlockTokens + t;
                const h16 *src = (tok < a.n_before) ? a.k_raw + tok * row
                                                    : a.k_new + (tok - a.n_before) * row;
                const h16x4 xl = *(const h16x4 *)(src + lo);
                const h16x4 xh = *(const h16x4 *)(src + hi);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    mlo[j] += (float)xl[j];
                    mhi[j] += (float)xh[j];
                }
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            mlo[j] *= 0.25f;
            mhi[j] *= 0.25f;
            ss += mlo[j] * mlo[j] + mhi[j] * mhi[j];
        }
        // reduce over the d/8 lanes of this head (qph is a power of two <= 64)
        for (int o = 1; o < qph; o <<= 1)
            ss += __shfl_xor(ss, o, kWave);
        const float rms = sqrtf(ss / (float)d + a.eps);
        if (active) {
            h16x4 ol, oh;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float wl = a.rms_w ? a.rms_w[i0 + j] : 1.f;
                const float wh = a.rms_w ? a.rms_w[i0 + j + half] : 1.f;
                const float nl = mlo[j] / rms * wl;
                const float nh = mhi[j] / rms * wh;
                const f32x2 c = cs[bl * half + i0 + j];
                ol[j] = (h16)(nl * c[0] - nh * c[1]);
                oh[j] = (h16)(nl * c[1] + nh * c[0]);
            }
            *(h16x4 *)(a.k_pool + b * row + lo) = ol;
            *(h16x4 *)(a.k_pool + b * row + hi) = oh;
        }
    }
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
