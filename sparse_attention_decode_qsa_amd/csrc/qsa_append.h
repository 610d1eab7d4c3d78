// Append work shared by the stand-alone append kernel and the fused decode scan:
// row copies, and the pooled summary of completed 4-token blocks (Qiita part 10,
// "QSAとQSA indexerについて": average pooling -> RMS norm -> RoPE).
#pragma once

#include "qsa_internal.h"

namespace qsa {

constexpr int kAppendThreads = 256;

// Copies of AppendArgs::seg by work group wg of nwg, NT threads each (16-byte
// units, coalesced).
template <int NT = kAppendThreads>
__device__ __forceinline__ void append_copy(const AppendArgs &a, int wg, int nwg)
{
    const int64_t stride = (int64_t)nwg * NT;
#pragma unroll
    for (int s = 0; s < 3; s++) {
        const uint4 *src = (const uint4 *)a.seg[s].src;
        uint4 *dst = (uint4 *)a.seg[s].dst;
        for (int64_t i = (int64_t)wg * NT + threadIdx.x; i < a.seg[s].n16; i += stride)
            dst[i] = src[i];
    }
}

// Pooled rows of blocks [b0, b0 + nbk) by one work group of NT threads.
// cs: LDS for nbk * d/2 (cos, sin) pairs.  row_lds (may be NULL, nbk == 1): the
// pooled row is also left there in binary16.  A block's tokens below n_before
// come from k_raw, the others from k_new.
template <int NT = kAppendThreads>
__device__ void append_pool(const AppendArgs &a, int32_t b0, int32_t nbk, f32x2 *cs, h16 *row_lds)
{
    const int32_t d = a.d, H = a.H, half = d / 2;
    const int64_t row = (int64_t)H * d;
    // RoPE angles of pair i at block position 4b: 4b * base^(-2i/d), in fp64; the
    // power as 2^(-2i/d * log2(base)) (the fused decode scan's register count, and so
    // its occupancy, is set by this code: pow takes 16 more registers than exp2)
    for (int e = threadIdx.x; e < nbk * half; e += NT) {
        const int bl = e / half, i = e - bl * half;
        const double pos = (double)kBlockTokens * (double)(b0 + bl);
        const double inv = exp2(-2.0 * (double)i / (double)d * log2((double)a.base));
        double sn, cn;
        sincos(pos * inv, &sn, &cn);
        cs[e] = f32x2{(float)cn, (float)sn};
    }
    __syncthreads();
    // A unit is (block, head, quad): 4 RoPE pairs (i0..i0+3, i0+d/2..i0+d/2+3).
    // The d/8 units of one head sit in consecutive lanes of one wave.
    const int32_t qph = d / 8;
    const int32_t units = nbk * H * qph;
    for (int32_t ub = 0; ub < units; ub += NT) {
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
            if (row_lds) {
                *(h16x4 *)(row_lds + lo) = ol;
                *(h16x4 *)(row_lds + hi) = oh;
            }
        }
    }
}

}  // namespace qsa
