// Device-side helpers shared by the QSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace qsa {

typedef _Float16 h16;
typedef h16 h16x2 __attribute__((ext_vector_type(2)));
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kBlockTokens = 4;

// Order-preserving map of an fp32 score to uint32: a larger key is a higher
// rank.  -0 is folded onto +0 (they tie) and NaN maps to 0, below every number.
__device__ __forceinline__ uint32_t score_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if (s != s)
        return 0u;
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Total order of (score, block id) pairs as one 64-bit word: the score key in
// the high half, the complemented id in the low half, so a larger word ranks
// higher and equal scores rank the lower id first.  0 ranks below every pair
// and marks an empty slot.
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t id)
{
    return ((uint64_t)score_key(s) << 32) | (uint32_t)~id;
}
__device__ __forceinline__ uint32_t rank_id(uint64_t r) { return ~(uint32_t)r; }

__device__ __forceinline__ float dot8(h16x8 a, h16x8 b, float acc)
{
    acc = __builtin_amdgcn_fdot2(h16x2{a[0], a[1]}, h16x2{b[0], b[1]}, acc, false);
    acc = __builtin_amdgcn_fdot2(h16x2{a[2], a[3]}, h16x2{b[2], b[3]}, acc, false);
    acc = __builtin_amdgcn_fdot2(h16x2{a[4], a[5]}, h16x2{b[4], b[5]}, acc, false);
    acc = __builtin_amdgcn_fdot2(h16x2{a[6], a[7]}, h16x2{b[6], b[7]}, acc, false);
    return acc;
}

// Sum over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// ---- cross-lane moves without LDS round trips (DPP within 16-lane rows, then
// v_readlane across the 4 rows of the wave)
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// sum over each aligned group of 4 lanes, result in all 4
__device__ __forceinline__ float quad_sum(float x)
{
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    return x;
}

__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, dpp<kDppQuadXor1>(x));
    x = fmaxf(x, dpp<kDppQuadXor2>(x));
    x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp<kDppRowMirror>(x));  // every lane of a row holds the row's max
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    x += dpp<kDppRowHalfMirror>(x);
    x += dpp<kDppRowMirror>(x);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (a + b) + (c + d);
}

// Maximum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the matching lanes of the four
// 16-lane rows), every such lane gets it: the gfx950 row swaps leave a lane's own
// value and its partner's (16, then 32 lanes away) in the two results, so the
// maximum of the pair is the same whichever result holds which.
__device__ __forceinline__ float max_across_rows(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Minimum / maximum of a uint32 over the 64 lanes (every lane gets it).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x)
{
    x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor1, 0xf, 0xf, false));
    x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor2, 0xf, 0xf, false));
    x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowHalfMirror, 0xf, 0xf, false));
    x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowMirror, 0xf, 0xf, false));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return min(min(a, b), min(c, d));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor1, 0xf, 0xf, false));
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor2, 0xf, 0xf, false));
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowHalfMirror, 0xf, 0xf, false));
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowMirror, 0xf, 0xf, false));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return max(max(a, b), max(c, d));
}

// Maximum of a uint64 over the 64 lanes (every lane gets it).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x)
{
    auto step = [](uint64_t v, uint64_t o) { return o > v ? o : v; };
    auto dpp64 = [](uint64_t v, auto ctrl) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, decltype(ctrl)::value, 0xf, 0xf, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), decltype(ctrl)::value, 0xf, 0xf, false);
        return ((uint64_t)hi << 32) | lo;
    };
    x = step(x, dpp64(x, std::integral_constant<int, kDppQuadXor1>{}));
    x = step(x, dpp64(x, std::integral_constant<int, kDppQuadXor2>{}));
    x = step(x, dpp64(x, std::integral_constant<int, kDppRowHalfMirror>{}));
    x = step(x, dpp64(x, std::integral_constant<int, kDppRowMirror>{}));
    auto rl = [](uint64_t v, int l) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
        return ((uint64_t)hi << 32) | lo;
    };
    return step(step(rl(x, 0), rl(x, 16)), step(rl(x, 32), rl(x, 48)));
}

// Inclusive prefix sum over the 64 lanes: shifts of 1, 2, 4, 8 inside each row of
// 16 lanes (lanes shifted in from outside the row read 0), then the totals of
// the rows below are added from lanes 15, 31 and 47.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const uint32_t row = lane_id() >> 4;
    return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Rank of this lane among the set lanes of a 64-bit ballot mask.
__device__ __forceinline__ uint32_t rank_in_mask(uint64_t mask)
{
    const uint32_t l = lane_id();
    const uint64_t below = (l == 0) ? 0ull : (mask & (~0ull >> (64 - l)));
    return (uint32_t)__popcll(below);
}

// Appends from the lanes with `want` set to a global list whose length is *cnt;
// one atomic per wave.  Returns this lane's slot (only meaningful when want).
__device__ __forceinline__ uint32_t wave_append_slot(bool want, uint32_t *cnt)
{
    const uint64_t mask = __ballot(want);
    if (mask == 0)
        return 0;
    const uint32_t leader = (uint32_t)(__ffsll((unsigned long long)mask) - 1);
    uint32_t base = 0;
    if (lane_id() == leader)
        base = atomicAdd(cnt, (uint32_t)__popcll(mask));
    base = __shfl(base, leader, kWave);
    return base + rank_in_mask(mask);
}

}  // namespace qsa
