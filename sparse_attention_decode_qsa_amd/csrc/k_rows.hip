// Per-row attention of a prefill chunk on the matrix cores (Qiita part 10,
// "selected QSA K/V gather（COMMON-005）": a query row attends over the cells of
// its own chosen blocks plus its tail, exactly as a decode step at that row's
// length would; "QSAとQSA indexerについて": every row of a prefill chunk is such
// a decode at its own length).
//
// rows_attn_kernel<G>: one work group per (KV head, row), 4 waves; wave w takes
// tiles w, w + 4, ... of 32 cells.  Each tile goes from the caches straight into
// the matrix operands (v_mfma_f32_16x16x32_f16), nothing staged in LDS:
//   S^T = K Q^T     A = 16 cells x 32 dims of K (64-byte pieces of each K row),
//                   B = the G query heads of the group, zero-padded to 16;
//   O^T += V^T P^T  A = 16 value dims x 32 cells: a lane reads the 16-byte piece
//                   8m .. 8m+7 of 8 V rows (each read instruction covers whole
//                   256-byte rows) and transposes the 8 x 8 halves in registers,
//                   so MFMA r of the tile holds value dims 8m + r;
//                   B = P^T as the score product leaves it in the lane (cells
//                   16t + 4j + e of tile half t): the k slots of the PV product
//                   are those cells, and the V rows a lane reads are the same
//                   cells, two whole 4-token blocks.
// A lane therefore holds the scores, the softmax state and 32 output dims of one
// head (its column of S^T and O^T), and no value crosses lanes except the maximum
// over the 4 lane rows of the head.  Online softmax in the log2 domain; P is
// rounded to binary16 for the PV product.  At the end the four waves' (m, l, O)
// are merged through LDS.
//
// With a union-size array (grouped-union prefill) the kernel leaves out the rows
// whose group the union kernel takes (union size at most u_limit blocks).
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kRThreads = 256;
constexpr int kRWaves = kRThreads / kWave;
constexpr int kRTile = 32;   // cells per tile
constexpr int kRDim = 128;   // D = DV
constexpr int kROPitch = kRDim + 4;  // LDS pitch of a head's merged outputs (floats)
constexpr float kLog2e = 1.4426950408889634f;
// cells of a row: 4 per chosen block and up to 3 of the tail, up to a whole tile;
// a multiple of 64 (the table is filled a wave, i.e. two tiles, at a time)
constexpr int kRMaxCells = ((kBlockTokens * kMaxTopk + 3 + 63) / 64) * 64;

// Sum over lanes l, l ^ 16, l ^ 32, l ^ 48, in the same order in all four (the
// row swaps leave a lane's own value and its partner's; fp addition of two terms
// commutes).
__device__ __forceinline__ float sum_across_rows(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS of a work group: the byte offset of every cell's row from the head's base
// (token 0 for a cell that is not there) and a validity mask per tile of 32 cells;
// after the tiles the same bytes hold the four waves' partial outputs.
template <int G>
struct RowsLds {
    union {
        struct {
            uint32_t coff[kRMaxCells];
            int32_t bl[kRMaxCells / kBlockTokens];  // the row's block ids, -1 dropped
        };
        float om[kRWaves][G][kROPitch];
    };
    uint32_t tmask[kRMaxCells / kRTile];
    float mm[kRWaves][G], ll[kRWaves][G];
};

// A row of a union group: merge of the union kernel's split partials for the
// group's heads (p = [row][hq][splits][kUnionPartStride]: m, l, -, -, then the
// outputs), o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <int G>
__device__ void combine_union_row(const RowsArgs &a, int32_t row, int g)
{
    const int S = a.splits;
    for (int i = threadIdx.x; i < G * (kRDim / 4); i += kRThreads) {
        const int h = g * G + i / (kRDim / 4), c = i % (kRDim / 4);
        const float *pb = a.part + ((int64_t)row * a.hq + h) * S * kUnionPartStride;
        float M = -INFINITY;
        for (int sp = 0; sp < S; sp++)
            M = fmaxf(M, pb[sp * kUnionPartStride]);
        const float mref = (M == -INFINITY) ? 0.f : M;
        float L = 0.f;
        f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < S; sp++) {
            const f32x4 ml = *(const f32x4 *)(pb + sp * kUnionPartStride);
            const float w = __builtin_amdgcn_exp2f(ml[0] - mref);
            L += w * ml[1];
            o += w * *(const f32x4 *)(pb + sp * kUnionPartStride + 4 + 4 * c);
        }
        *(f32x4 *)(a.out + ((int64_t)row * a.hq + h) * kRDim + 4 * c) = o * (1.f / L);
    }
}

// 4 waves per SIMD (at most 128 registers): with two loads per lane in flight that
// is the ~32 KiB per CU the gather runs best at
template <int G>
__global__ __launch_bounds__(kRThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void
rows_attn_kernel(RowsArgs a)
{
    static_assert(G == 4 || G == 8 || G == 16, "query heads per KV head");
    __shared__ __attribute__((aligned(16))) RowsLds<G> sm;

    const int g = blockIdx.x;
    const int32_t row = blockIdx.y;
    if (a.n_u && a.n_u[row / a.group_rows] <= a.u_limit) {
        // this row's group is the union kernel's (uniform over the group): only the
        // merge of its split partials, if it has several
        if (a.splits > 1)
            combine_union_row<G>(a, row, g);
        return;
    }
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    const int n = lane & 15, j4 = lane >> 4;

    const int32_t N = a.pos0 + row + 1;  // tokens this row sees
    const int32_t nbr = N / kBlockTokens, nsel = min(a.k, nbr);
    const int32_t tail = N - kBlockTokens * nbr;
    const int32_t count = kBlockTokens * nsel + tail;
    const int32_t ntile = (count + kRTile - 1) / kRTile;
    const uint32_t rowb = (uint32_t)a.hkv * kRDim * sizeof(h16);  // bytes per token row
    // the row's blocks: its chosen ids (an id outside [0, nbr) can only come from a
    // broken selection: its cells are dropped), then the tail's block, read with
    // all loads in flight at once
    const int32_t *br = a.blk + (int64_t)row * a.ldb;
    constexpr int kBPer = (kRMaxCells / kBlockTokens + kRThreads - 1) / kRThreads;
    int32_t ids[kBPer];
#pragma unroll
    for (int j = 0; j < kBPer; j++) {
        const int32_t i = t + j * kRThreads;
        ids[j] = (i < nsel) ? br[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kBPer; j++) {
        const int32_t i = t + j * kRThreads;
        if (i < ntile * (kRTile / kBlockTokens)) {
            int32_t id = -1;
            if (i < nsel)
                id = ((uint32_t)ids[j] < (uint32_t)nbr) ? ids[j] : -1;
            else if (i == nsel && tail > 0)
                id = nbr;
            sm.bl[i] = id;
        }
    }
    __syncthreads();
    // cells: 4 tokens per block; the tail block's cells past the row's count are not there
    for (int32_t c = t; c < ntile * kRTile; c += kRThreads) {
        const int32_t b = sm.bl[c / kBlockTokens];
        const int32_t tok = (b >= 0 && c < count) ? kBlockTokens * b + (c & 3) : -1;
        sm.coff[c] = tok >= 0 ? (uint32_t)tok * rowb : 0u;
        const uint64_t there = __ballot(tok >= 0);  // cells of two tiles per wave
        if (lane == 0) {
            sm.tmask[c / kRTile] = (uint32_t)there;
            sm.tmask[c / kRTile + 1] = (uint32_t)(there >> 32);
        }
    }

    const char *kg = (const char *)(a.k_cache + (int64_t)g * kRDim);
    const char *vg = (const char *)(a.v_cache + (int64_t)g * kRDim);
    // B of the score product: head n of the group, dims 32 kk + 8 j4 .. + 8
    h16x8 qf[4];
    const h16 *qr = a.q + ((int64_t)row * a.hq + (int64_t)g * G + (n < G ? n : 0)) * kRDim;
#pragma unroll
    for (int kk = 0; kk < 4; kk++)
        qf[kk] = (n < G) ? *(const h16x8 *)(qr + 32 * kk + 8 * j4) : h16x8{0, 0, 0, 0, 0, 0, 0, 0};

    f32x4 oacc[8];
#pragma unroll
    for (int r = 0; r < 8; r++)
        oacc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = a.scale * kLog2e;
    __syncthreads();

    // Few loads in flight: a gather from the caches keeps ~0.5 us latency only while
    // a CU has about 32-64 KiB of loads outstanding (4 waves per SIMD x 2-4 pieces
    // of 1 KiB per wave); with more in flight the latency grows faster than the
    // bytes and the rate falls to about half.  So each step below issues two to four
    // 16-byte pieces per lane and uses them before the next step's loads go out
    // (the compiler barriers keep it from hoisting loads across steps).
    auto fence = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto piece = [](const char *base, uint32_t off) { return *(const h16x8 *)(base + off); };
    for (int32_t tile = wave; tile < ntile; tile += kRWaves) {
        const int32_t c0 = tile * kRTile;
        // S^T = K Q^T over 4 k-steps; step kk reads dims 32 kk + 8 j4 of cells
        // c0 + n and c0 + 16 + n (the A rows of the two cell halves).  Steps go out
        // in pairs: steps 2p and 2p + 1 read bytes 128p .. 128p + 127 of each K row,
        // one whole line per round trip (a line read in two halves a step apart took
        // 2-4% longer; all four steps at once, 6% longer)
        uint32_t koff[2];
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
            koff[tt] = sm.coff[c0 + 16 * tt + n] + 16u * j4;
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kp = 0; kp < 2; kp++) {
            h16x8 kf[2][2];
#pragma unroll
            for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
                for (int tt = 0; tt < 2; tt++)
                    kf[k2][tt] = piece(kg + 64 * (2 * kp + k2), koff[tt]);
#pragma unroll
            for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
                for (int tt = 0; tt < 2; tt++)
                    sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[k2][tt], qf[2 * kp + k2],
                                                                      sacc[tt], 0, 0, 0);
            fence();
        }

        // the lane's cells in the score layout: c0 + 16 tt + 4 j4 + e (two whole
        // 4-token blocks, also the V rows it reads below); bit 4 tt + e of vm says
        // the cell is there (none for a padding head)
        const uint32_t tm = sm.tmask[tile];
        const uint32_t vm = (n < G) ? (((tm >> (4 * j4)) & 0xfu) | (((tm >> (16 + 4 * j4)) & 0xfu) << 4))
                                    : 0u;
        uint32_t voff[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
            const uint4 o = *(const uint4 *)&sm.coff[c0 + 16 * tt + 4 * j4];
            voff[tt][0] = o.x + 16u * n;
            voff[tt][1] = o.y + 16u * n;
            voff[tt][2] = o.z + 16u * n;
            voff[tt][3] = o.w + 16u * n;
        }
        // the first half's first two V pieces go out before the softmax (a cell that
        // is not there reads token 0: a real, finite row, and its p is 0)
        h16x8 vin[4];
        vin[0] = piece(vg, voff[0][0]);
        vin[1] = piece(vg, voff[0][1]);

        // online softmax of head n over the tile's cells (order 4 tt + e)
        float s[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            s[i] = ((vm >> i) & 1u) ? sacc[i / 4][i % 4] : -INFINITY;
            tmax = fmaxf(tmax, s[i]);
        }
        tmax = max_across_rows(tmax);
        const float mnew = fmaxf(m_run, tmax * sl2);
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mref);
        const bool moved = mnew != m_run;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -mref));
            psum += s[i];
        }
        l_run = l_run * alpha + psum;
        m_run = mnew;
        if (__any(moved)) {
#pragma unroll
            for (int r = 0; r < 8; r++)
                oacc[r] *= alpha;
        }

        // O^T += V^T P^T, one 16-cell half at a time (v_mfma_f32_16x16x16_f16: the
        // lane's k slots are its 4 cells of the half, one 4-token block); the V
        // pieces are dims 8 n .. + 8 of those 4 rows, two per step, transposed so
        // that MFMA r takes dims 8 n + r
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
            if (tt == 1) {
                vin[0] = piece(vg, voff[1][0]);
                vin[1] = piece(vg, voff[1][1]);
            }
            // the pair in flight is used before the next pair goes out
            asm volatile("" : "+v"(vin[0]), "+v"(vin[1]));
            fence();
            vin[2] = piece(vg, voff[tt][2]);
            vin[3] = piece(vg, voff[tt][3]);
            const h16x4 pf = h16x4{(h16)s[4 * tt], (h16)s[4 * tt + 1], (h16)s[4 * tt + 2],
                                   (h16)s[4 * tt + 3]};
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const h16x4 vt = h16x4{vin[0][r], vin[1][r], vin[2][r], vin[3][r]};
                oacc[r] = __builtin_amdgcn_mfma_f32_16x16x16f16(vt, pf, oacc[r], 0, 0, 0);
            }
            fence();
        }
    }

    // merge of the four waves: head n's dims 32 j4 + 8 e + r from this lane (the
    // cell offsets are dead once every wave is past its tiles)
    const float lsum = sum_across_rows(l_run);
    __syncthreads();
    if (n < G) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            float *op = &sm.om[wave][n][32 * j4 + 8 * e];
            *(f32x4 *)op = f32x4{oacc[0][e], oacc[1][e], oacc[2][e], oacc[3][e]};
            *(f32x4 *)(op + 4) = f32x4{oacc[4][e], oacc[5][e], oacc[6][e], oacc[7][e]};
        }
        if (j4 == 0) {
            sm.mm[wave][n] = m_run;
            sm.ll[wave][n] = lsum;
        }
    }
    __syncthreads();
    float *orow = a.out + ((int64_t)row * a.hq + (int64_t)g * G) * kRDim;
    for (int i = t; i < G * kRDim; i += kRThreads) {
        const int h = i / kRDim, d = i - h * kRDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kRWaves; w++)
            M = fmaxf(M, sm.mm[w][h]);
        const float Mref = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kRWaves; w++) {
            const float sc = __builtin_amdgcn_exp2f(sm.mm[w][h] - Mref);
            L += sc * sm.ll[w][h];
            o += sc * sm.om[w][h][d];
        }
        orow[i] = o / L;
    }
}

}  // namespace

bool rows_supported(int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t k, int64_t n_tokens)
{
    if (hkv <= 0 || hq % hkv || d != kRDim || dv != kRDim || k > kMaxTopk)
        return false;
    // cell offsets are 32-bit byte offsets into the caches
    if (n_tokens * hkv * kRDim * (int64_t)sizeof(h16) > (int64_t)UINT32_MAX)
        return false;
    const int32_t G = hq / hkv;
    return G == 4 || G == 8 || G == 16;
}

hipError_t launch_rows_attn(const RowsArgs &a, hipStream_t s)
{
    if (a.n_q <= 0)
        return hipSuccess;
    if (!rows_supported(a.hq, a.hkv, kRDim, kRDim, a.k, (int64_t)a.pos0 + a.n_q) ||
        (a.n_u && a.group_rows <= 0) || (a.splits > 1 && (!a.n_u || !a.part)))
        return hipErrorInvalidValue;
    const dim3 grid((uint32_t)a.hkv, (uint32_t)a.n_q);
    switch (a.hq / a.hkv) {
    case 4: hipLaunchKernelGGL(rows_attn_kernel<4>, grid, dim3(kRThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL(rows_attn_kernel<8>, grid, dim3(kRThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(rows_attn_kernel<16>, grid, dim3(kRThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace qsa
