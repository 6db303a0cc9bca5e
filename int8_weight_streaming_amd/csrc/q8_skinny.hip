// q8_skinny.hip -- batch 1..8 decode products over Q8_0 weights.
//
//   y[m][j] = sum_b wd[j][b] * sum_{i<32} wq[j][32b+i] * x[m][32b+i]
//
// The weights are streamed from HBM exactly once per call for all m rows
// [Frigg README, Finding 8: a batched kernel reads each weight once, so its
// cost is nearly flat in the batch size; "The machine": at batch 1 the time is
// weight bytes / bandwidth].
//
// Work layout (wave64):
//  * A lane group of G lanes (G = 16 for tall matrices, 32 or 64 for short
//    ones) owns R weight rows.  The rows are cut into 16-byte chunks (half a Q8
//    block); lane g takes chunks g, g+G, g+2G, ..., so one load instruction of a
//    group reads G*16 contiguous bytes of a row.  Weight loads are non-temporal
//    (streamed once, kept out of the caches) and are issued before the
//    activations are fetched, so the two memory latencies overlap.
//  * K is walked in tiles of G*CPL chunks.  Activations of a tile live in
//    registers at batch 1-2; larger batches stage them in LDS once per
//    workgroup and tile.
//  * bf16 activations (W8A16): the int8 codes are converted exactly to packed
//    bf16 pairs and multiplied with v_dot2_f32_bf16 (fp32 accumulate); each
//    chunk's partial is folded with its block scale by one FMA.
//  * Q8 activations: four v_dot4_i32_i8 give the chunk's exact int32 sum; the
//    two halves of a block (neighbouring lanes) are added as integers with one
//    DPP step, so the block sum is exact, then converted and folded with wd*xd
//    once per block [fak MODEL-BASELINE-RESULTS, ACT 4 "How the GEMM was
//    closed": deferred reduction, one fold per block].
//  * Chunks past the end of a row are computed with a zero scale instead of
//    being skipped, so every lane stays active for the DPP steps.
//  * The G partial sums of a row are combined by a fixed DPP tree (no atomics,
//    no cross-workgroup split): every output is written by exactly one group and
//    results are bitwise reproducible [Frigg README, Finding 8: a partials
//    buffer instead of atomics keeps graph replay bit-identical].
#include "q8_skinny_kernel.hpp"

namespace q8 {

// ------------------------------------------------------------------ launch

template <int M, int ACT, int G, int R, int CPL>
static hipError_t launch_cfg(const int8_t* wq, const uint16_t* wd, int64_t n, int nb,
                             const void* x, const uint16_t* xd, float* y, hipStream_t stream) {
    constexpr int RPW = 4 * (64 / G) * R;
    constexpr int TCH = G * CPL;
    size_t lds = 0;
    if (!x_in_registers<M, ACT>())
        lds = ACT == 0 ? (size_t)M * TCH * 32 : (size_t)M * TCH * 16 + (size_t)M * (TCH / 2) * 4;
    const int64_t grid = (n + RPW - 1) / RPW;
    skinny_kernel<M, ACT, G, R, CPL><<<(unsigned)grid, 256, lds, stream>>>(wq, wd, n, nb, x, xd, y, FuseArgs{0, 0});
    return hipGetLastError();
}

// Configurations measured per Mimir shape and batch (graph replay, weights
// rotated past the caches, batch 1, 2, 4 and 8):
//  * tall matrices: 16-lane groups, 2 rows per group, 6 chunks per lane per
//    K tile (K = 1536 in one tile) -- at batch 1-2 from 32 rows per compute
//    unit on, above batch 2 only from 128 (below that one workgroup per
//    compute unit leaves the per-lane arithmetic of 3-8 rows exposed);
//  * shorter matrices need smaller row tiles to cover every compute unit:
//    32-lane groups, one row each, K tile = 96 chunks (K = 1536 in one tile);
//    for longer K, 32-lane groups with a 256-chunk tile at batch 1-2
//    (activations in registers) and one wave per row above that.
SkinnyLayout skinny_layout(int64_t n, int64_t k, int m, int cu_count) {
    const int64_t tall_wgs = (n + 31) / 32;
    if (tall_wgs >= (int64_t)cu_count * (m <= 2 ? 1 : 4)) return {16, 2, 6, false};
    if (k / 32 <= 48) return {32, 1, 3, false};
    if (m <= 2) return {32, 1, 8, false};
    return {64, 1, 2, false};
}

template <int M, int ACT>
static hipError_t launch_m(const int8_t* wq, const uint16_t* wd, int64_t n, int nb,
                           const void* x, const uint16_t* xd, float* y,
                           const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
    const SkinnyLayout L = skinny_layout(n, (int64_t)nb * 32, M, dev.cu_count);
    if (L.g == 16) return launch_cfg<M, ACT, 16, 2, 6>(wq, wd, n, nb, x, xd, y, stream);
    if (L.cpl == 3) return launch_cfg<M, ACT, 32, 1, 3>(wq, wd, n, nb, x, xd, y, stream);
    if constexpr (M <= 2) {
        return launch_cfg<M, ACT, 32, 1, 8>(wq, wd, n, nb, x, xd, y, stream);
    } else {
        return launch_cfg<M, ACT, 64, 1, 2>(wq, wd, n, nb, x, xd, y, stream);
    }
}

template <int ACT>
static hipError_t launch_act(const int8_t* wq, const uint16_t* wd, int64_t n, int nb, int m,
                             const void* x, const uint16_t* xd, float* y,
                             const DeviceInfo& dev, hipStream_t stream) {
    switch (m) {
        case 1: return launch_m<1, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 2: return launch_m<2, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 3: return launch_m<3, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 4: return launch_m<4, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 5: return launch_m<5, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 6: return launch_m<6, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 7: return launch_m<7, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 8: return launch_m<8, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_skinny(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m,
                         int act, const void* x, const uint16_t* xd, float* y,
                         const DeviceInfo& dev, hipStream_t stream) {
    if (act == 0 && skinny_mfma_applies(n, k, m, dev.cu_count))
        return launch_skinny_mfma(wq, wd, n, k, m, x, y, dev, stream);
    const int nb = (int)(k / 32);
    if (act == 0) return launch_act<0>(wq, wd, n, nb, m, x, xd, y, dev, stream);
    return launch_act<1>(wq, wd, n, nb, m, x, xd, y, dev, stream);
}

// ------------------------------------------------------------------ block dots

// isum[t][j][b] for t < m: a lane pair per (t, j, b), each lane one 16-byte
// half of the block, summed by block_dot_halves -- the routine the
// Q8-activation decode products use.  The loop bound is uniform per
// workgroup and a lane past the end computes a clamped pair without storing,
// so both lanes of every pair reach the DPP step together.
__global__ __launch_bounds__(256) void block_dots_kernel(const int8_t* __restrict__ wq, int64_t n, int nb,
                                                         int m, const int8_t* __restrict__ xq,
                                                         int32_t* __restrict__ isum) {
    const int64_t total = (int64_t)m * n * nb;
    const int64_t k = (int64_t)nb * 32;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < 2 * total;
         base += (int64_t)gridDim.x * blockDim.x) {
        const int64_t li = base + threadIdx.x;
        const bool live = li < 2 * total;
        const int64_t i = live ? li >> 1 : 0;
        const int half = (int)(li & 1);
        const int b = (int)(i % nb);
        const int64_t j = (i / nb) % n;
        const int t = (int)(i / ((int64_t)nb * n));
        const u32x4 w = *reinterpret_cast<const u32x4*>(wq + j * k + (int64_t)b * 32 + 16 * half);
        const u32x4 x = *reinterpret_cast<const u32x4*>(xq + t * k + (int64_t)b * 32 + 16 * half);
        const int s = block_dot_halves(w, x);
        if (live && half == 0) isum[i] = s;
    }
}

hipError_t launch_block_dots(const int8_t* wq, int64_t n, int64_t k, int m, const int8_t* xq,
                             int32_t* isum, const DeviceInfo& dev, hipStream_t stream) {
    const int nb = (int)(k / 32);
    const int64_t lanes = 2 * (int64_t)m * n * nb;
    int64_t grid = (lanes + 255) / 256;
    const int64_t cap = (int64_t)dev.cu_count * 16;
    if (grid > cap) grid = cap;
    (void)hipGetLastError();
    block_dots_kernel<<<(int)grid, 256, 0, stream>>>(wq, n, nb, m, xq, isum);
    return hipGetLastError();
}

}  // namespace q8
