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
#include "q8_device.hpp"
#include "q8_internal.hpp"

namespace q8 {

// Activations of one K tile: registers or LDS.
template <int M, int ACT, int CPL>
struct XRegs {
    // bf16: 8 dwords per chunk; Q8: 4 dwords of codes per chunk + block scale.
    uint32_t v[M][CPL][ACT == 0 ? 8 : 4];
    float s[M][CPL];
};

template <int M, int ACT>
constexpr bool x_in_registers() { return M <= 2; }

template <int M, int ACT, int G, int R, int CPL>
__global__ __launch_bounds__(256) void skinny_kernel(const int8_t* __restrict__ wq,
                                                     const uint16_t* __restrict__ wd, int64_t n,
                                                     int nb, const void* __restrict__ xv,
                                                     const uint16_t* __restrict__ xdp,
                                                     float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    constexpr int GPW = 64 / G;                  // lane groups per wave
    constexpr int RPW = 4 * GPW * R;             // rows per workgroup
    constexpr int TCH = G * CPL;                 // chunks per K tile
    constexpr bool XREG = x_in_registers<M, ACT>();
    constexpr int XCH_BYTES = ACT == 0 ? 32 : 16;   // activation bytes per chunk and row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gl = lane & (G - 1), grp = lane / G;
    const int nch = nb * 2;
    const int64_t k = (int64_t)nb * 32;
    const int64_t rbase = (int64_t)blockIdx.x * RPW + (int64_t)(wave * GPW + grp) * R;

    const int8_t* wrow[R];
    const uint16_t* srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = rbase + r < n ? rbase + r : n - 1;   // clamp: loads stay in bounds
        wrow[r] = wq + row * k;
        srow[r] = wd + row * nb;
    }
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    for (int c0 = 0; c0 < nch; c0 += TCH) {
        // ---- activations held in registers: fetched first (small, cache
        // resident), so their latency hides under the weight stream
        XRegs<M, ACT, CPL> xr;
        if (XREG) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = c0 + gl + G * j;
                const int cc = c < nch ? c : 0;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if (ACT == 0) {
                        const uint4* p = reinterpret_cast<const uint4*>(
                            static_cast<const uint16_t*>(xv) + m * k + (int64_t)cc * 16);
                        const uint4 a = p[0], b = p[1];
                        xr.v[m][j][0] = a.x; xr.v[m][j][1] = a.y; xr.v[m][j][2] = a.z; xr.v[m][j][3] = a.w;
                        xr.v[m][j][4] = b.x; xr.v[m][j][5] = b.y; xr.v[m][j][6] = b.z; xr.v[m][j][7] = b.w;
                    } else {
                        const uint4 a = *reinterpret_cast<const uint4*>(
                            static_cast<const int8_t*>(xv) + m * k + (int64_t)cc * 16);
                        xr.v[m][j][0] = a.x; xr.v[m][j][1] = a.y; xr.v[m][j][2] = a.z; xr.v[m][j][3] = a.w;
                        xr.s[m][j] = half_bits_to_float(xdp[(int64_t)m * nb + (cc >> 1)]);
                    }
                }
            }
        }
        // ---- weights and their block scales (raw binary16, converted at use)
        u32x4 w[CPL][R];
        uint16_t sb[CPL][R];
        bool okj[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = c0 + gl + G * j;
            okj[j] = c < nch;
            const int cc = okj[j] ? c : 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                w[j][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[r] + (int64_t)cc * 16));
                sb[j][r] = srow[r][cc >> 1];
            }
        }
        if (!XREG) {
            // stage the tile in LDS while the weight loads are in flight:
            // [m][chunk] with XCH_BYTES per chunk, then the Q8 scales
            const int tch = nch - c0 < TCH ? nch - c0 : TCH;
            __syncthreads();
            const int pieces = M * tch * (XCH_BYTES / 16);
            for (int i = threadIdx.x; i < pieces; i += 256) {
                const int q = ACT == 0 ? (i & 1) : 0;
                const int rest = ACT == 0 ? (i >> 1) : i;
                const int ch = rest % tch, m = rest / tch;
                const unsigned char* src = static_cast<const unsigned char*>(xv) +
                    ((int64_t)m * k + (int64_t)(c0 + ch) * 16) * (ACT == 0 ? 2 : 1) + q * 16;
                *reinterpret_cast<uint4*>(lds + (m * TCH + ch) * XCH_BYTES + q * 16) =
                    *reinterpret_cast<const uint4*>(src);
            }
            if (ACT == 1) {
                float* sc = reinterpret_cast<float*>(lds + M * TCH * XCH_BYTES);
                for (int i = threadIdx.x; i < M * (tch >> 1); i += 256) {
                    const int bl = i % (tch >> 1), m = i / (tch >> 1);
                    sc[m * (TCH / 2) + bl] = half_bits_to_float(xdp[(int64_t)m * nb + (c0 >> 1) + bl]);
                }
            }
            __syncthreads();
        }
        // keep every load of the tile ahead of the arithmetic
        __builtin_amdgcn_sched_barrier(0);
        float ws[CPL][R];
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r) ws[j][r] = okj[j] ? half_bits_to_float(sb[j][r]) : 0.0f;

        // ---- compute
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int cl = gl + G * j;                    // chunk index inside the tile
            const int clc = c0 + cl < nch ? cl : 0;       // LDS slot that exists
            if (ACT == 0) {
                uint32_t wbf[R][8];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    i8x4_to_bf16x4(w[j][r].x, wbf[r][0], wbf[r][1]);
                    i8x4_to_bf16x4(w[j][r].y, wbf[r][2], wbf[r][3]);
                    i8x4_to_bf16x4(w[j][r].z, wbf[r][4], wbf[r][5]);
                    i8x4_to_bf16x4(w[j][r].w, wbf[r][6], wbf[r][7]);
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    uint32_t xc[8];
                    if (XREG) {
#pragma unroll
                        for (int d = 0; d < 8; ++d) xc[d] = xr.v[m][j][d];
                    } else {
                        const uint4* xp = reinterpret_cast<const uint4*>(lds + (m * TCH + clc) * 32);
                        const uint4 a = xp[0], b = xp[1];
                        xc[0] = a.x; xc[1] = a.y; xc[2] = a.z; xc[3] = a.w;
                        xc[4] = b.x; xc[5] = b.y; xc[6] = b.z; xc[7] = b.w;
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float pa = 0.0f, pb = 0.0f;
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            pa = dot2_bf16(wbf[r][d], xc[d], pa);
                            pb = dot2_bf16(wbf[r][4 + d], xc[4 + d], pb);
                        }
                        acc[r][m] = fmaf(pa + pb, ws[j][r], acc[r][m]);
                    }
                }
            } else {
                const bool even = (gl & 1) == 0;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    uint32_t xc[4];
                    float xs;
                    if (XREG) {
#pragma unroll
                        for (int d = 0; d < 4; ++d) xc[d] = xr.v[m][j][d];
                        xs = xr.s[m][j];
                    } else {
                        const uint4 a = *reinterpret_cast<const uint4*>(lds + (m * TCH + clc) * 16);
                        xc[0] = a.x; xc[1] = a.y; xc[2] = a.z; xc[3] = a.w;
                        xs = reinterpret_cast<const float*>(lds + M * TCH * 16)[m * (TCH / 2) + (clc >> 1)];
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        int s = 0;
                        s = __builtin_amdgcn_sdot4((int)w[j][r].x, (int)xc[0], s, false);
                        s = __builtin_amdgcn_sdot4((int)w[j][r].y, (int)xc[1], s, false);
                        s = __builtin_amdgcn_sdot4((int)w[j][r].z, (int)xc[2], s, false);
                        s = __builtin_amdgcn_sdot4((int)w[j][r].w, (int)xc[3], s, false);
                        // exact int32 block sum: add the neighbouring lane's half
                        s += __builtin_amdgcn_update_dpp(0, s, 0xB1, 0xF, 0xF, true);
                        const float t = even ? ws[j][r] * xs : 0.0f;
                        acc[r][m] = fmaf((float)s, t, acc[r][m]);
                    }
                }
            }
        }
    }

    // Combine the G partial sums of every (row, m); all lanes of the group end
    // with the same value.
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = group_sum<G>(acc[r][m]);

    // Lane g of the group stores value g (then g + G, ...): rows of one m land on
    // consecutive lanes.
    constexpr int NV = R * M;
#pragma unroll
    for (int base = 0; base < NV; base += G) {
        const int idx = base + gl;
        float out = 0.0f;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (idx == m * R + r) out = acc[r][m];
        if (idx < NV) {
            const int m = idx / R, r = idx % R;
            const int64_t row = rbase + r;
            if (row < n) y[(int64_t)m * n + row] = out;
        }
    }
}

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
    skinny_kernel<M, ACT, G, R, CPL><<<(unsigned)grid, 256, lds, stream>>>(wq, wd, n, nb, x, xd, y);
    return hipGetLastError();
}

template <int M, int ACT>
static hipError_t launch_m(const int8_t* wq, const uint16_t* wd, int64_t n, int nb,
                           const void* x, const uint16_t* xd, float* y,
                           const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
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
    const int64_t tall_wgs = (n + 31) / 32;
    if (tall_wgs >= (int64_t)dev.cu_count * (M <= 2 ? 1 : 4))
        return launch_cfg<M, ACT, 16, 2, 6>(wq, wd, n, nb, x, xd, y, stream);
    if (nb <= 48) return launch_cfg<M, ACT, 32, 1, 3>(wq, wd, n, nb, x, xd, y, stream);
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
    const int nb = (int)(k / 32);
    if (act == 0) return launch_act<0>(wq, wd, n, nb, m, x, xd, y, dev, stream);
    return launch_act<1>(wq, wd, n, nb, m, x, xd, y, dev, stream);
}

// ------------------------------------------------------------------ block dots

// isum[t][j][b] for t < m: one thread per (t, j, b), using the whole-block
// int8 dot routine.
__global__ __launch_bounds__(256) void block_dots_kernel(const int8_t* __restrict__ wq, int64_t n, int nb,
                                                         int m, const int8_t* __restrict__ xq,
                                                         int32_t* __restrict__ isum) {
    const int64_t total = (int64_t)m * n * nb;
    const int64_t k = (int64_t)nb * 32;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int b = (int)(i % nb);
        const int64_t j = (i / nb) % n;
        const int t = (int)(i / ((int64_t)nb * n));
        const uint4* wp = reinterpret_cast<const uint4*>(wq + j * k + (int64_t)b * 32);
        const uint4* xp = reinterpret_cast<const uint4*>(xq + t * k + (int64_t)b * 32);
        const uint4 w0 = wp[0], w1 = wp[1], x0 = xp[0], x1 = xp[1];
        const uint32_t wc[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        const uint32_t xc[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        isum[i] = block_dot_i8(wc, xc);
    }
}

hipError_t launch_block_dots(const int8_t* wq, int64_t n, int64_t k, int m, const int8_t* xq,
                             int32_t* isum, const DeviceInfo& dev, hipStream_t stream) {
    const int nb = (int)(k / 32);
    const int64_t total = (int64_t)m * n * nb;
    int64_t grid = (total + 255) / 256;
    const int64_t cap = (int64_t)dev.cu_count * 16;
    if (grid > cap) grid = cap;
    (void)hipGetLastError();
    block_dots_kernel<<<(int)grid, 256, 0, stream>>>(wq, n, nb, m, xq, isum);
    return hipGetLastError();
}

}  // namespace q8
