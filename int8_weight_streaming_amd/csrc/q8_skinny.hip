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
//  * A lane group of G lanes (G = 16 or 64) owns R weight rows at a time.
//    Lane g of the group takes the 32-element blocks g, g+G, g+2G, ... of those
//    rows, loading each block as two 16-byte loads, so one group load
//    instruction reads G*16 contiguous bytes of a row and every byte of a weight
//    row is read once.
//  * The activation rows are staged once per workgroup in LDS (80-byte stride
//    per bf16 block, 48-byte stride per int8 block, so 16-byte reads of
//    consecutive blocks hit distinct banks), and every block read from LDS
//    serves all R rows.
//  * bf16 activations (W8A16): the int8 codes are converted exactly to packed
//    bf16 pairs and multiplied with v_dot2_f32_bf16 (fp32 accumulate); each
//    block's partial is folded with its scale by one FMA.
//  * Q8 activations: the exact int32 block sum comes from eight v_dot4_i32_i8,
//    is converted to fp32 and folded with wd*xd [fak MODEL-BASELINE-RESULTS,
//    ACT 4 "How the GEMM was closed": deferred reduction, one fold per block].
//  * The partial sums of a group are combined by a fixed DPP tree (no atomics,
//    no cross-workgroup split), so every output is written by exactly one group
//    and results are bitwise reproducible [Frigg README, Finding 8: a partials
//    buffer instead of atomics keeps graph replay bit-identical].
#include "q8_device.hpp"
#include "q8_internal.hpp"

namespace q8 {

constexpr int kStrideBf16 = 80;   // bytes per (row, block) of staged bf16 activations
constexpr int kStrideQ8 = 48;     // bytes per (row, block) of staged int8 codes
constexpr int kLdsBudget = 48 * 1024;

template <int M, int ACT>
__device__ __forceinline__ void stage_act(unsigned char* lds, const void* xv, const uint16_t* xdp,
                                          int64_t k, int nb, int b0, int nblk, int kt) {
    if (ACT == 0) {
        const uint16_t* x = static_cast<const uint16_t*>(xv);
        const int pieces = M * nblk * 4;
        for (int i = threadIdx.x; i < pieces; i += blockDim.x) {
            const int q = i & 3, rest = i >> 2;
            const int blk = rest % nblk, m = rest / nblk;
            const uint4 v = *reinterpret_cast<const uint4*>(x + m * k + (int64_t)(b0 + blk) * 32 + q * 8);
            *reinterpret_cast<uint4*>(lds + (m * kt + blk) * kStrideBf16 + q * 16) = v;
        }
    } else {
        const int8_t* x = static_cast<const int8_t*>(xv);
        const int pieces = M * nblk * 2;
        for (int i = threadIdx.x; i < pieces; i += blockDim.x) {
            const int q = i & 1, rest = i >> 1;
            const int blk = rest % nblk, m = rest / nblk;
            const uint4 v = *reinterpret_cast<const uint4*>(x + m * k + (int64_t)(b0 + blk) * 32 + q * 16);
            *reinterpret_cast<uint4*>(lds + (m * kt + blk) * kStrideQ8 + q * 16) = v;
        }
        float* sc = reinterpret_cast<float*>(lds + M * kt * kStrideQ8);
        for (int i = threadIdx.x; i < M * nblk; i += blockDim.x) {
            const int blk = i % nblk, m = i / nblk;
            sc[m * kt + blk] = half_bits_to_float(xdp[(int64_t)m * nb + b0 + blk]);
        }
    }
}

template <int M, int ACT, int G, int R, int U>
__global__ __launch_bounds__(256) void skinny_kernel(const int8_t* __restrict__ wq,
                                                     const uint16_t* __restrict__ wd, int64_t n,
                                                     int nb, const void* __restrict__ xv,
                                                     const uint16_t* __restrict__ xdp,
                                                     float* __restrict__ y, int kt,
                                                     int64_t n_row_tiles) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    constexpr int GPW = 64 / G;          // lane groups per wave
    constexpr int RPW = 4 * GPW * R;     // rows per workgroup tile
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gl = lane & (G - 1), grp = lane / G;
    const int ntiles = (nb + kt - 1) / kt;
    const int64_t k = (int64_t)nb * 32;

    for (int64_t rt = blockIdx.x; rt < n_row_tiles; rt += gridDim.x) {
        const int64_t rbase = rt * RPW + (int64_t)(wave * GPW + grp) * R;
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

        for (int t = 0; t < ntiles; ++t) {
            const int b0 = t * kt;
            const int nblk = nb - b0 < kt ? nb - b0 : kt;
            if (ntiles > 1 || rt == (int64_t)blockIdx.x) {
                __syncthreads();
                stage_act<M, ACT>(lds, xv, xdp, k, nb, b0, nblk, kt);
                __syncthreads();
            }
            for (int bl = gl; bl < nblk; bl += G * U) {
                u32x4 wa[U][R], wb[U][R];
                float ws[U][R];
                bool ok[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    ok[u] = bl + u * G < nblk;
                    const int bg = b0 + (ok[u] ? bl + u * G : bl);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const u32x4* p = reinterpret_cast<const u32x4*>(wrow[r] + (int64_t)bg * 32);
                        wa[u][r] = __builtin_nontemporal_load(p);
                        wb[u][r] = __builtin_nontemporal_load(p + 1);
                        ws[u][r] = half_bits_to_float(srow[r][bg]);
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!ok[u]) continue;
                    const int blu = bl + u * G;
                    if (ACT == 0) {
                        uint32_t wbf[R][16];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const uint32_t wv[8] = {wa[u][r].x, wa[u][r].y, wa[u][r].z, wa[u][r].w,
                                                    wb[u][r].x, wb[u][r].y, wb[u][r].z, wb[u][r].w};
#pragma unroll
                            for (int d = 0; d < 8; ++d) i8x4_to_bf16x4(wv[d], wbf[r][2 * d], wbf[r][2 * d + 1]);
                        }
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            const uint4* xp = reinterpret_cast<const uint4*>(lds + (m * kt + blu) * kStrideBf16);
                            const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
                            const uint32_t xv2[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                                      x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                float pa = 0.0f, pb = 0.0f;
#pragma unroll
                                for (int d = 0; d < 8; ++d) {
                                    pa = dot2_bf16(wbf[r][d], xv2[d], pa);
                                    pb = dot2_bf16(wbf[r][8 + d], xv2[8 + d], pb);
                                }
                                acc[r][m] = fmaf(pa + pb, ws[u][r], acc[r][m]);
                            }
                        }
                    } else {
                        const float* sc = reinterpret_cast<const float*>(lds + M * kt * kStrideQ8);
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            const uint4* xp = reinterpret_cast<const uint4*>(lds + (m * kt + blu) * kStrideQ8);
                            const uint4 x0 = xp[0], x1 = xp[1];
                            const uint32_t xc[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                            const float xs = sc[m * kt + blu];
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                const uint32_t wc[8] = {wa[u][r].x, wa[u][r].y, wa[u][r].z, wa[u][r].w,
                                                        wb[u][r].x, wb[u][r].y, wb[u][r].z, wb[u][r].w};
                                const int isum = block_dot_i8(wc, xc);
                                acc[r][m] = fmaf((float)isum, ws[u][r] * xs, acc[r][m]);
                            }
                        }
                    }
                }
            }
        }

        // Combine the G partial sums of every (row, m); all lanes of the group
        // end with the same value.
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = group_sum<G>(acc[r][m]);

        // Lane g of the group stores value g (then g + G, ...): rows of one m
        // land on consecutive lanes, so the stores coalesce.
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
}

// ------------------------------------------------------------------ launch

template <int M, int ACT>
static hipError_t launch_m(const int8_t* wq, const uint16_t* wd, int64_t n, int nb,
                           const void* x, const uint16_t* xd, float* y,
                           const DeviceInfo& dev, hipStream_t stream) {
    const int per_block = ACT == 0 ? M * kStrideBf16 : M * (kStrideQ8 + 4);
    int kt = kLdsBudget / per_block;
    if (kt > nb) kt = nb;
    const size_t lds = (size_t)kt * per_block;
    const int64_t cap = (int64_t)dev.cu_count * 8;
    // Large outputs: 16-lane groups, 4 rows each (64 rows per workgroup).
    // Small outputs: one wave per row, so that even a 1536-row matrix spreads
    // over all compute units.
    const int64_t tiles_big = (n + 63) / 64;
    (void)hipGetLastError();
    if (tiles_big >= 2 * (int64_t)dev.cu_count) {
        const int64_t grid = tiles_big < cap ? tiles_big : cap;
        skinny_kernel<M, ACT, 16, 4, 2><<<(int)grid, 256, lds, stream>>>(wq, wd, n, nb, x, xd, y, kt, tiles_big);
    } else {
        const int64_t tiles = (n + 3) / 4;
        const int64_t grid = tiles < cap ? tiles : cap;
        skinny_kernel<M, ACT, 64, 1, 2><<<(int)grid, 256, lds, stream>>>(wq, wd, n, nb, x, xd, y, kt, tiles);
    }
    return hipGetLastError();
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

// isum[t][j][b] for t < m: one thread per (t, j, b), the same block-dot routine
// as the Q8-activation products above.
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
