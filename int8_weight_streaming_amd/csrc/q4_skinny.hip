// q4_skinny.hip -- int4 weights: block quantizer and batch 1..8 decode products.
//
// Format: the Q8_0 block rule with the largest 4-bit magnitude in place of 127.
// A row of K weights is cut into K/32 blocks along the reduction axis; a block
// keeps one binary16 scale d = maxabs / 7 and 32 codes
// clamp(round_half_away(w / d), -7, 7), packed two to a byte as 4-bit two's
// complement: byte j of the block's 16 bytes holds element j in bits 0-3 and
// element j + 16 in bits 4-7.  18 bytes per 32 weights [Frigg README: the
// bytes-per-token table prices an "int4 core + int8 vocab" build, the benchmark
// matrix measures "int4 W / int8 vocab", and "Known limits" reports int4 as
// slower and less accurate than int8 on the page's card; the page names no
// int4 layout].
//
// Products: y[m][j] = sum_b d[j][b] * sum_{i<32} c[j][32b+i] * x[m][32b+i].
//
// Work layout (wave64), as for the Q8_0 decode products: a group of G lanes
// owns R rows; a lane takes whole blocks (16 bytes of codes + the 2-byte scale)
// g, g+G, g+2G, ... so one load instruction of a group reads G*16 contiguous
// bytes of a row.  Per 4-byte word of codes the low nibbles are elements
// 4i..4i+3 of the block and the high nibbles elements 16+4i..16+4i+3, so both
// line up with contiguous activation words.  A nibble is moved to the top of its
// byte ((w << 4) & 0xF0F0F0F0 for the low ones, w & 0xF0F0F0F0 for the high
// ones): each byte then reads as the signed integer 16 * code, which the int8
// routines take as they are; the factor 16 is removed exactly by folding the
// scale as d / 16.
//  * bf16 activations: bytes -> exact bf16 pairs, v_dot2_f32_bf16, one FMA per
//    block and row with d / 16.
//  * Q8 activations: eight v_dot4_i32_i8 give 16 * (exact int32 block sum);
//    one FMA per block and row with (d / 16) * xd.
// Group partials are combined by a fixed DPP tree; no atomics, bitwise
// reproducible.
#include "q8_device.hpp"
#include "q8_internal.hpp"

namespace q8 {

// ------------------------------------------------------------------ quantizer

// One block is handled by 8 consecutive lanes, 4 values each: lanes 0-3 of the
// group hold elements 0..15 (the low nibbles of bytes 0..15), lanes 4-7 hold
// elements 16..31 (the high nibbles of the same bytes).
__global__ __launch_bounds__(256) void q4_quantize_kernel(const float* __restrict__ src, int64_t nblocks,
                                                          uint8_t* __restrict__ q,
                                                          uint16_t* __restrict__ d) {
    const int sub = threadIdx.x & 7;
    const int64_t stride = ((int64_t)gridDim.x * blockDim.x) >> 3;
    for (int64_t b = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3; b < nblocks; b += stride) {
        const float4 f = *reinterpret_cast<const float4*>(src + b * 32 + sub * 4);
        const float v[4] = {f.x, f.y, f.z, f.w};
        float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        a = fmaxf(a, __shfl_xor(a, 1, 8));
        a = fmaxf(a, __shfl_xor(a, 2, 8));
        a = fmaxf(a, __shfl_xor(a, 4, 8));
        // binary16 of the correctly rounded fp32 quotient amax / 7
        const uint16_t sb = __builtin_bit_cast(uint16_t, (_Float16)(a / 7.0f));
        const float s = half_bits_to_float(sb);
        uint32_t nib = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int c = 0;
            if (s != 0.0f) {
                float r = roundf(v[e] / s);          // half away from zero
                r = fminf(fmaxf(r, -7.0f), 7.0f);
                c = (int)r;
            }
            nib |= ((uint32_t)c & 0xFu) << (8 * e);
        }
        const uint32_t upper = __shfl_xor(nib, 4, 8);   // lanes 0-3 receive elements 16..31
        if (sub < 4)
            *reinterpret_cast<uint32_t*>(q + b * 16 + sub * 4) = nib | (upper << 4);
        if (sub == 0) d[b] = sb;
    }
}

hipError_t launch_q4_quantize(const float* w, int64_t nblocks, uint8_t* q, uint16_t* d,
                              const DeviceInfo& dev, hipStream_t stream) {
    const int64_t want = (nblocks * 8 + 255) / 256;
    const int64_t cap = (int64_t)dev.cu_count * 16;
    (void)hipGetLastError();
    q4_quantize_kernel<<<(int)(want < cap ? want : cap), 256, 0, stream>>>(w, nblocks, q, d);
    return hipGetLastError();
}

// ------------------------------------------------------------------ products

// The 32 codes of a word pair, as bytes holding 16 * code: low nibbles of word w
// (elements 4i..4i+3) and its high nibbles (elements 16+4i..16+4i+3).
__device__ __forceinline__ uint32_t q4_low16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t q4_high16(uint32_t w) { return w & 0xF0F0F0F0u; }

// XL = 1 stages each K tile's activations in LDS (shared by the workgroup's
// rows); XL = 0 keeps them in the registers of the lanes that use them.
template <int M, int ACT, int G, int R, int CPL, int XL>
__global__ __launch_bounds__(256) void q4_skinny_kernel(const uint8_t* __restrict__ wq,
                                                        const uint16_t* __restrict__ wd, int64_t n,
                                                        int nb, const void* __restrict__ xv,
                                                        const uint16_t* __restrict__ xdp,
                                                        float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    constexpr int GPW = 64 / G;                  // lane groups per wave
    constexpr int RPW = 4 * GPW * R;             // rows per workgroup
    constexpr int TCH = G * CPL;                 // blocks per K tile
    constexpr bool XREG = XL == 0;
    constexpr int XW = ACT == 0 ? 16 : 8;        // activation words per block and row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gl = lane & (G - 1), grp = lane / G;
    const int64_t k = (int64_t)nb * 32;
    const int64_t rbase = (int64_t)blockIdx.x * RPW + (int64_t)(wave * GPW + grp) * R;

    const uint8_t* wrow[R];
    const uint16_t* srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = rbase + r < n ? rbase + r : n - 1;   // clamp: loads stay in bounds
        wrow[r] = wq + row * (k / 2);
        srow[r] = wd + row * nb;
    }
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    // LDS-staged activations: each thread's 16-byte pieces of a tile (and the
    // Q8 scales) are fetched before the weights and written to LDS once the
    // weight loads are issued (loads return in order: fetched after the
    // weights, writing them would wait for the whole weight tile)
    constexpr int PIECES = XW / 4;               // 16-byte pieces per block and row
    constexpr int XP = XREG ? 1 : (M * TCH * PIECES + 255) / 256;
    constexpr int XS = XREG || ACT == 0 ? 1 : (M * TCH + 255) / 256;
    u32x4 xst[XP];
    uint16_t xsb[XS];
    for (int c0 = 0; c0 < nb; c0 += TCH) {
        const int tch = nb - c0 < TCH ? nb - c0 : TCH;   // blocks in this tile
        const int pieces = M * tch * PIECES;
        if constexpr (!XREG) {
            // unconditional loads, indices past the tile clamped to its last
            // piece (a load under a divergent branch is waited for at once)
#pragma unroll
            for (int u = 0; u < XP; ++u) {
                const int i0 = threadIdx.x + 256 * u;
                const int i = i0 < pieces ? i0 : pieces - 1;
                const int q = i % PIECES, rest = i / PIECES;
                const int ch = rest % tch, m = rest / tch;
                const unsigned char* src = static_cast<const unsigned char*>(xv) +
                    ((int64_t)m * k + (int64_t)(c0 + ch) * 32) * (ACT == 0 ? 2 : 1) + q * 16;
                xst[u] = *reinterpret_cast<const u32x4*>(src);
            }
            if constexpr (ACT == 1) {
#pragma unroll
                for (int u = 0; u < XS; ++u) {
                    const int i0 = threadIdx.x + 256 * u;
                    const int i = i0 < M * tch ? i0 : M * tch - 1;
                    xsb[u] = xdp[(int64_t)(i / tch) * nb + c0 + i % tch];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        uint32_t xr[XREG ? M : 1][XREG ? CPL : 1][XW];
        float xsr[XREG ? M : 1][XREG ? CPL : 1];
        if constexpr (XREG) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = c0 + gl + G * j;
                const int cc = c < nb ? c : 0;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const uint4* p = ACT == 0
                        ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + m * k + (int64_t)cc * 32)
                        : reinterpret_cast<const uint4*>(static_cast<const int8_t*>(xv) + m * k + (int64_t)cc * 32);
#pragma unroll
                    for (int q = 0; q < XW / 4; ++q) {
                        const uint4 a = p[q];
                        xr[m][j][4 * q] = a.x; xr[m][j][4 * q + 1] = a.y;
                        xr[m][j][4 * q + 2] = a.z; xr[m][j][4 * q + 3] = a.w;
                    }
                    if (ACT == 1) xsr[m][j] = half_bits_to_float(xdp[(int64_t)m * nb + cc]);
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
            okj[j] = c < nb;
            const int cc = okj[j] ? c : 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                w[j][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[r] + (int64_t)cc * 16));
                sb[j][r] = srow[r][cc];
            }
        }
        if constexpr (!XREG) {
            // the tile's activations into LDS, [m][block] with XW words each,
            // then the Q8 scales as fp32 (a lane past the tile writes its
            // clamped piece again, with the same bytes)
            __syncthreads();
#pragma unroll
            for (int u = 0; u < XP; ++u) {
                const int i0 = threadIdx.x + 256 * u;
                const int i = i0 < pieces ? i0 : pieces - 1;
                const int q = i % PIECES, rest = i / PIECES;
                const int ch = rest % tch, m = rest / tch;
                *reinterpret_cast<u32x4*>(lds + ((m * TCH + ch) * PIECES + q) * 16) = xst[u];
            }
            if constexpr (ACT == 1) {
                float* sc = reinterpret_cast<float*>(lds + M * TCH * 32);
#pragma unroll
                for (int u = 0; u < XS; ++u) {
                    const int i0 = threadIdx.x + 256 * u;
                    const int i = i0 < M * tch ? i0 : M * tch - 1;
                    sc[(i / tch) * TCH + i % tch] = half_bits_to_float(xsb[u]);
                }
            }
            __syncthreads();
        }
        __builtin_amdgcn_sched_barrier(0);
        float ws[CPL][R];
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r)
                ws[j][r] = okj[j] ? half_bits_to_float(sb[j][r]) * 0.0625f : 0.0f;

#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int cl = gl + G * j;
            const int clc = c0 + cl < nb ? cl : 0;        // LDS slot that exists
            if constexpr (ACT == 0) {
                // bf16 pairs of 16 * code: words 0..7 elements 0..15, 8..15 elements 16..31
                uint32_t wbf[R][16];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t ww[4] = {w[j][r].x, w[j][r].y, w[j][r].z, w[j][r].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        i8x4_to_bf16x4(q4_low16(ww[i]), wbf[r][2 * i], wbf[r][2 * i + 1]);
                        i8x4_to_bf16x4(q4_high16(ww[i]), wbf[r][8 + 2 * i], wbf[r][9 + 2 * i]);
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    uint32_t xc[16];
                    if constexpr (XREG) {
#pragma unroll
                        for (int d = 0; d < 16; ++d) xc[d] = xr[m][j][d];
                    } else {
                        const uint4* xp = reinterpret_cast<const uint4*>(lds + (m * TCH + clc) * 64);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint4 a = xp[q];
                            xc[4 * q] = a.x; xc[4 * q + 1] = a.y; xc[4 * q + 2] = a.z; xc[4 * q + 3] = a.w;
                        }
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float pa = 0.0f, pb = 0.0f;
#pragma unroll
                        for (int d = 0; d < 8; ++d) {
                            pa = dot2_bf16(wbf[r][d], xc[d], pa);
                            pb = dot2_bf16(wbf[r][8 + d], xc[8 + d], pb);
                        }
                        acc[r][m] = fmaf(pa + pb, ws[j][r], acc[r][m]);
                    }
                }
            } else {
                uint32_t lo[R][4], hi[R][4];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t ww[4] = {w[j][r].x, w[j][r].y, w[j][r].z, w[j][r].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        lo[r][i] = q4_low16(ww[i]);
                        hi[r][i] = q4_high16(ww[i]);
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    uint32_t xc[8];
                    float xs;
                    if constexpr (XREG) {
#pragma unroll
                        for (int d = 0; d < 8; ++d) xc[d] = xr[m][j][d];
                        xs = xsr[m][j];
                    } else {
                        const uint4* xp = reinterpret_cast<const uint4*>(lds + (m * TCH + clc) * 32);
                        const uint4 a = xp[0], b = xp[1];
                        xc[0] = a.x; xc[1] = a.y; xc[2] = a.z; xc[3] = a.w;
                        xc[4] = b.x; xc[5] = b.y; xc[6] = b.z; xc[7] = b.w;
                        xs = reinterpret_cast<const float*>(lds + M * TCH * 32)[m * TCH + clc];
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        // 16 * (exact int32 block sum); |.| <= 16 * 32 * 7 * 127
                        int s = 0;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            s = __builtin_amdgcn_sdot4((int)lo[r][i], (int)xc[i], s, false);
                            s = __builtin_amdgcn_sdot4((int)hi[r][i], (int)xc[4 + i], s, false);
                        }
                        acc[r][m] = fmaf((float)s, ws[j][r] * xs, acc[r][m]);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = group_sum<G>(acc[r][m]);

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

template <int M, int ACT, int G, int R, int CPL, int XL>
static hipError_t q4_launch_cfg(const uint8_t* wq, const uint16_t* wd, int64_t n, int nb,
                                const void* x, const uint16_t* xd, float* y, hipStream_t stream) {
    constexpr int RPW = 4 * (64 / G) * R;
    constexpr int TCH = G * CPL;
    size_t lds = 0;
    if (XL) lds = ACT == 0 ? (size_t)M * TCH * 64 : (size_t)M * TCH * 32 + (size_t)M * TCH * 4;
    const int64_t grid = (n + RPW - 1) / RPW;
    q4_skinny_kernel<M, ACT, G, R, CPL, XL><<<(unsigned)grid, 256, lds, stream>>>(wq, wd, n, nb, x, xd, y);
    return hipGetLastError();
}

// Configurations measured on the Mimir shapes and the 262144 x 1536 lm_head
// (graph replay, weights rotated past the caches, batch 1, 2, 4 and 8).  The
// bf16 form is bound by its arithmetic (unpack, convert, dot), so lane
// occupancy decides more than for the Q8_0 products:
//  * at least 4 workgroups of 64 rows per compute unit: 16-lane groups; at
//    batch 1 two rows each and 16-block K tiles (bf16) or 48-block tiles
//    (Q8); above that four rows each with the activation tile in LDS;
//  * from half a workgroup of 32 rows per compute unit: 16-lane groups of
//    two rows, 48-block tiles (K = 1536 in one tile);
//  * shorter matrices: one row per 32-lane group, 64-block tiles; for K
//    above 2048 at batch 1-2 a 128-block tile, above that one wave per row
//    with 128-block tiles staged in LDS.
Q4Layout q4_layout(int64_t n, int64_t k, int m, int act, int cu_count) {
    const int64_t nb = k / 32;
    if ((n + 63) / 64 >= 4 * (int64_t)cu_count) {
        if (m == 1) return act == 0 ? Q4Layout{16, 2, 1, 0} : Q4Layout{16, 2, 3, 0};
        return {16, 4, 3, 1};
    }
    if (2 * ((n + 31) / 32) >= (int64_t)cu_count) return {16, 2, 3, m > 2};
    if (nb <= 64) return {32, 1, 2, m > 2};
    if (m <= 2) return {32, 1, 4, 0};
    return {64, 1, 2, 1};
}

template <int M, int ACT>
static hipError_t q4_launch_m(const uint8_t* wq, const uint16_t* wd, int64_t n, int nb,
                              const void* x, const uint16_t* xd, float* y,
                              const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
    const Q4Layout L = q4_layout(n, (int64_t)nb * 32, M, ACT, dev.cu_count);
    if (L.g == 16 && L.r == 2 && L.cpl == 1) {
        if constexpr (M == 1 && ACT == 0) return q4_launch_cfg<M, ACT, 16, 2, 1, 0>(wq, wd, n, nb, x, xd, y, stream);
    } else if (L.g == 16 && L.r == 2 && L.cpl == 3 && L.xl == 0) {
        if constexpr (M <= 2) return q4_launch_cfg<M, ACT, 16, 2, 3, 0>(wq, wd, n, nb, x, xd, y, stream);
    } else if (L.g == 16 && L.r == 2 && L.cpl == 3) {
        if constexpr (M > 2) return q4_launch_cfg<M, ACT, 16, 2, 3, 1>(wq, wd, n, nb, x, xd, y, stream);
    } else if (L.g == 16 && L.r == 4) {
        if constexpr (M > 1) return q4_launch_cfg<M, ACT, 16, 4, 3, 1>(wq, wd, n, nb, x, xd, y, stream);
    } else if (L.g == 32 && L.cpl == 2) {
        return q4_launch_cfg<M, ACT, 32, 1, 2, (M > 2)>(wq, wd, n, nb, x, xd, y, stream);
    } else if (L.g == 32 && L.cpl == 4) {
        if constexpr (M <= 2) return q4_launch_cfg<M, ACT, 32, 1, 4, 0>(wq, wd, n, nb, x, xd, y, stream);
    } else if (L.g == 64) {
        if constexpr (M > 2) return q4_launch_cfg<M, ACT, 64, 1, 2, 1>(wq, wd, n, nb, x, xd, y, stream);
    }
    return hipErrorInvalidValue;                 // no layout is chosen outside the cases above
}

template <int ACT>
static hipError_t q4_launch_act(const uint8_t* wq, const uint16_t* wd, int64_t n, int nb, int m,
                                const void* x, const uint16_t* xd, float* y,
                                const DeviceInfo& dev, hipStream_t stream) {
    switch (m) {
        case 1: return q4_launch_m<1, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 2: return q4_launch_m<2, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 3: return q4_launch_m<3, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 4: return q4_launch_m<4, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 5: return q4_launch_m<5, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 6: return q4_launch_m<6, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 7: return q4_launch_m<7, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        case 8: return q4_launch_m<8, ACT>(wq, wd, n, nb, x, xd, y, dev, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_q4_skinny(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m,
                            int act, const void* x, const uint16_t* xd, float* y,
                            const DeviceInfo& dev, hipStream_t stream) {
    const int nb = (int)(k / 32);
    if (act == 0 && q4_mfma_applies(n, k, m, dev.cu_count)) return launch_q4_mfma(wq, wd, n, k, m, x, y, dev, stream);
    if (act == 0) return q4_launch_act<0>(wq, wd, n, nb, m, x, xd, y, dev, stream);
    return q4_launch_act<1>(wq, wd, n, nb, m, x, xd, y, dev, stream);
}

}  // namespace q8
