// q8_prefill_frag.hip -- Q8 x Q8 prefill product on operands stored in the
// int8 matrix core's fragment order.
//
//   y[t][j] = sum_b wd[j][b] * xd[t][b] * isum[t][j][b],
//   isum[t][j][b] = sum_{i<32} wq[j][32b+i] * xq[t][32b+i]  (exact int32)
//
// [fak MODEL-BASELINE-RESULTS, ACT 4, "How the GEMM was closed": keep each
// block's int32 sum and fold it once into a float accumulator; register-block
// the output so every loaded block serves several outputs.]
//
// Fragment order.  One v_mfma_i32_32x32x32_i8 takes, per lane (i, h) = (lane %
// 32, lane / 32), the 16 bytes 16h .. 16h + 15 of one 32-element block of
// operand row i.  A Q8_0 matrix is stored so that those 64 x 16 bytes are one
// contiguous kilobyte per 32-row tile and block:
//
//   codes  [rows64 / 32][nbp][64 lanes][16 B]   lane (i, h) of (tile t, block b)
//          holds codes 32b + 16h .. + 15 of row 32t + i,
//   scales [rows64 / 32][nbp / 4][32 rows][4]   the binary16 scales of row
//          32t + i, blocks 4g .. 4g + 3,
//
// rows64 = rows rounded up to 64 and nbp = K/32 rounded up to 4; padding rows
// and blocks hold zero codes and zero scales.  A wave then loads each operand
// fragment with one fully coalesced 16-byte load per lane straight into the
// registers the matrix core reads, with no LDS round trip: the row-major
// kernels stage every operand through LDS, and at the matrix core's rate that
// staging alone would take the whole LDS bandwidth of a compute unit.  The
// activation side is packed per call (q8_pack_frag on the quantized rows); the
// weights once, next to their row-major copy.
//
// Kernel.  A wave owns a 32 (tokens) x 32*WN (weight rows) output tile over a
// contiguous range of K steps (four blocks each); KS waves share a tile and
// their partial tiles are added through LDS in wave order, so results are
// bitwise reproducible.  Per block: the int8 product (exact int32 sums), the
// scale outer product xd (x) wd on the f16 matrix core (exact: a product of two
// binary16 numbers needs at most 22 bits), and the fold acc += float(isum) *
// scale on the vector ALUs.  Only one product pair is in flight and the
// operand registers of a block are refilled with the next step's block as
// soon as its products are issued, which keeps the kernel at <= 128 VGPRs
// (WN = 1: four waves per SIMD) or <= 168 (WN = 2: three); the matrix core and
// the vector ALUs of a SIMD co-issue across those waves.  Workgroups are dealt
// to the eight XCDs (workgroup id % 8) by column ranges of the weights and walk
// their tiles token-major, so each XCD's L2 holds its weight columns and
// fetches every activation tile once.  Long prompts take a 64 x 64 form of the
// same loop (prefill_frag64_kernel: two token tiles per wave).
#include "q8_device.hpp"
#include "q8_internal.hpp"

#include <type_traits>

namespace q8 {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ packing

// One thread per 16-byte code chunk of the fragment array, then one per
// 8-byte scale group.  Rows and blocks past the matrix are written as zeros.
__global__ __launch_bounds__(256) void pack_frag_kernel(const int8_t* __restrict__ q,
                                                        const uint16_t* __restrict__ d, int64_t rows,
                                                        int nb, int nbp, int64_t tiles,
                                                        int8_t* __restrict__ qf, uint16_t* __restrict__ df) {
    const int64_t nchunk = tiles * nbp * 64;
    const int64_t ngroup = tiles * (nbp / 4) * 32;
    const int64_t k = (int64_t)nb * 32;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < nchunk + ngroup;
         e += (int64_t)gridDim.x * 256) {
        if (e < nchunk) {
            const int lane = (int)(e & 63);
            const int64_t tb = e >> 6;
            const int b = (int)(tb % nbp);
            const int64_t row = (tb / nbp) * 32 + (lane & 31);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row < rows && b < nb)
                v = *reinterpret_cast<const u32x4*>(q + row * k + (int64_t)b * 32 + 16 * (lane >> 5));
            *reinterpret_cast<u32x4*>(qf + e * 16) = v;
        } else {
            const int64_t g = e - nchunk;
            const int i = (int)(g & 31);
            const int64_t tg = g >> 5;
            const int grp = (int)(tg % (nbp / 4));
            const int64_t row = (tg / (nbp / 4)) * 32 + i;
            uint16_t s[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int b = 4 * grp + u;
                s[u] = row < rows && b < nb ? d[row * nb + b] : (uint16_t)0;
            }
            const uint2 w = make_uint2((uint32_t)s[0] | ((uint32_t)s[1] << 16),
                                       (uint32_t)s[2] | ((uint32_t)s[3] << 16));
            *reinterpret_cast<uint2*>(df + g * 4) = w;
        }
    }
}

// ------------------------------------------------------------------ product

template <int KS>
constexpr int frag_waves() { return KS > 4 ? KS : 4; }

constexpr int kFoldBias = 0x4B400000;        // binary32 bits of 1.5 * 2^23
constexpr float kFoldBiasF = 12582912.0f;    // 1.5 * 2^23

template <int WN, int KS>
__global__ __launch_bounds__(64 * frag_waves<KS>())
__attribute__((amdgpu_waves_per_eu(WN == 1 ? 4 : 3, WN == 1 ? 4 : 3)))
void prefill_frag_kernel(const i32x4* __restrict__ wf, const i32x2* __restrict__ wsf, int64_t n,
                         int nbp, int64_t p, const i32x4* __restrict__ xf, const i32x2* __restrict__ xsf,
                         float* __restrict__ y) {
    constexpr int W = frag_waves<KS>();
    constexpr int T = W / KS;                        // output tiles per workgroup
    __shared__ __attribute__((aligned(16))) float red[KS > 1 ? W * WN * 16 * 64 : 4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int ntn = (int)((n + 31) / 32), ntp = (int)((p + 31) / 32);
    const int ntw = (ntn + WN - 1) / WN;             // wave columns of WN weight tiles
    const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
    const int c0 = (int)((int64_t)ntw * xcd / 8), nc = (int)((int64_t)ntw * (xcd + 1) / 8) - c0;
    const int tile = jw * T + wave / KS;
    const bool live = nc > 0 && tile < nc * ntp;
    const int tp = live ? tile / nc : 0;
    const int tn0 = live ? (c0 + tile % nc) * WN : 0;
    const int kw = wave % KS;
    const int SS = nbp / 4;                          // four-block steps over K
    const int s_lo = (int)((int64_t)SS * kw / KS), S = (int)((int64_t)SS * (kw + 1) / KS) - s_lo;
    const int i = lane & 31, h = lane >> 5;

    float acc[WN][16];
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;

    if (live && S > 0) {
        // Buffer descriptors over this wave's tiles (all of K); a block is
        // addressed by the scalar offset of its kilobyte, a step's scales by
        // the scalar offset of their 256 bytes, so load addresses cost no
        // vector instructions.
        const char* xb = reinterpret_cast<const char*>(xf);
        const char* wb = reinterpret_cast<const char*>(wf);
        const char* xsb = reinterpret_cast<const char*>(xsf);
        const char* wsb = reinterpret_cast<const char*>(wsf);
        const __amdgpu_buffer_rsrc_t ra = range_rsrc32(xb + (int64_t)tp * nbp * 1024, nbp * 1024);
        const __amdgpu_buffer_rsrc_t rsa = range_rsrc32(xsb + (int64_t)tp * SS * 256, SS * 256);
        __amdgpu_buffer_rsrc_t rb[WN], rsb[WN];
#pragma unroll
        for (int b = 0; b < WN; ++b) {
            rb[b] = range_rsrc32(wb + (int64_t)(tn0 + b) * nbp * 1024, nbp * 1024);
            rsb[b] = range_rsrc32(wsb + (int64_t)(tn0 + b) * SS * 256, SS * 256);
        }
        const int vo = lane * 16, vs = i * 8;
        auto ld_code = [&](__amdgpu_buffer_rsrc_t r, int blk) {
            return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, blk * 1024, 0));
        };
        auto ld_scale = [&](__amdgpu_buffer_rsrc_t r, int st) {
            return __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, vs, st * 256, 0));
        };
        // The int8 product accumulates onto the bit pattern of 1.5 * 2^23: a
        // block sum S has |S| <= 32 * 128 * 128 < 2^22, so the int32 result's
        // bits read as a binary32 number are exactly 1.5 * 2^23 + S, and one
        // exact subtraction gives float(S) -- an add issues faster than the
        // int-to-float conversion it replaces, and the fold is bit for bit
        // the same.
        i32x16 cb;
#pragma unroll
        for (int r = 0; r < 16; ++r) cb[r] = kFoldBias;
        asm volatile("" : "+v"(cb));
        const f32x16 zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // The scales go out before the codes, in the order a step issues its
        // loads, so the wait for them at the head of the step loop leaves the
        // code loads of the step in flight.
        i32x4 a[4], bw[WN][4];
        i32x2 sa, sb[WN], sa_n = {0, 0}, sb_n[WN];
        sa = ld_scale(rsa, s_lo);
#pragma unroll
        for (int b = 0; b < WN; ++b) {
            sb[b] = ld_scale(rsb[b], s_lo);
            sb_n[b] = (i32x2){0, 0};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = ld_code(ra, 4 * s_lo + u);
#pragma unroll
            for (int b = 0; b < WN; ++b) bw[b][u] = ld_code(rb[b], 4 * s_lo + u);
        }

        // One four-block step; with REFILL the next step's scales are fetched
        // first and each block's operand registers are reloaded with the next
        // step's block as soon as its products are issued.
        auto step = [&](int s, auto refill_tag) {
            constexpr bool REFILL = decltype(refill_tag)::value;
            const int gs = s_lo + s;
            if constexpr (REFILL) {
                sa_n = ld_scale(rsa, gs + 1);
#pragma unroll
                for (int b = 0; b < WN; ++b) sb_n[b] = ld_scale(rsb[b], gs + 1);
            }
            // Scale operands: the weight side holds its four blocks' scales in
            // k = 0..3 (lanes 32..63, k = 8..11, meet zeros); the activation
            // side block u's scale in k = u on lanes 0..31 only, built once per
            // block for all WN weight tiles; the single nonzero product is
            // xd_u * wd_u.
            i32x4 stb[WN];
#pragma unroll
            for (int b = 0; b < WN; ++b) stb[b] = (i32x4){sb[b][0], sb[b][1], 0, 0};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int xw = (u >> 1) ? sa[1] : sa[0];
                const int half = (u & 1) ? (xw & (int)0xFFFF0000u) : (xw & 0xFFFF);
                const int hv = h ? 0 : half;
                const i32x4 sta = {(u >> 1) ? 0 : hv, (u >> 1) ? hv : 0, 0, 0};
#pragma unroll
                for (int b = 0; b < WN; ++b) {
                    const i32x16 c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[u], bw[b][u], cb, 0, 0, 0);
                    const f32x16 t = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(f16x8, sta), __builtin_bit_cast(f16x8, stb[b]), zf, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (REFILL) {
                        if (b == WN - 1) {
                            a[u] = ld_code(ra, 4 * (gs + 1) + u);
#pragma unroll
                            for (int b2 = 0; b2 < WN; ++b2) bw[b2][u] = ld_code(rb[b2], 4 * (gs + 1) + u);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[b][r] = fmaf(__int_as_float(c[r]) - kFoldBiasF, t[r], acc[b][r]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (REFILL) {
                sa = sa_n;
#pragma unroll
                for (int b = 0; b < WN; ++b) sb[b] = sb_n[b];
            }
        };
        for (int s = 0; s + 1 < S; ++s) step(s, std::true_type{});
        step(S - 1, std::false_type{});
    }

    // Result r of lane (i, h) is row 8 (r / 4) + 4 h + r % 4 of the tile and
    // column i of weight tile tn0 + b.  A quad q holds results 4q .. 4q + 3
    // (rows 8q + 4h .. + 3).  Whole tiles store unguarded through one base
    // pointer per lane; ragged ones check rows and columns.
    const int64_t prow0 = (int64_t)tp * 32 + 4 * h;
    const bool full = (int64_t)(tp + 1) * 32 <= p && (int64_t)(tn0 + WN) * 32 <= n;
    float* const ybase = y + prow0 * n + (int64_t)tn0 * 32 + i;
    auto store_quad = [&](int b, int q, const float4& v) {
        float* yq = ybase + (int64_t)(8 * q) * n + 32 * b;
        if (full) {
            yq[0] = v.x;
            yq[n] = v.y;
            yq[2 * n] = v.z;
            yq[3 * n] = v.w;
        } else {
            const int64_t row = prow0 + 8 * q, col = (int64_t)(tn0 + b) * 32 + i;
            if (col < n) {
                if (row < p) yq[0] = v.x;
                if (row + 1 < p) yq[n] = v.y;
                if (row + 2 < p) yq[2 * n] = v.z;
                if (row + 3 < p) yq[3 * n] = v.w;
            }
        }
    };
    if constexpr (KS > 1) {
        // every wave leaves its partial tile in LDS as 16-byte records
        // [wave][b][q][lane]; the (b, q) items are dealt over the KS waves of
        // the tile, and each sums its items' KS partials in wave order
        float4* red4 = reinterpret_cast<float4*>(red);
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red4[((wave * WN + b) * 4 + q) * 64 + lane] =
                    make_float4(acc[b][4 * q], acc[b][4 * q + 1], acc[b][4 * q + 2], acc[b][4 * q + 3]);
        __syncthreads();
        if (live) {
            const int w0 = wave - kw;                      // first wave of this tile
            for (int item = kw; item < 4 * WN; item += KS) {
                const int b = item >> 2, q = item & 3;
                float4 v = red4[((w0 * WN + b) * 4 + q) * 64 + lane];
                for (int w = 1; w < KS; ++w) {
                    const float4 u = red4[(((w0 + w) * WN + b) * 4 + q) * 64 + lane];
                    v.x += u.x;
                    v.y += u.y;
                    v.z += u.z;
                    v.w += u.w;
                }
                store_quad(b, q, v);
            }
        }
    } else if (live) {
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store_quad(b, q, make_float4(acc[b][4 * q], acc[b][4 * q + 1], acc[b][4 * q + 2], acc[b][4 * q + 3]));
    }
}


// The 64 x 64 form for long prompts: a wave owns two token tiles x two weight
// tiles over all of K, so each block's four operand loads serve four
// block-tiles (one load per block-tile against 1.5 for the 32 x 64 tile).  The
// operand registers hold two blocks (a block's registers are reloaded with the
// block two ahead as soon as its last product pair is issued) and the fold
// converts the int32 sums directly (the biased accumulator's 16 registers would
// push the kernel past three waves per SIMD); per output the fold order is the
// 32 x 64 kernel's with K whole, so the results are the same bits.  Workgroups
// of four waves, 4 / KS tiles of 64 x 64, dealt to XCDs by weight columns as
// above.  With KS = 2 the two waves of a tile take half of K each; wave kw
// stores token tile kw, taking the other wave's partial sums of it through LDS
// and adding the two in wave order.
template <int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void prefill_frag64_kernel(const i32x4* __restrict__ wf, const i32x2* __restrict__ wsf, int64_t n, int nbp,
                           int64_t p, const i32x4* __restrict__ xf, const i32x2* __restrict__ xsf,
                           float* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int ntn = (int)((n + 31) / 32), ntp = (int)((p + 31) / 32);
    const int ntw = (ntn + 1) / 2, ntq = (ntp + 1) / 2;   // wave columns and rows of tile pairs
    const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
    const int c0 = (int)((int64_t)ntw * xcd / 8), nc = (int)((int64_t)ntw * (xcd + 1) / 8) - c0;
    const int tile = jw * (4 / KS) + wave / KS;
    const bool live = nc > 0 && tile < nc * ntq;
    // the second tile of a pair exists in the padded fragment arrays (rows64)
    const int tp0 = live ? (tile / nc) * 2 : 0;
    const int tn0 = live ? (c0 + tile % nc) * 2 : 0;
    const int kw = wave % KS;
    const int SS = nbp / 4;                          // four-block steps over K
    const int s_lo = SS * kw / KS, S = SS * (kw + 1) / KS - s_lo;
    const int i = lane & 31, h = lane >> 5;

    float acc[2][2][16];                                  // [token tile][weight tile]
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[pp][b][r] = 0.0f;

    if (live && S > 0) {
        const char* xb = reinterpret_cast<const char*>(xf);
        const char* wb = reinterpret_cast<const char*>(wf);
        const char* xsb = reinterpret_cast<const char*>(xsf);
        const char* wsb = reinterpret_cast<const char*>(wsf);
        __amdgpu_buffer_rsrc_t ra[2], rsa[2], rb[2], rsb[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            ra[q] = range_rsrc32(xb + (int64_t)(tp0 + q) * nbp * 1024, nbp * 1024);
            rsa[q] = range_rsrc32(xsb + (int64_t)(tp0 + q) * SS * 256, SS * 256);
            rb[q] = range_rsrc32(wb + (int64_t)(tn0 + q) * nbp * 1024, nbp * 1024);
            rsb[q] = range_rsrc32(wsb + (int64_t)(tn0 + q) * SS * 256, SS * 256);
        }
        const int vo = lane * 16, vs = i * 8;
        auto ld_code = [&](__amdgpu_buffer_rsrc_t r, int blk) {
            return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, blk * 1024, 0));
        };
        auto ld_scale = [&](__amdgpu_buffer_rsrc_t r, int st) {
            return __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, vs, st * 256, 0));
        };
        const i32x16 zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        const f32x16 zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // operand registers of two blocks (slot = block % 2), scales of one step;
        // the scales go out first
        i32x4 a[2][2], bw[2][2];
        i32x2 sa[2], sb[2], sa_n[2], sb_n[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            sa[q] = ld_scale(rsa[q], s_lo);
            sb[q] = ld_scale(rsb[q], s_lo);
            sa_n[q] = (i32x2){0, 0};
            sb_n[q] = (i32x2){0, 0};
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                a[q][u] = ld_code(ra[q], 4 * s_lo + u);
                bw[q][u] = ld_code(rb[q], 4 * s_lo + u);
            }
        auto step = [&](int gs, auto refill_tag) {
            constexpr bool REFILL = decltype(refill_tag)::value;
            if constexpr (REFILL) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    sa_n[q] = ld_scale(rsa[q], gs + 1);
                    sb_n[q] = ld_scale(rsb[q], gs + 1);
                }
            }
            // scale operands as in prefill_frag_kernel
            i32x4 stb[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) stb[b] = (i32x4){sb[b][0], sb[b][1], 0, 0};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const int xw = (u >> 1) ? sa[pp][1] : sa[pp][0];
                    const int half = (u & 1) ? (xw & (int)0xFFFF0000u) : (xw & 0xFFFF);
                    const int hv = h ? 0 : half;
                    const i32x4 sta = {(u >> 1) ? 0 : hv, (u >> 1) ? hv : 0, 0, 0};
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const i32x16 c =
                            __builtin_amdgcn_mfma_i32_32x32x32_i8(a[pp][u & 1], bw[b][u & 1], zi, 0, 0, 0);
                        const f32x16 t = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8, sta), __builtin_bit_cast(f16x8, stb[b]), zf, 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                        if (pp == 1 && b == 1 && (REFILL || u < 2)) {     // the block two ahead
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                a[q][u & 1] = ld_code(ra[q], 4 * gs + u + 2);
                                bw[q][u & 1] = ld_code(rb[q], 4 * gs + u + 2);
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[pp][b][r] = fmaf((float)c[r], t[r], acc[pp][b][r]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            if constexpr (REFILL) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    sa[q] = sa_n[q];
                    sb[q] = sb_n[q];
                }
            }
        };
        for (int s = s_lo; s + 1 < s_lo + S; ++s) step(s, std::true_type{});
        step(s_lo + S - 1, std::false_type{});
    }

    if constexpr (KS == 2) {
        // wave kw hands its partial sums of token tile 1 - kw to the other wave
        __shared__ __attribute__((aligned(16))) float4 part[4][2][4][64];   // [wave][b][q][lane]
        auto put = [&](const float (&t)[2][16]) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    part[wave][b][q][lane] = make_float4(t[b][4 * q], t[b][4 * q + 1], t[b][4 * q + 2], t[b][4 * q + 3]);
        };
        if (kw == 0)
            put(acc[1]);
        else
            put(acc[0]);
        __syncthreads();
        // token tile kw: the partial of wave 0 first, then that of wave 1
        auto add = [&](float (&t)[2][16], bool first) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 o = part[wave ^ 1][b][q][lane];
                    const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        t[b][4 * q + e] = first ? t[b][4 * q + e] + ov[e] : ov[e] + t[b][4 * q + e];
                }
        };
        if (kw == 0)
            add(acc[0], true);
        else
            add(acc[1], false);
    }

    // stores as in prefill_frag_kernel, per token tile (wave kw of a split
    // stores token tile kw)
    if (live) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            if (KS == 2 && pp != kw) continue;
            const int64_t prow0 = (int64_t)(tp0 + pp) * 32 + 4 * h;
            const bool full = (int64_t)(tp0 + pp + 1) * 32 <= p && (int64_t)(tn0 + 2) * 32 <= n;
            float* const ybase = y + prow0 * n + (int64_t)tn0 * 32 + i;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float* yq = ybase + (int64_t)(8 * q) * n + 32 * b;
                    const float v0 = acc[pp][b][4 * q], v1 = acc[pp][b][4 * q + 1];
                    const float v2 = acc[pp][b][4 * q + 2], v3 = acc[pp][b][4 * q + 3];
                    if (full) {
                        yq[0] = v0;
                        yq[n] = v1;
                        yq[2 * n] = v2;
                        yq[3 * n] = v3;
                    } else {
                        const int64_t row = prow0 + 8 * q, col = (int64_t)(tn0 + b) * 32 + i;
                        if (col < n) {
                            if (row < p) yq[0] = v0;
                            if (row + 1 < p) yq[n] = v1;
                            if (row + 2 < p) yq[2 * n] = v2;
                            if (row + 3 < p) yq[3 * n] = v3;
                        }
                    }
                }
        }
    }
}

template <int WN, int KS>
hipError_t launch_frag_cfg(const int8_t* wf, const uint16_t* wsf, int64_t n, int64_t k, int64_t p,
                           const int8_t* xf, const uint16_t* xsf, float* y, int64_t grid, hipStream_t stream) {
    constexpr int W = frag_waves<KS>();
    const int nbp = (int)frag_blocks(k);
    prefill_frag_kernel<WN, KS><<<(unsigned)grid, 64 * W, 0, stream>>>(
        reinterpret_cast<const i32x4*>(wf), reinterpret_cast<const i32x2*>(wsf), n, nbp, p,
        reinterpret_cast<const i32x4*>(xf), reinterpret_cast<const i32x2*>(xsf), y);
    return hipGetLastError();
}

}  // namespace

int64_t frag_rows(int64_t rows) { return (rows + 63) / 64 * 64; }
int64_t frag_blocks(int64_t k) { return (k / 32 + 3) / 4 * 4; }

// Tile shape and K split, from sweeps of the Mimir shapes at P = 128 .. 4096
// (graph replay, every form forced on the same box): two weight tiles per wave
// once that leaves four wave columns of tiles per compute unit, then the
// smallest split of K that puts enough waves on every compute unit.  With two
// tiles per wave there are then at least four tiles per compute unit, so the
// split is 1 or 2; with one, 4 from 1.5 tiles per compute unit, else 8 -- the
// four forms compiled below, whatever the compute-unit count (at P = 256 qkv
// 9.75 us with <1,4> against 10.5 with two tiles per wave, down 8.8 against
// 9.1 with <1,8>).  With at least three 64 x 64 tiles per SIMD the
// two-token-tile kernel takes over (measured at P = 4096: gate_up 138-140
// against 149 us, qkv 89-90 against 91-94), also with K split over two waves
// where whole K would leave fewer.
FragLayout prefill_frag_layout(int64_t n, int64_t p, int cu_count) {
    const int64_t ntn = (n + 31) / 32, ntp = (p + 31) / 32, cus = cu_count;
    const int wn = (ntn + 1) / 2 * ntp >= 4 * cus ? 2 : 1;
    const int64_t tiles = (ntn + wn - 1) / wn * ntp;
    int ks;
    if (wn == 2)
        ks = tiles >= 8 * cus ? 1 : 2;
    else
        ks = 2 * tiles >= 3 * cus ? 4 : 8;
    const int64_t ntw = (ntn + wn - 1) / wn;
    // 64 x 64 per wave once that still leaves three waves of work per SIMD,
    // with K whole or split over two waves
    const int64_t ntq = (ntp + 1) / 2;
    int wp = 1;
    if (wn == 2) {
        if (ntw * ntq >= 12 * cus) {
            wp = 2;
            ks = 1;
        } else if (2 * ntw * ntq >= 12 * cus) {
            wp = 2;
            ks = 2;
        }
    }
    const int waves = ks > 4 ? ks : 4;
    const int per_wg = waves / ks;
    const int64_t rows_w = wp == 2 ? ntq : ntp;
    int64_t maxwg = 0;
    for (int x = 0; x < 8; ++x) {
        const int64_t nc = ntw * (x + 1) / 8 - ntw * x / 8;
        const int64_t wgs = (nc * rows_w + per_wg - 1) / per_wg;
        maxwg = wgs > maxwg ? wgs : maxwg;
    }
    return FragLayout{wn, ks, 8 * maxwg, wp};
}

hipError_t launch_pack_frag(const int8_t* q, const uint16_t* d, int64_t rows, int64_t k, int8_t* qf,
                            uint16_t* df, const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
    const int nb = (int)(k / 32), nbp = (int)frag_blocks(k);
    const int64_t tiles = frag_rows(rows) / 32;
    const int64_t work = tiles * nbp * 64 + tiles * (nbp / 4) * 32;
    int64_t grid = (work + 255) / 256;
    const int64_t cap = (int64_t)dev.cu_count * 16;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    pack_frag_kernel<<<(unsigned)grid, 256, 0, stream>>>(q, d, rows, nb, nbp, tiles, qf, df);
    return hipGetLastError();
}

hipError_t launch_prefill_frag(const int8_t* wf, const uint16_t* wsf, int64_t n, int64_t k, int64_t p,
                               const int8_t* xf, const uint16_t* xsf, float* y, const DeviceInfo& dev,
                               hipStream_t stream) {
    (void)hipGetLastError();
    const FragLayout L = prefill_frag_layout(n, p, dev.cu_count);
    if (L.wp == 2) {
        const auto wa = reinterpret_cast<const i32x4*>(wf);
        const auto ws = reinterpret_cast<const i32x2*>(wsf);
        const auto xa = reinterpret_cast<const i32x4*>(xf);
        const auto xs = reinterpret_cast<const i32x2*>(xsf);
        const int nbp = (int)frag_blocks(k);
        if (L.ks == 2)
            prefill_frag64_kernel<2><<<(unsigned)L.grid, 256, 0, stream>>>(wa, ws, n, nbp, p, xa, xs, y);
        else
            prefill_frag64_kernel<1><<<(unsigned)L.grid, 256, 0, stream>>>(wa, ws, n, nbp, p, xa, xs, y);
        return hipGetLastError();
    }
    if (L.wn == 2) {
        if (L.ks == 1) return launch_frag_cfg<2, 1>(wf, wsf, n, k, p, xf, xsf, y, L.grid, stream);
        return launch_frag_cfg<2, 2>(wf, wsf, n, k, p, xf, xsf, y, L.grid, stream);
    }
    if (L.ks == 4) return launch_frag_cfg<1, 4>(wf, wsf, n, k, p, xf, xsf, y, L.grid, stream);
    return launch_frag_cfg<1, 8>(wf, wsf, n, k, p, xf, xsf, y, L.grid, stream);
}

}  // namespace q8
