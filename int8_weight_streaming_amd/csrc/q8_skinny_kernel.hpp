// q8_skinny_kernel.hpp -- the batch 1..8 decode product kernel over Q8_0
// weights, shared by the plain products (q8_skinny.hip) and the fused decode-step
// products (q8_fused.hip).  The work layout is described in q8_skinny.hip.
#pragma once

#include "q8_device.hpp"
#include "q8_internal.hpp"

namespace q8 {

// Fused prologues and epilogues: the glue of a decode step around the W8A16
// products [Frigg README, "The model, as verified": RMSNorm without a learnable
// weight (eps 1e-6) before every product that reads the residual stream, the
// default rotary embedding (theta 10,000) on the query and key rows, SwiGLU
// between the gate/up and down products, residual adds after the output and
// down products].
enum { kProBf16 = 0, kProF32 = 1, kProNorm = 2, kProAttn = 3, kProAttn16 = 4 };
enum { kEpiF32 = 0, kEpiAdd = 1, kEpiSwiglu = 2, kEpiRope = 3 };
constexpr float kRmsEps = 1e-6f;
constexpr double kRopeTheta = 10000.0;
constexpr int kRopeHead = 128;                 // head width of the rotated rows

struct FuseArgs {
    int64_t rope_rows;                         // rows [0, rope_rows) hold rotated heads
    int64_t pos;                               // position of the token
    int64_t attn_chunks;                       // attention prologue: chunk partials per head
};

__device__ __forceinline__ uint16_t to_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return (uint32_t)to_bf16(a) | ((uint32_t)to_bf16(b) << 16);
}

// Eight consecutive fp32 activations times `mul`, rounded to bf16 (nearest,
// ties to even), as four packed pairs.
__device__ __forceinline__ uint4 load_x8_f32(const float* p, float mul) {
    const float4 f0 = reinterpret_cast<const float4*>(p)[0], f1 = reinterpret_cast<const float4*>(p)[1];
    return make_uint4(pack_bf16(f0.x * mul, f0.y * mul), pack_bf16(f0.z * mul, f0.w * mul),
                      pack_bf16(f1.x * mul, f1.y * mul), pack_bf16(f1.z * mul, f1.w * mul));
}

// Sixteen activations of one chunk as eight bf16 pairs: read as bf16, or
// converted from fp32 (scaled by `mul`).
template <int PRO>
__device__ __forceinline__ void load_x16(const void* xv, int64_t off, float mul, uint32_t out[8]) {
    uint4 a, b;
    if constexpr (PRO == kProBf16) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + off);
        a = p[0];
        b = p[1];
    } else {
        const float* p = static_cast<const float*>(xv) + off;
        a = load_x8_f32(p, mul);
        b = load_x8_f32(p + 8, mul);
    }
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Inverse RMS of each of the M fp32 rows of x [M][k]: 1 / sqrt(mean(x^2) + eps),
// summed in one fixed order: thread t of the 256 takes the eight-value groups
// t, t + 256, ... of the row (values 8g .. 8g + 7) and sums their squares in
// order (fmaf), a fixed DPP tree sums each wave, and the four waves are added
// 0 + 1 + 2 + 3.  Every workgroup computes it for itself (a few KiB from L2).
// rms_finish is the part after the per-thread sums; it must be reached by every
// thread of the 256-thread workgroup, at most once per kernel.
template <int M>
__device__ __forceinline__ void rms_finish(float ss[M], int64_t k, float inv[M]) {
    __shared__ float red[4][M];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        ss[m] = group_sum<64>(ss[m]);
        if (lane == 0) red[wave][m] = ss[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float t = ((red[0][m] + red[1][m]) + red[2][m]) + red[3][m];
        inv[m] = 1.0f / sqrtf(t / (float)k + kRmsEps);
    }
}

__device__ __forceinline__ float sumsq8(const float4& a, const float4& b, float s) {
    s = fmaf(a.x, a.x, s); s = fmaf(a.y, a.y, s); s = fmaf(a.z, a.z, s); s = fmaf(a.w, a.w, s);
    s = fmaf(b.x, b.x, s); s = fmaf(b.y, b.y, s); s = fmaf(b.z, b.z, s); s = fmaf(b.w, b.w, s);
    return s;
}

template <int M>
__device__ __forceinline__ void row_inv_rms(const float* x, int64_t k, float inv[M]) {
    float ss[M];
#pragma unroll
    for (int m = 0; m < M; ++m) ss[m] = 0.0f;
    for (int64_t g = threadIdx.x; 8 * g < k; g += 256)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float4* p = reinterpret_cast<const float4*>(x + (int64_t)m * k + 8 * g);
            ss[m] = sumsq8(p[0], p[1], ss[m]);
        }
    rms_finish<M>(ss, k, inv);
}

// Row staging of fp32 activations, rows of k <= kStageK: thread t holds values
// 8t .. 8t + 7 of every row -- its one group of the norm's order above -- so
// the same registers give the inverse RMS and, scaled and rounded to bf16, the
// staged tile.  The loads are unconditional (clamped to the row).
constexpr int kStageK = 256 * 8;
template <int M>
__device__ __forceinline__ void stage_load(const float* x, int64_t k, float4 v[M][2]) {
    const int64_t g = 8 * (int64_t)threadIdx.x < k ? threadIdx.x : 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float4* p = reinterpret_cast<const float4*>(x + (int64_t)m * k + 8 * g);
        v[m][0] = p[0];
        v[m][1] = p[1];
    }
}

// Attention-output prologue (batch 1): the activation row is the decode
// attention output [heads][128], combined here from the per-chunk partials the
// attention left in the workspace -- per (head, chunk) a record of
// kAttnPartFloats floats: numerator [128], maximum m, denominator l -- exactly
// as the attention's own combine does it:
//   a[h][d] = sum_c o_c[d] e^(m_c - M) / sum_c l_c e^(m_c - M),  M = max_c m_c,
// the sums in chunk order.  Thread t takes values 8t .. 8t + 7 (head t / 16);
// all partials of up to NC chunks (8, or 16 for kProAttn16) are fetched at once
// (indices past the last chunk repeat it and get weight zero).
template <int NC>
__device__ __forceinline__ void attn_parts_load(const float* w, int64_t k, int nchunks, float4 ao[NC][2],
                                                float2 aml[NC]) {
    const int t = 8 * (int64_t)threadIdx.x < k ? (int)threadIdx.x : 0;
    const int h = t >> 4, d0 = (8 * t) & 127;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int cc = c < nchunks ? c : nchunks - 1;
        const float* part = w + ((int64_t)h * nchunks + cc) * kAttnPartFloats;
        ao[c][0] = *reinterpret_cast<const float4*>(part + d0);
        ao[c][1] = *reinterpret_cast<const float4*>(part + d0 + 4);
        aml[c] = *reinterpret_cast<const float2*>(part + 128);
    }
}
template <int NC>
__device__ __forceinline__ void attn_combine(const float4 ao[NC][2], const float2 aml[NC], int nchunks,
                                             float4 out[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < NC; ++c) mx = fmaxf(mx, aml[c].x);
    float num[8], den = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c < nchunks) {                       // uniform
            const float e = expf(aml[c].x - mx);
            const float v[8] = {ao[c][0].x, ao[c][0].y, ao[c][0].z, ao[c][0].w,
                                ao[c][1].x, ao[c][1].y, ao[c][1].z, ao[c][1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) num[i] = fmaf(v[i], e, num[i]);
            den = fmaf(aml[c].y, e, den);
        }
    }
    out[0] = make_float4(num[0] / den, num[1] / den, num[2] / den, num[3] / den);
    out[1] = make_float4(num[4] / den, num[5] / den, num[6] / den, num[7] / den);
}

// theta^(-i/64) = 10000^(-i/64), i = 0..63: the rotary frequencies of a
// 128-wide head, to double precision.
static __constant__ double kRopeInvFreq[kRopeHead / 2] = {
    1.0, 0.8659643233600653, 0.7498942093324559, 0.6493816315762113,
    0.5623413251903491, 0.4869675251658631, 0.4216965034285822, 0.3651741272548377,
    0.31622776601683794, 0.27384196342643613, 0.23713737056616552, 0.2053525026457146,
    0.1778279410038923, 0.1539926526059492, 0.1333521432163324, 0.11547819846894582,
    0.1, 0.08659643233600653, 0.07498942093324558, 0.06493816315762113,
    0.05623413251903491, 0.04869675251658631, 0.042169650342858224, 0.03651741272548377,
    0.03162277660168379, 0.027384196342643614, 0.023713737056616554, 0.02053525026457146,
    0.01778279410038923, 0.01539926526059492, 0.01333521432163324, 0.011547819846894581,
    0.01, 0.008659643233600654, 0.007498942093324558, 0.006493816315762113,
    0.005623413251903491, 0.004869675251658631, 0.004216965034285823, 0.003651741272548377,
    0.0031622776601683794, 0.0027384196342643613, 0.0023713737056616554, 0.002053525026457146,
    0.0017782794100389228, 0.001539926526059492, 0.001333521432163324, 0.0011547819846894581,
    0.001, 0.0008659643233600654, 0.0007498942093324559, 0.0006493816315762113,
    0.0005623413251903491, 0.0004869675251658631, 0.00042169650342858224, 0.0003651741272548377,
    0.00031622776601683794, 0.0002738419634264361, 0.00023713737056616554, 0.0002053525026457146,
    0.00017782794100389227, 0.0001539926526059492, 0.0001333521432163324, 0.00011547819846894582,
};

// Rotation of the pair that starts at stored row `row` (rows below rope_rows):
// pair p = row / 2 is dimension i = p % 64 of its head, turned by
// pos * theta^(-i/64).  rope_freq reads the frequency (issued first, so its
// latency hides under the weight loads).  rope_turn forms the angle in fp64 and
// reduces it to r in [-pi/4, pi/4] with a quadrant q (angle = q pi/2 + r; pi/2
// in two parts, so for positions below 2^24 r is accurate to ~1e-9 rad), then
// takes sin r and cos r from their Taylor series to r^9 and r^10 (truncation
// error below 2e-9 on that interval) in fp32, branch-free.
__device__ __forceinline__ double rope_freq(int64_t row, const FuseArgs& fa) {
    return row < fa.rope_rows ? kRopeInvFreq[(row >> 1) % (kRopeHead / 2)] : 0.0;
}
__device__ __forceinline__ void rope_turn(double freq, const FuseArgs& fa, float& c, float& s) {
    const double ang = (double)fa.pos * freq;
    const double q = rint(ang * 0.63661977236758134);             // 2 / pi
    const double pio2_hi = 1.5707963267948966, pio2_lo = 6.123233995736766e-17;
    const float r = (float)fma(-q, pio2_lo, fma(-q, pio2_hi, ang));
    const float r2 = r * r;
    const float sn = r * (1.0f + r2 * (-1.0f / 6 + r2 * (1.0f / 120 + r2 * (-1.0f / 5040 + r2 * (1.0f / 362880)))));
    const float cs = 1.0f + r2 * (-0.5f + r2 * (1.0f / 24 + r2 * (-1.0f / 720 + r2 * (1.0f / 40320 +
                                                                                       r2 * (-1.0f / 3628800)))));
    const int qi = (int)((int64_t)q & 3);
    // cos and sin of q pi/2 + r
    c = qi == 0 ? cs : qi == 1 ? -sn : qi == 2 ? -cs : sn;
    s = qi == 0 ? sn : qi == 1 ? cs : qi == 2 ? -sn : -cs;
}

template <int EPI>
__device__ __forceinline__ void paired_epilogue(float a, float b, int64_t row, int m, int64_t n,
                                                const FuseArgs& fa, float c, float s, uint16_t* out) {
    const int64_t p = row >> 1;
    if constexpr (EPI == kEpiSwiglu) {
        out[(int64_t)m * (n >> 1) + p] = to_bf16(a / (1.0f + expf(-a)) * b);
    } else {
        if (row < fa.rope_rows) {
            const int64_t h = p / (kRopeHead / 2);
            const int i = (int)(p % (kRopeHead / 2));
            uint16_t* o = out + (int64_t)m * n + h * kRopeHead + i;
            o[0] = to_bf16(a * c - b * s);
            o[kRopeHead / 2] = to_bf16(b * c + a * s);
        } else {
            out[(int64_t)m * n + row] = to_bf16(a);
            out[(int64_t)m * n + row + 1] = to_bf16(b);
        }
    }
}

// Activations of one K tile: registers or LDS.
template <int M, int ACT, int CPL>
struct XRegs {
    // bf16: 8 dwords per chunk; Q8: 4 dwords of codes per chunk + the block
    // scale's binary16 bits (converted where it is used: a conversion next to
    // the load would wait for it before the weight loads are issued).
    uint32_t v[M][CPL][ACT == 0 ? 8 : 4];
    uint16_t s[M][CPL];
};

// Activations in registers at batch 1-2 (bf16 or Q8 input); fp32 input
// (fused prologues) is converted once per workgroup into LDS instead.
template <int M, int ACT, int PRO = 0>
constexpr bool x_in_registers() { return M <= 2 && PRO == 0; }

template <int M, int ACT, int G, int R, int CPL, int PRO = kProBf16, int EPI = kEpiF32>
__global__ __launch_bounds__(256) void skinny_kernel(const int8_t* __restrict__ wq,
                                                     const uint16_t* __restrict__ wd, int64_t n,
                                                     int nb, const void* __restrict__ xv,
                                                     const uint16_t* __restrict__ xdp,
                                                     void* __restrict__ yv, FuseArgs fa) {
    static_assert(PRO == kProBf16 || ACT == 0, "fp32 prologues take bf16-product weights");
    static_assert(EPI < kEpiSwiglu || R == 2 || (R == 1 && G == 32),
                  "paired epilogues need both rows of a pair in one wave");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    constexpr int GPW = 64 / G;                  // lane groups per wave
    constexpr int RPW = 4 * GPW * R;             // rows per workgroup
    constexpr int TCH = G * CPL;                 // chunks per K tile
    constexpr bool XREG = x_in_registers<M, ACT, PRO>();
    constexpr int XCH_BYTES = ACT == 0 ? 32 : 16;   // activation bytes per chunk and row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gl = lane & (G - 1), grp = lane / G;
    const int nch = nb * 2;
    const int64_t k = (int64_t)nb * 32;
    const int64_t rbase = (int64_t)blockIdx.x * RPW + (int64_t)(wave * GPW + grp) * R;
    float* y = static_cast<float*>(yv);

    // Prologue: per activation row the factor its fp32 values are scaled by
    // before rounding to bf16 (the inverse RMS for the norm prologue, else 1);
    // computed once the first tile's weight loads are in flight.
    float xmul[M];
#pragma unroll
    for (int m = 0; m < M; ++m) xmul[m] = 1.0f;
    // Residual-add epilogue: lane g of a group adds into output value g (see
    // the store below); its old value is fetched now, under the weight stream.
    float hres = 0.0f;
    if constexpr (EPI == kEpiAdd) {
        static_assert(R * M <= G, "one store per lane");
        if (gl < R * M) {
            const int64_t row = rbase + gl % R;
            if (row < n) hres = y[(int64_t)(gl / R) * n + row];
        }
    }
    // RoPE epilogue: the pair's rotation, computed once the first tile's loads
    // are issued.
    float rc = 1.0f, rs = 0.0f;
    double rfreq = 0.0;
    if constexpr (EPI == kEpiRope) rfreq = rope_freq(rbase, fa);
    // fp32 activations at batch 1-2 with the whole row in one tile: staged
    // from registers fetched before anything else (rows read once per
    // workgroup); otherwise per tile from memory, below.
    constexpr bool RS = PRO != kProBf16 && M <= 2;
    const bool rstage = RS && k <= kStageK && k <= (int64_t)TCH * 16;
    float4 sv[RS ? M : 1][2];
    constexpr bool AT = PRO == kProAttn || PRO == kProAttn16;
    constexpr int NC = PRO == kProAttn16 ? 16 : 8;           // chunks the prologue combines
    static_assert(!AT || M == 1, "the attention prologue is a batch-1 prologue");
    float4 ao[AT ? NC : 1][2];
    float2 aml[AT ? NC : 1];
    if constexpr (AT) attn_parts_load<NC>(static_cast<const float*>(xv), k, (int)fa.attn_chunks, ao, aml);
    else if constexpr (RS) stage_load<M>(static_cast<const float*>(xv), k, sv);

    // Q8 activations: the products (row r, activation row m), numbered
    // c = m R + r, are taken two at a time; the even lane of a chunk pair
    // accumulates product 2p of slot p, the odd lane product 2p + 1 (an odd
    // last product: the even lane alone), so that one DPP add finishes both
    // block sums (block_dot_pair) and each is converted and folded once.
    static_assert(ACT == 0 || EPI == kEpiF32 || EPI == kEpiAdd, "Q8 activations store one value per lane");
    constexpr int NPS = (R * M + 1) / 2;
    const bool even = (gl & 1) == 0;

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
    float pacc[ACT == 1 ? NPS : 1];
#pragma unroll
    for (int p = 0; p < (ACT == 1 ? NPS : 1); ++p) pacc[p] = 0.0f;

    // staged activation pieces of a tile (batch 3-8), see below
    constexpr bool XPRE = !XREG && PRO == kProBf16;
    constexpr int XP = XPRE ? (M * TCH * (XCH_BYTES / 16) + 255) / 256 : 1;
    constexpr int XS = XPRE && ACT == 1 ? (M * (TCH / 2) + 255) / 256 : 1;
    u32x4 xst[XP];
    uint16_t xsb[XS];
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
                        load_x16<PRO>(xv, m * k + (int64_t)cc * 16, xmul[m], xr.v[m][j]);
                    } else {
                        const uint4 a = *reinterpret_cast<const uint4*>(
                            static_cast<const int8_t*>(xv) + m * k + (int64_t)cc * 16);
                        xr.v[m][j][0] = a.x; xr.v[m][j][1] = a.y; xr.v[m][j][2] = a.z; xr.v[m][j][3] = a.w;
                        xr.s[m][j] = xdp[(int64_t)m * nb + (cc >> 1)];
                    }
                }
            }
        }
        // ---- bf16 / Q8 activations staged in LDS (batch 3-8): this thread's
        // pieces of the tile are fetched now, before the weights, and written
        // to LDS once the weight loads are in flight (loads return in order:
        // fetched after the weights, writing them would wait for the whole
        // weight tile)
        const int tch = nch - c0 < TCH ? nch - c0 : TCH;          // chunks in this tile
        const int pieces = M * tch * (XCH_BYTES / 16);
        if constexpr (XPRE) {
            // unconditional loads (indices past the tile clamped to its last
            // piece): a load inside a divergent branch is waited for at once
#pragma unroll
            for (int u = 0; u < XP; ++u) {
                const int i0 = threadIdx.x + 256 * u;
                const int i = i0 < pieces ? i0 : pieces - 1;
                const int q = ACT == 0 ? (i & 1) : 0;
                const int rest = ACT == 0 ? (i >> 1) : i;
                const int ch = rest % tch, m = rest / tch;
                const unsigned char* src = static_cast<const unsigned char*>(xv) +
                    ((int64_t)m * k + (int64_t)(c0 + ch) * 16) * (ACT == 0 ? 2 : 1) + q * 16;
                xst[u] = *reinterpret_cast<const u32x4*>(src);
            }
            if constexpr (ACT == 1) {
                const int nsc = M * (tch >> 1);
#pragma unroll
                for (int u = 0; u < XS; ++u) {
                    const int i0 = threadIdx.x + 256 * u;
                    const int i = i0 < nsc ? i0 : nsc - 1;
                    const int bl = i % (tch >> 1), m = i / (tch >> 1);
                    xsb[u] = xdp[(int64_t)m * nb + (c0 >> 1) + bl];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
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
        if constexpr (EPI == kEpiRope) {
            // the pair's rotation first: its math overlaps the wait for the rows
            if (c0 == 0 && rbase < fa.rope_rows) {
                pin(rfreq);
                rope_turn(rfreq, fa, rc, rs);
            }
        }
        if constexpr (AT) {
            // the attention partials: combined now, after the weight loads are issued
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                pin(aml[c].x); pin(aml[c].y);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    pin(ao[c][h].x); pin(ao[c][h].y); pin(ao[c][h].z); pin(ao[c][h].w);
                }
            }
            attn_combine<NC>(ao, aml, (int)fa.attn_chunks, sv[0]);
        } else if constexpr (RS) {
            // staged rows: wanted only now, after the weight loads are issued
            if (rstage) {
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        pin(sv[m][h].x); pin(sv[m][h].y); pin(sv[m][h].z); pin(sv[m][h].w);
                    }
            }
        }
        if (c0 == 0) {
            if constexpr (PRO == kProNorm) {
                if (RS && rstage) {
                    float ss[M];
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        ss[m] = 8 * (int64_t)threadIdx.x < k ? sumsq8(sv[m][0], sv[m][1], 0.0f) : 0.0f;
                    rms_finish<M>(ss, k, xmul);
                } else {
                    row_inv_rms<M>(static_cast<const float*>(xv), k, xmul);
                }
            }
        }
        if (RS && rstage) {
            // the one tile, from the staged rows: values 8t .. 8t + 7 of row m
            // go to bytes 16t .. 16t + 15 of the row's slot
            if (8 * (int64_t)threadIdx.x < k) {
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const float mul = xmul[m];
                    const float4 f0 = sv[m][0], f1 = sv[m][1];
                    *reinterpret_cast<uint4*>(lds + m * TCH * 32 + threadIdx.x * 16) =
                        make_uint4(pack_bf16(f0.x * mul, f0.y * mul), pack_bf16(f0.z * mul, f0.w * mul),
                                   pack_bf16(f1.x * mul, f1.y * mul), pack_bf16(f1.z * mul, f1.w * mul));
                }
            }
            __syncthreads();
        } else if (!XREG) {
            // stage the tile in LDS while the weight loads are in flight:
            // [m][chunk] with XCH_BYTES per chunk, then the Q8 scales
            __syncthreads();
            if constexpr (XPRE) {
                // (indices clamped as for the loads: a lane past the tile
                // writes its last piece again, with the same bytes)
#pragma unroll
                for (int u = 0; u < XP; ++u) {
                    const int i0 = threadIdx.x + 256 * u;
                    const int i = i0 < pieces ? i0 : pieces - 1;
                    const int q = ACT == 0 ? (i & 1) : 0;
                    const int rest = ACT == 0 ? (i >> 1) : i;
                    const int ch = rest % tch, m = rest / tch;
                    *reinterpret_cast<u32x4*>(lds + (m * TCH + ch) * XCH_BYTES + q * 16) = xst[u];
                }
                if constexpr (ACT == 1) {
                    float* sc = reinterpret_cast<float*>(lds + M * TCH * XCH_BYTES);
                    const int nsc = M * (tch >> 1);
#pragma unroll
                    for (int u = 0; u < XS; ++u) {
                        const int i0 = threadIdx.x + 256 * u;
                        const int i = i0 < nsc ? i0 : nsc - 1;
                        const int bl = i % (tch >> 1), m = i / (tch >> 1);
                        pin(xsb[u]);      // converted here, not hoisted above the weight loads
                        sc[m * (TCH / 2) + bl] = half_bits_to_float(xsb[u]);
                    }
                }
            } else {
                // fp32 rows (fused prologues above batch 2): scaled and rounded here
                for (int i = threadIdx.x; i < pieces; i += 256) {
                    const int q = i & 1;
                    const int ch = (i >> 1) % tch, m = (i >> 1) / tch;
                    float mul = 1.0f;
#pragma unroll
                    for (int mm = 0; mm < M; ++mm) mul = mm == m ? xmul[mm] : mul;
                    *reinterpret_cast<uint4*>(lds + (m * TCH + ch) * XCH_BYTES + q * 16) =
                        load_x8_f32(static_cast<const float*>(xv) + (int64_t)m * k + (int64_t)(c0 + ch) * 16 + q * 8, mul);
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
                // exact int32 block sums: this lane's half and its neighbour's
                auto xload = [&](int m, u32x4& xc, float& xs) {
                    if (XREG) {
                        xc = (u32x4){xr.v[m][j][0], xr.v[m][j][1], xr.v[m][j][2], xr.v[m][j][3]};
                        xs = half_bits_to_float(xr.s[m][j]);
                    } else {
                        const uint4 a = *reinterpret_cast<const uint4*>(lds + (m * TCH + clc) * 16);
                        xc = (u32x4){a.x, a.y, a.z, a.w};
                        xs = reinterpret_cast<const float*>(lds + M * TCH * 16)[m * (TCH / 2) + (clc >> 1)];
                    }
                };
#pragma unroll
                for (int p = 0; p < NPS; ++p) {
                    const int ca = 2 * p, cb = 2 * p + 1;
                    const int ma = ca / R, ra = ca % R;
                    u32x4 xa;
                    float sa;
                    xload(ma, xa, sa);
                    if (cb < R * M) {
                        const int mb = cb / R, rb = cb % R;
                        u32x4 xb = xa;
                        float sb2 = sa;
                        if (mb != ma) xload(mb, xb, sb2);
                        const int s = block_dot_pair(w[j][ra], xa, w[j][rb], xb, even);
                        const float t = (even ? ws[j][ra] : ws[j][rb]) * (even ? sa : sb2);
                        pacc[p] = fmaf((float)s, t, pacc[p]);
                    } else {
                        const int s = block_dot_halves(w[j][ra], xa);
                        pacc[p] = fmaf((float)s, even ? ws[j][ra] * sa : 0.0f, pacc[p]);
                    }
                }
            }
        }
    }

    // Combine the G partial sums of every (row, m); all lanes of the group end
    // with the same value.  Q8 activations: the sums over the lanes of one
    // parity, so a lane of parity q holds product 2p + q of every slot p (the
    // lane that stores a product has its parity, see the store below).
    if constexpr (ACT == 1) {
#pragma unroll
        for (int p = 0; p < NPS; ++p) {
            const float v = group_sum_parity<G>(pacc[p]);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                if (2 * p + q < R * M) acc[(2 * p + q) % R][(2 * p + q) / R] = v;
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = group_sum<G>(acc[r][m]);
    }

    if constexpr (EPI == kEpiF32 || EPI == kEpiAdd) {
        // Lane g of the group stores value g (then g + G, ...): rows of one m
        // land on consecutive lanes.
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
                if (row < n) {
                    if constexpr (EPI == kEpiAdd) y[(int64_t)m * n + row] = hres + out;
                    else y[(int64_t)m * n + row] = out;
                }
            }
        }
    } else {
        // Paired rows (2p, 2p + 1): both values of every m, on every lane of the
        // group that holds the even row; its lane m stores activation row m.
        float pa[M], pb[M];
        bool lead = true;
        if constexpr (R == 2) {
#pragma unroll
            for (int m = 0; m < M; ++m) { pa[m] = acc[0][m]; pb[m] = acc[1][m]; }
        } else {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float other = xor32_value(acc[0][m]);
                pa[m] = grp == 0 ? acc[0][m] : other;
                pb[m] = grp == 0 ? other : acc[0][m];
            }
            lead = grp == 0;
        }
        if (lead && gl < M && rbase < n) {
            float a = 0.0f, b = 0.0f;
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (m == gl) { a = pa[m]; b = pb[m]; }
            paired_epilogue<EPI>(a, b, rbase, gl, n, fa, rc, rs, static_cast<uint16_t*>(yv));
        }
    }
}

}  // namespace q8
