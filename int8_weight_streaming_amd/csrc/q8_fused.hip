// q8_fused.hip -- the glue of a decode step fused into the W8A16 products, and
// the standalone weightless RMSNorm.
//
// A decode block [Frigg README, "The model, as verified": pre-norm blocks with
// RMSNorm without a learnable weight, eps 1e-6; rotary embedding theta 10,000,
// default rotation; SwiGLU MLP; one final norm per module run] needs, besides
// its four products, a norm before qkv and before gate/up, the rotation of the
// query and key rows, the SwiGLU between gate/up and down, and two residual
// adds.  Each of these is folded into the product next to it, so a block is
// its four product launches plus attention:
//   qkv      RMSNorm prologue (fp32 residual -> bf16), RoPE epilogue (bf16 q|k|v)
//   o        fp32 -> bf16 prologue (attention output), residual-add epilogue
//   gate/up  RMSNorm prologue, SwiGLU epilogue (bf16)
//   down     bf16 prologue, residual-add epilogue
//   lm_head  fp32 -> bf16 prologue (or RMSNorm), fp32 logits
// The paired epilogues need both rows of a pair in one wave: the weights of
// the query/key rows and of gate/up are stored pair-interleaved (row 2j and
// 2j + 1 of the matrix are the two members of pair j), a layout chosen when the
// weights are prepared.  Outputs are written in natural order.
#include "q8_skinny_kernel.hpp"

namespace q8 {

template <int M, int G, int R, int CPL, int PRO, int EPI>
static hipError_t fused_cfg(const int8_t* wq, const uint16_t* wd, int64_t n, int nb, const void* x,
                            void* out, const FuseArgs& fa, hipStream_t stream) {
    constexpr int RPW = 4 * (64 / G) * R;
    constexpr int TCH = G * CPL;
    const size_t lds = x_in_registers<M, 0, PRO>() ? 0 : (size_t)M * TCH * 32;
    const int64_t grid = (n + RPW - 1) / RPW;
    skinny_kernel<M, 0, G, R, CPL, PRO, EPI><<<(unsigned)grid, 256, lds, stream>>>(wq, wd, n, nb, x, nullptr,
                                                                               out, fa);
    return hipGetLastError();
}

// The launch shapes of the plain W8A16 products; a shape whose pair partner
// would sit in another wave (one row per wave) is replaced by 32-lane groups.
template <int M, int PRO, int EPI>
static hipError_t fused_m(const int8_t* wq, const uint16_t* wd, int64_t n, int nb, const void* x,
                          void* out, const FuseArgs& fa, const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
    const int64_t tall_wgs = (n + 31) / 32;
    if (tall_wgs >= (int64_t)dev.cu_count * (M <= 2 ? 1 : 4))
        return fused_cfg<M, 16, 2, 6, PRO, EPI>(wq, wd, n, nb, x, out, fa, stream);
    if (nb <= 48) return fused_cfg<M, 32, 1, 3, PRO, EPI>(wq, wd, n, nb, x, out, fa, stream);
    if constexpr (M <= 2 || EPI >= kEpiSwiglu) {
        return fused_cfg<M, 32, 1, 8, PRO, EPI>(wq, wd, n, nb, x, out, fa, stream);
    } else {
        return fused_cfg<M, 64, 1, 2, PRO, EPI>(wq, wd, n, nb, x, out, fa, stream);
    }
}

template <int PRO, int EPI>
static hipError_t fused_pe(const int8_t* wq, const uint16_t* wd, int64_t n, int nb, int m, const void* x,
                           void* out, const FuseArgs& fa, const DeviceInfo& dev, hipStream_t stream) {
    switch (m) {
        case 1: return fused_m<1, PRO, EPI>(wq, wd, n, nb, x, out, fa, dev, stream);
        case 2: return fused_m<2, PRO, EPI>(wq, wd, n, nb, x, out, fa, dev, stream);
        case 3: return fused_m<3, PRO, EPI>(wq, wd, n, nb, x, out, fa, dev, stream);
        case 4: return fused_m<4, PRO, EPI>(wq, wd, n, nb, x, out, fa, dev, stream);
        case 5: return fused_m<5, PRO, EPI>(wq, wd, n, nb, x, out, fa, dev, stream);
        case 6: return fused_m<6, PRO, EPI>(wq, wd, n, nb, x, out, fa, dev, stream);
        case 7: return fused_m<7, PRO, EPI>(wq, wd, n, nb, x, out, fa, dev, stream);
        case 8: return fused_m<8, PRO, EPI>(wq, wd, n, nb, x, out, fa, dev, stream);
        default: return hipErrorInvalidValue;
    }
}

bool fused_combo_supported(int pro, int epi) {
    return (pro == kProNorm && epi == kEpiRope) || (pro == kProF32 && epi == kEpiAdd) ||
           (pro == kProNorm && epi == kEpiSwiglu) || (pro == kProBf16 && epi == kEpiAdd) ||
           (pro == kProF32 && epi == kEpiF32) || (pro == kProNorm && epi == kEpiF32);
}

hipError_t launch_fused(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m, int pro,
                        const void* x, int epi, void* out, int64_t rope_rows, int64_t pos,
                        const DeviceInfo& dev, hipStream_t stream) {
    const int nb = (int)(k / 32);
    const FuseArgs fa{rope_rows, pos};
    if (pro == kProNorm && epi == kEpiRope) return fused_pe<kProNorm, kEpiRope>(wq, wd, n, nb, m, x, out, fa, dev, stream);
    if (pro == kProF32 && epi == kEpiAdd) return fused_pe<kProF32, kEpiAdd>(wq, wd, n, nb, m, x, out, fa, dev, stream);
    if (pro == kProNorm && epi == kEpiSwiglu) return fused_pe<kProNorm, kEpiSwiglu>(wq, wd, n, nb, m, x, out, fa, dev, stream);
    if (pro == kProBf16 && epi == kEpiAdd) return fused_pe<kProBf16, kEpiAdd>(wq, wd, n, nb, m, x, out, fa, dev, stream);
    if (pro == kProF32 && epi == kEpiF32) return fused_pe<kProF32, kEpiF32>(wq, wd, n, nb, m, x, out, fa, dev, stream);
    if (pro == kProNorm && epi == kEpiF32) return fused_pe<kProNorm, kEpiF32>(wq, wd, n, nb, m, x, out, fa, dev, stream);
    return hipErrorInvalidValue;
}

template <int PRO>
static hipError_t attn_residual_pro(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int nb,
                                    const float* work, float* y, const FuseArgs& fa, const DeviceInfo& dev,
                                    hipStream_t stream) {
    const int64_t tall_wgs = (n + 31) / 32;
    if (tall_wgs >= (int64_t)dev.cu_count && k <= 16 * 6 * 16)
        return fused_cfg<1, 16, 2, 6, PRO, kEpiAdd>(wq, wd, n, nb, work, y, fa, stream);
    if (nb <= 48) return fused_cfg<1, 32, 1, 3, PRO, kEpiAdd>(wq, wd, n, nb, work, y, fa, stream);
    return fused_cfg<1, 32, 1, 8, PRO, kEpiAdd>(wq, wd, n, nb, work, y, fa, stream);
}

// The output projection reading the attention partials directly (batch 1,
// residual add): the prologue combines the row once per workgroup, so the
// whole row must fit one K tile -- only such shapes are used.
hipError_t launch_attn_residual(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, const float* work,
                                int nchunks, float* y, const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
    const int nb = (int)(k / 32);
    const FuseArgs fa{0, 0, nchunks};
    if (nchunks <= 8) return attn_residual_pro<kProAttn>(wq, wd, n, k, nb, work, y, fa, dev, stream);
    return attn_residual_pro<kProAttn16>(wq, wd, n, k, nb, work, y, fa, dev, stream);
}

// ------------------------------------------------------------------ RMSNorm

// One workgroup per row: y = x * inv_rms(x), with the product prologue's own
// reduction, so y rounded to bf16 is exactly what a norm prologue feeds its
// product.  In place is allowed: every element is read before the barrier
// inside the reduction and written after it.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, int64_t k, float* y) {
    const float* xr = x + (int64_t)blockIdx.x * k;
    float* yr = y + (int64_t)blockIdx.x * k;
    float inv[1];
    row_inv_rms<1>(xr, k, inv);
    for (int64_t i = threadIdx.x; i < k; i += 256) yr[i] = xr[i] * inv[0];
}

hipError_t launch_rmsnorm(const float* x, int64_t m, int64_t k, float* y, hipStream_t stream) {
    (void)hipGetLastError();
    rmsnorm_kernel<<<(unsigned)m, 256, 0, stream>>>(x, k, y);
    return hipGetLastError();
}

// ------------------------------------------- prologue fused with the quantizer

// The activation side of a Q8 x Q8 prefill product in one launch: each fp32
// row is scaled (by its inverse RMS for the norm prologue -- the reduction of
// q8_rmsnorm -- else by 1), rounded to bf16 and coded as Q8_0 blocks with the
// activation quantizer's rule.  One workgroup per row; thread t takes the
// eight-value groups t, t + 256, ... of the row, so a 32-value block is four
// consecutive threads and its maximum is combined over the quad.  A row of
// k <= 2048 is read once (the norm's registers are the values quantized).
// With FRAG the codes and scales go out in fragment order, one workgroup per
// row of the padded array (rows past m write zeros).
template <int PRO, bool FRAG>
__global__ __launch_bounds__(256) void act_prologue_quantize_kernel(const float* __restrict__ x, int64_t m,
                                                                    int64_t k, int8_t* __restrict__ xq,
                                                                    uint16_t* __restrict__ xd) {
    // Fragment order: workgroups are dealt round-robin to the eight XCDs, so
    // rows are mapped to make the 32 rows of a tile (which share every
    // kilobyte of the fragment array) run on one XCD and meet in its L2:
    // workgroup j of XCD x takes row 32 (8 (j / 32) + x) + j % 32.
    const int64_t row = FRAG ? ((int64_t)((blockIdx.x >> 8) * 8 + (blockIdx.x & 7)) * 32 + ((blockIdx.x >> 3) & 31))
                             : (int64_t)blockIdx.x;
    const int nb = (int)(k / 32);
    // fragment order (the int8 matrix core's operand layout, see
    // q8_prefill_frag.hip): 1 KB per (32-row tile, block), lane i + 32h holding
    // bytes 16h .. 16h + 15 of row i; scales [tile][block / 4][32][4]; blocks
    // up to nbp and the rows of the last 64-row group are written too, as zeros
    const int nbp = (nb + 3) / 4 * 4;
    const int64_t tile = row >> 5;
    const int ri = (int)(row & 31);
    if (FRAG && row >= (m + 63) / 64 * 64) return;     // past the padded array (grid rounded to 256)
    if (FRAG && row >= m) {
        for (int g = threadIdx.x; g < 4 * nbp; g += 256) {
            const int b = g >> 2, hh = (g >> 1) & 1;
            *reinterpret_cast<uint2*>(xq + ((tile * nbp + b) * 64 + hh * 32 + ri) * 16 + 8 * (g & 1)) =
                make_uint2(0u, 0u);
            if ((g & 3) == 0) xd[((tile * (nbp / 4) + b / 4) * 32 + ri) * 4 + (b & 3)] = 0;
        }
        return;
    }
    const float* xr = x + row * k;
    const bool one = k <= kStageK;                 // uniform: the row in registers
    float4 sv[1][2];
    stage_load<1>(xr, k, sv);
    float mul = 1.0f;
    if constexpr (PRO == kProNorm) {
        if (one) {
            float ss[1] = {8 * (int64_t)threadIdx.x < k ? sumsq8(sv[0][0], sv[0][1], 0.0f) : 0.0f};
            rms_finish<1>(ss, k, &mul);
        } else {
            row_inv_rms<1>(xr, k, &mul);
        }
    }
    // k is a multiple of 32: the four threads of a quad leave the loop together
    for (int64_t g = threadIdx.x; 8 * g < k; g += 256) {
        float4 a = sv[0][0], b = sv[0][1];
        if (!one) {
            const float4* p = reinterpret_cast<const float4*>(xr + 8 * g);
            a = p[0];
            b = p[1];
        }
        float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[e] = __uint_as_float((uint32_t)to_bf16(v[e] * mul) << 16);
            amax = fmaxf(amax, fabsf(v[e]));
        }
        amax = fmaxf(amax, dpp_f<0xB1>(amax));     // quad_perm [1,0,3,2]
        amax = fmaxf(amax, dpp_f<0x4E>(amax));     // quad_perm [2,3,0,1]
        const uint16_t sb = block_scale_bits(amax);
        const float s = half_bits_to_float(sb);
        uint32_t c[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            c[h] = ((uint32_t)block_code(v[4 * h], s) & 0xFFu) | (((uint32_t)block_code(v[4 * h + 1], s) & 0xFFu) << 8) |
                   (((uint32_t)block_code(v[4 * h + 2], s) & 0xFFu) << 16) |
                   ((uint32_t)block_code(v[4 * h + 3], s) << 24);
        if constexpr (FRAG) {
            const int64_t b = g >> 2;
            const int hh = (int)((g >> 1) & 1);
            *reinterpret_cast<uint2*>(xq + ((tile * nbp + b) * 64 + hh * 32 + ri) * 16 + 8 * (g & 1)) =
                make_uint2(c[0], c[1]);
            if ((threadIdx.x & 3) == 0) xd[((tile * (nbp / 4) + b / 4) * 32 + ri) * 4 + (b & 3)] = sb;
        } else {
            *reinterpret_cast<uint2*>(xq + row * k + 8 * g) = make_uint2(c[0], c[1]);
            if ((threadIdx.x & 3) == 0) xd[row * nb + g / 4] = sb;
        }
    }
    if constexpr (FRAG) {
        // the padding blocks nb .. nbp - 1 of this row
        for (int g = 4 * nb + threadIdx.x; g < 4 * nbp; g += 256) {
            const int b = g >> 2, hh = (g >> 1) & 1;
            *reinterpret_cast<uint2*>(xq + ((tile * nbp + b) * 64 + hh * 32 + ri) * 16 + 8 * (g & 1)) =
                make_uint2(0u, 0u);
            if ((g & 3) == 0) xd[((tile * (nbp / 4) + b / 4) * 32 + ri) * 4 + (b & 3)] = 0;
        }
    }
}

hipError_t launch_act_prologue_quantize(const float* x, int64_t m, int64_t k, int pro, int8_t* xq,
                                        uint16_t* xd, hipStream_t stream) {
    (void)hipGetLastError();
    if (pro == kProNorm)
        act_prologue_quantize_kernel<kProNorm, false><<<(unsigned)m, 256, 0, stream>>>(x, m, k, xq, xd);
    else
        act_prologue_quantize_kernel<kProF32, false><<<(unsigned)m, 256, 0, stream>>>(x, m, k, xq, xd);
    return hipGetLastError();
}

hipError_t launch_act_prologue_quantize_frag(const float* x, int64_t m, int64_t k, int pro, int8_t* xqf,
                                             uint16_t* xdf, hipStream_t stream) {
    (void)hipGetLastError();
    const int64_t rows = (m + 255) / 256 * 256;    // every row of the fragment array, padding included, in
                                                   // groups of eight tiles (one per XCD)
    if (pro == kProNorm)
        act_prologue_quantize_kernel<kProNorm, true><<<(unsigned)rows, 256, 0, stream>>>(x, m, k, xqf, xdf);
    else
        act_prologue_quantize_kernel<kProF32, true><<<(unsigned)rows, 256, 0, stream>>>(x, m, k, xqf, xdf);
    return hipGetLastError();
}

}  // namespace q8
