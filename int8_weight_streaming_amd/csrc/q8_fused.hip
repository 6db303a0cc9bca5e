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

}  // namespace q8
