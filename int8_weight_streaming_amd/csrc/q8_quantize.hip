// q8_quantize.hip -- Q8_0 block quantizers for fp32 weights and bf16 activations.
//
// One 32-element block is handled by 8 consecutive lanes, 4 elements each, so a
// wave covers 8 blocks: the fp32 input is read as one 1 KB contiguous span per
// wave instruction (bf16: 512 B), codes are written as one 256 B span and the
// eight binary16 scales as 16 B.  The block's largest magnitude is combined over
// the 8 lanes by DPP, then each lane rounds its own 4 values
// [fak MODEL-BASELINE-RESULTS, ACT 3 item 1 (format), ACT 4 "Correctness" and
// ACT 5 "What moved" item 3 (round half away from zero)].  HBM-bound.
#include "q8_device.hpp"
#include "q8_internal.hpp"

namespace q8 {

__device__ __forceinline__ void load4(const float* p, float v[4]) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}

__device__ __forceinline__ void load4(const uint16_t* p, float v[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
}

template <typename T>
__global__ __launch_bounds__(256) void quantize_kernel(const T* __restrict__ src, int64_t nblocks,
                                                       int8_t* __restrict__ q,
                                                       uint16_t* __restrict__ d) {
    const int sub = threadIdx.x & 7;
    const int64_t stride = ((int64_t)gridDim.x * blockDim.x) >> 3;
    // All 8 lanes of a block share `b`, so the loop exit is uniform per group
    // and the width-8 shuffles only ever read active lanes.
    for (int64_t b = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3; b < nblocks; b += stride) {
        float v[4];
        load4(src + b * 32 + sub * 4, v);
        float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        // maximum over the block's 8 lanes by DPP: xor 1 and xor 2 inside the
        // quad, then the half-row mirror (lane i of 8 with lane 7 - i, in the
        // other quad); a maximum is exact in any order
        a = fmaxf(a, dpp_f<0xB1>(a));
        a = fmaxf(a, dpp_f<0x4E>(a));
        a = fmaxf(a, dpp_f<0x141>(a));
        const uint16_t sb = block_scale_bits(a);
        const float s = half_bits_to_float(sb);
        const uint32_t c0 = (uint32_t)block_code(v[0], s) & 0xFFu;
        const uint32_t c1 = (uint32_t)block_code(v[1], s) & 0xFFu;
        const uint32_t c2 = (uint32_t)block_code(v[2], s) & 0xFFu;
        const uint32_t c3 = (uint32_t)block_code(v[3], s) & 0xFFu;
        *reinterpret_cast<uint32_t*>(q + b * 32 + sub * 4) = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
        if (sub == 0) d[b] = sb;
    }
}

static int quantize_grid(int64_t nblocks, const DeviceInfo& dev) {
    const int64_t want = (nblocks * 8 + 255) / 256;
    const int64_t cap = (int64_t)dev.cu_count * 16;
    return (int)(want < cap ? want : cap);
}

hipError_t launch_quantize_f32(const float* w, int64_t nblocks, int8_t* q, uint16_t* d,
                               const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
    quantize_kernel<float><<<quantize_grid(nblocks, dev), 256, 0, stream>>>(w, nblocks, q, d);
    return hipGetLastError();
}

hipError_t launch_quantize_bf16(const uint16_t* x, int64_t nblocks, int8_t* q, uint16_t* d,
                                const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
    quantize_kernel<uint16_t><<<quantize_grid(nblocks, dev), 256, 0, stream>>>(x, nblocks, q, d);
    return hipGetLastError();
}

}  // namespace q8
