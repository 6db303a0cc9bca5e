// q8_prefill.hip -- Q8 x Q8 prefill product on the int8 matrix cores.
//
//   y[t][j] = sum_b wd[j][b] * xd[t][b] * isum[t][j][b],
//   isum[t][j][b] = sum_{i<32} wq[j][32b+i] * xq[t][32b+i]  (exact int32)
//
// [fak MODEL-BASELINE-RESULTS, ACT 4, "How the GEMM was closed": keep the
// block's int32 sum, fold each block into a float accumulator with one
// convert + scale step, register-block the output tile so every weight block
// serves several tokens and every activation block several rows.]
//
// On gfx950 a single v_mfma_i32_32x32x32_i8 covers exactly one 32-wide Q8 block
// of a 32 x 32 output tile, so the per-block int32 sums come straight out of the
// matrix core and are folded into fp32 accumulators by the vector ALUs.  Both
// operands are K-contiguous (codes [rows][K]), so each lane reads its 16-byte
// operand slice directly.  Workgroup tile: 64 activation rows x 64 weight rows,
// one 32 x 32 tile per wave; the K/32 scales of the tile are staged in LDS as
// fp32.
#include "q8_device.hpp"
#include "q8_internal.hpp"

namespace q8 {

constexpr int kPrefillKt = 64;   // blocks of scales staged per K tile

__global__ __launch_bounds__(256) void prefill_kernel(const int8_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ wd, int64_t n,
                                                      int nb, int64_t p,
                                                      const int8_t* __restrict__ xq,
                                                      const uint16_t* __restrict__ xd,
                                                      float* __restrict__ y) {
    __shared__ float xs_l[kPrefillKt * 64];
    __shared__ float ws_l[kPrefillKt * 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wp = wave & 1, wn = wave >> 1;
    const int64_t p0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    const int i = lane & 31, h = lane >> 5;
    const int64_t k = (int64_t)nb * 32;

    // The 32x32 result layout gives lane (i, h) rows 8*(r/4) + 4*h + r%4,
    // r = 0..15.  Operand row i is loaded from activation row pl(i) so that the
    // lane's 16 results are the 16 consecutive activation rows 16*h + r.
    const int pl = 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    const int64_t pa = p0 + 32 * wp + pl < p ? p0 + 32 * wp + pl : p - 1;
    const int64_t nbw = n0 + 32 * wn + i < n ? n0 + 32 * wn + i : n - 1;
    const int8_t* arow = xq + pa * k + 16 * h;
    const int8_t* brow = wq + nbw * k + 16 * h;

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const i32x16 zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    for (int b0 = 0; b0 < nb; b0 += kPrefillKt) {
        const int nblk = nb - b0 < kPrefillKt ? nb - b0 : kPrefillKt;
        __syncthreads();
        for (int idx = threadIdx.x; idx < 64 * nblk; idx += 256) {
            const int row = idx & 63, blk = idx >> 6;
            const int64_t pr = p0 + row < p ? p0 + row : p - 1;
            const int64_t nr = n0 + row < n ? n0 + row : n - 1;
            xs_l[blk * 64 + row] = half_bits_to_float(xd[pr * nb + b0 + blk]);
            ws_l[blk * 64 + row] = half_bits_to_float(wd[nr * nb + b0 + blk]);
        }
        __syncthreads();
        for (int bl = 0; bl < nblk; ++bl) {
            const int64_t off = (int64_t)(b0 + bl) * 32;
            const i32x4 A = *reinterpret_cast<const i32x4*>(arow + off);
            const i32x4 B = *reinterpret_cast<const i32x4*>(brow + off);
            const i32x16 c = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, zero, 0, 0, 0);
            const float wsc = ws_l[bl * 64 + 32 * wn + i];
            const float4* xs4 = reinterpret_cast<const float4*>(&xs_l[bl * 64 + 32 * wp + 16 * h]);
            const float4 s0 = xs4[0], s1 = xs4[1], s2 = xs4[2], s3 = xs4[3];
            const float xsv[16] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w,
                                   s2.x, s2.y, s2.z, s2.w, s3.x, s3.y, s3.z, s3.w};
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf((float)c[r], xsv[r] * wsc, acc[r]);
        }
    }

    const int64_t nout = n0 + 32 * wn + i;
    if (nout < n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t pout = p0 + 32 * wp + 16 * h + r;
            if (pout < p) y[pout * n + nout] = acc[r];
        }
    }
}

hipError_t launch_prefill(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t p,
                          const int8_t* xq, const uint16_t* xd, float* y,
                          const DeviceInfo& dev, hipStream_t stream) {
    (void)dev;
    const int nb = (int)(k / 32);
    const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((p + 63) / 64));
    (void)hipGetLastError();
    prefill_kernel<<<grid, 256, 0, stream>>>(wq, wd, n, nb, p, xq, xd, y);
    return hipGetLastError();
}

}  // namespace q8
