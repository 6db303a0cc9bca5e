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
// On gfx950 one v_mfma_i32_32x32x32_i8 covers exactly one 32-wide Q8 block of
// a 32 x 32 output tile, so every block sum comes straight from the matrix core
// as an exact int32.  The per-(t, j) scale product wd*xd of the same block is a
// rank-1 outer product: a v_mfma_f32_32x32x2_f32 with a single non-zero k term
// produces it in the same register layout, exactly (every binary16 value,
// subnormals included, is a normal fp32 number, and a product of two of them
// needs at most 22 significant bits).  The vector ALUs then only convert and
// accumulate: two operations per output and block.
//
// Work layout.  A workgroup computes one 32 x 32 output tile; its four waves
// take contiguous quarters of the K blocks (more waves in flight), and the four
// partial tiles are added through LDS in a fixed order, so results are bitwise
// reproducible.  Operands are K-contiguous (codes [rows][K]).  Each wave copies
// its 32 activation rows and 32 weight rows, four blocks (128 bytes) per row at
// a time, into its own LDS slice with full-cache-line 16-byte loads (eight
// lanes per row), prefetching the next four blocks into registers; the MFMA
// operand slices are then read from LDS (row pitch padded to 144 bytes so the
// 16-byte reads of 32 rows are bank-conflict free).  Gathering the operand
// slices straight from global memory touches 32 cache lines per instruction
// and measured 5-8x slower.  The next step is fetched into registers while the
// current one is multiplied.  The binary16 scales of the tile's rows (one
// contiguous range per operand) are copied to LDS once, coalesced, while the
// first step is in flight.
// Workgroups that share a weight tile get ids that land
// on the same XCD (ids are dealt round-robin to the 8 XCDs), so its L2 fetches
// each weight tile from HBM once.
#include "q8_device.hpp"
#include "q8_internal.hpp"

namespace q8 {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGroup = 4;                      // blocks per pipeline step (128 B per row)
constexpr int kPitch = 144;                    // LDS bytes per staged row (128 + 16 pad)
constexpr int kWaveSlice = 2 * 32 * kPitch;    // A and B rows of one wave: 9216 B

// One pipeline step of one wave: 16 bytes of each of 4 + 4 copied rows.
struct Stage {
    i32x4 a[4], b[4];
};
constexpr int kScaleBatch = 16;                // binary16 scales copied per thread per batch

__global__ __launch_bounds__(256) void prefill_kernel(const int8_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ wd, int64_t n,
                                                      int nb, int64_t p,
                                                      const int8_t* __restrict__ xq,
                                                      const uint16_t* __restrict__ xd,
                                                      float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int ntn = (int)((n + 31) / 32), ntp = (int)((p + 31) / 32);
    // id = xcd + 8 * (tp + ntp * c)  ->  weight tile tn = 8c + xcd, activation tile tp
    const int id = blockIdx.x;
    const int xcd = id & 7, rest = id >> 3;
    const int tp = rest % ntp, tn = 8 * (rest / ntp) + xcd;
    if (tn >= ntn) return;                             // whole padding workgroup leaves

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t p0 = (int64_t)tp * 32, n0 = (int64_t)tn * 32;
    const int64_t k = (int64_t)nb * 32;

    // ---- this wave's K range and LDS slice
    const int b_lo = (int)((int64_t)nb * wave / 4), b_hi = (int)((int64_t)nb * (wave + 1) / 4);
    const int nblk = b_hi - b_lo;
    unsigned char* slA = lds + wave * kWaveSlice;      // [32 rows][kPitch]
    unsigned char* slB = slA + 32 * kPitch;

    // copy lanes: lane l moves bytes 16*(l%8) of row 8*j + l/8 (j = 0..3)
    const int cr = lane >> 3, cb = (lane & 7) * 16;
    const int8_t* ga[4];
    const int8_t* gb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * j + cr;
        const int64_t pr = p0 + r < p ? p0 + r : p - 1;
        const int64_t nr = n0 + r < n ? n0 + r : n - 1;
        ga[j] = xq + pr * k;
        gb[j] = wq + nr * k;
    }

    // MFMA lanes: the 32x32 result layout gives lane (i, h) rows
    // 8*(r/4) + 4*h + r%4, r = 0..15; operand row i is taken from tile row pl(i)
    // so that the lane's 16 results are the 16 consecutive tile rows 16*h + r.
    const int i = lane & 31, h = lane >> 5;
    const int pl = 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    const bool lo_half = h == 0;
    // binary16 scales of the tile's 32 activation rows and 32 weight rows,
    // [row][nb] each, behind the four wave slices
    uint16_t* sA = reinterpret_cast<uint16_t*>(lds + 4 * kWaveSlice);
    uint16_t* sB = sA + 32 * nb;

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    const int ngroups = (nblk + kGroup - 1) / kGroup;
    auto fetch = [&](Stage& st, int g) {
        // 128 bytes of each copied row from block b_lo + 4g on; the offset is
        // clamped to the row so the last step never reads past it
        int64_t off = (int64_t)(b_lo + kGroup * g) * 32 + cb;
        off = off < k - 16 ? off : k - 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            st.a[j] = *reinterpret_cast<const i32x4*>(ga[j] + off);
            st.b[j] = *reinterpret_cast<const i32x4*>(gb[j] + off);
        }
    };
    const i32x16 zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const f32x16 zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // Step g: copy the staged step into the LDS slice, keep its scales, refill
    // the stage with step g + 1 (unconditionally: addresses are clamped in
    // bounds, so the compiler counts outstanding loads exactly), then multiply
    // step g (nothing past the wave's blocks).  LDS operations of one wave stay
    // in order, so the previous step's reads are done before this write.
    Stage st;
    fetch(st, 0);                                      // first step in flight ...
    {
        // ... while the scales are copied: the 32 rows of a tile are one
        // contiguous range of the scale array, so consecutive lanes read
        // consecutive scales; rows past the matrix get scale 0.
        const int64_t na = (int64_t)((p0 + 32 < p ? p0 + 32 : p) - p0) * nb;
        const int64_t nbv = (int64_t)((n0 + 32 < n ? n0 + 32 : n) - n0) * nb;
        const uint16_t* srcA = xd + p0 * nb;
        const uint16_t* srcB = wd + n0 * nb;
        const int total = 64 * nb;
        const int total_pad = (total + 255) & ~255;    // uniform trip counts, no masked lanes
        for (int e0 = 0; e0 < total_pad; e0 += 256 * kScaleBatch) {
            uint16_t v[kScaleBatch];
#pragma unroll
            for (int q = 0; q < kScaleBatch; ++q) {
                const int e = e0 + q * 256 + (int)threadIdx.x;
                const bool isb = e >= 32 * nb;
                const int64_t f = isb ? e - 32 * nb : e;
                const bool valid = e < total && f < (isb ? nbv : na);
                const uint16_t val = (isb ? srcB : srcA)[valid ? f : 0];   // index 0: row p0 / n0
                v[q] = valid ? val : (uint16_t)0;
            }
#pragma unroll
            for (int q = 0; q < kScaleBatch; ++q) {
                const int e = e0 + q * 256 + (int)threadIdx.x;
                sA[e < total_pad ? e : total_pad] = v[q];   // slot total_pad is scratch
            }
        }
    }
    __syncthreads();
    for (int g = 0; g < ngroups; ++g) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<i32x4*>(slA + (8 * j + cr) * kPitch + cb) = st.a[j];
            *reinterpret_cast<i32x4*>(slB + (8 * j + cr) * kPitch + cb) = st.b[j];
        }
        fetch(st, g + 1);
        const int nu = nblk - kGroup * g < kGroup ? nblk - kGroup * g : kGroup;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            if (u >= nu) break;                        // uniform across the wave
            const i32x4 a = *reinterpret_cast<const i32x4*>(slA + pl * kPitch + u * 32 + 16 * h);
            const i32x4 b = *reinterpret_cast<const i32x4*>(slB + i * kPitch + u * 32 + 16 * h);
            const i32x16 c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zi, 0, 0, 0);
            // scale outer product: lanes 0..31 carry k = 0, lanes 32..63 the zero k = 1
            const int blk = b_lo + kGroup * g + u;
            const float xs = lo_half ? half_bits_to_float(sA[pl * nb + blk]) : 0.0f;
            const float ws = lo_half ? half_bits_to_float(sB[i * nb + blk]) : 0.0f;
            const f32x16 t = __builtin_amdgcn_mfma_f32_32x32x2f32(xs, ws, zf, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf((float)c[r], t[r], acc[r]);
        }
    }

    // ---- combine the four partial tiles in a fixed order (wave 0 + 1 + 2 + 3)
    __syncthreads();                                   // every wave is done with its slice
    float* part = reinterpret_cast<float*>(lds);       // [3][16][64], reuses the slices
    if (wave > 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) part[((wave - 1) * 16 + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (wave == 0) {
        const int64_t nout = n0 + i;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float v = ((acc[r] + part[r * 64 + lane]) + part[(16 + r) * 64 + lane]) +
                            part[(32 + r) * 64 + lane];
            const int64_t pout = p0 + 16 * h + r;
            if (nout < n && pout < p) y[pout * n + nout] = v;
        }
    }
}

size_t prefill_lds_bytes(int64_t k) {
    const size_t total_pad = ((size_t)64 * (size_t)(k / 32) + 255) & ~(size_t)255;
    return 4 * (size_t)kWaveSlice + (total_pad + 2) * 2;
}

hipError_t prefill_prepare(const DeviceInfo& dev) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
}

hipError_t launch_prefill(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t p,
                          const int8_t* xq, const uint16_t* xd, float* y,
                          const DeviceInfo& dev, hipStream_t stream) {
    (void)dev;
    const int nb = (int)(k / 32);
    const int64_t ntn = (n + 31) / 32, ntp = (p + 31) / 32;
    const int64_t grid = 8 * ntp * ((ntn + 7) / 8);
    (void)hipGetLastError();
    const size_t lds = prefill_lds_bytes(k);
    prefill_kernel<<<(unsigned)grid, 256, lds, stream>>>(wq, wd, n, nb, p, xq, xd, y);
    return hipGetLastError();
}

}  // namespace q8
