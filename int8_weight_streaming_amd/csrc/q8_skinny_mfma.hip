// q8_skinny_mfma.hip -- batch 2..8 W8A16 (and W4A16) products on the bf16
// matrix cores.
//
//   y[m][j] = sum_b wd[j][b] * sum_{i<32} wq[j][32b+i] * x[m][32b+i]
//
// Above batch 2 the vector-ALU form of the decode product spends about four
// dot instructions per weight on the activation rows, more than the weight
// bytes cost at HBM speed [Frigg README, Finding 8: a batched kernel's cost
// should stay nearly flat in the batch size].  Here the multiply-adds go to the
// matrix cores: per 32-element block and 16 weight rows one
// v_mfma_f32_16x16x32_bf16 takes the activation rows as A (16 x 32; rows m and
// up read as zero) and the exactly converted weight codes as B (32 x 16), so
// its fp32 result D[m][j] is the block's dot product; the vector ALUs only
// convert the codes (int8 -> bf16 is exact) and fold each block with its scale
// (lane (j, g) holds D[4g .. 4g + 3][j], one weight row, so one scale per lane
// and block).
//
// Loads stay coalesced: a wave's 16 RGW (or 8) weight rows arrive four blocks
// (128 bytes per row; 64 for int4) at a time with full-line 16-byte loads,
// eight lanes per row (four for int4), are written to the wave's LDS slice
// (row pitch 136 bytes; 80) and read back as B fragments (8 bytes per lane:
// row j, bytes 8g .. 8g + 7 of the block; for int4 the nibbles of elements
// 8g .. 8g + 7; the activation fragment uses the same k positions).  Loading
// fragments straight from memory touches 16 rows x 32 bytes per instruction
// and streamed the lm_head at under 2 TB/s.  The next four blocks are in flight while the
// current ones are multiplied (or, with a step count fixed at compile time,
// all of a wave's blocks).  KS waves of a workgroup split K (contiguous
// block ranges) and add their partial results through LDS in a fixed order,
// so results are bitwise reproducible; no atomics.
#include "q8_device.hpp"
#include "q8_internal.hpp"

namespace q8 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kMPitch = 136;                      // LDS bytes per staged row of 4 blocks (128 + 8)
constexpr int kQ4Pitch = 80;                      // the same for int4 codes (64 + 16: 8-byte fragment
                                                  // reads of 16 rows hit distinct banks)

// Workgroup of W waves: W / KS sets of 16 RGW rows (8 with HALF: the B
// operand's columns 8..15 are zero, so short matrices get twice the
// workgroups), each set's K split over KS waves.  NSC > 0: every wave has
// exactly NSC four-block steps, all issued before the first is multiplied (the
// launch checks it); 0: any number, two in flight.  Q4: int4 weights (16
// bytes of codes per block, element i in the low nibble of byte i and element
// i + 16 in its high nibble); a nibble moved to the top of its byte reads as
// the int8 16 * code, converted as the Q8_0 codes are, and the scale is folded
// as d / 16 (exact).
template <int M, int RGW, int KS, int NT, int W, int NSC = 0, int HALF = 0, int Q4 = 0>
__global__ __launch_bounds__(64 * W) void skinny_mfma_kernel(const int8_t* __restrict__ wq,
                                                          const uint16_t* __restrict__ wd, int64_t n, int nb,
                                                          const uint16_t* __restrict__ x, float* __restrict__ y) {
    static_assert(M >= 1 && M <= 16, "activation rows fill at most the 16 rows of the A operand");
    static_assert(!HALF || RGW == 1, "a half fragment is one 8-row group");
    constexpr int RS = W / KS;                       // row sets per workgroup
    constexpr int ROWS = HALF ? 8 : 16 * RGW;        // rows per wave
    constexpr int RB = Q4 ? 16 : 32;                 // code bytes per block
    constexpr int PITCH = Q4 ? kQ4Pitch : kMPitch;   // LDS bytes per staged row
    constexpr int LPR = RB / 4;                      // copy lanes per row (16 bytes each, four blocks)
    constexpr int RPI = 64 / LPR;                    // rows per copy instruction
    constexpr int NLW = (ROWS + RPI - 1) / RPI;      // 16-byte weight loads per lane per step
    // a wave's slice holds its staged rows, and at the end its partial tile
    constexpr int SLICE = ROWS * PITCH > (int)sizeof(float) * 4 * RGW * 64 ? ROWS * PITCH
                                                                            : (int)sizeof(float) * 4 * RGW * 64;
    __shared__ __attribute__((aligned(16))) unsigned char lds[W][SLICE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int ks = wave % KS, rs = wave / KS;
    const int64_t n0 = ((int64_t)blockIdx.x * RS + rs) * ROWS;
    const int k = nb * 32;
    const int rowb = nb * RB;                        // code bytes per weight row
    const int nbw = nb / KS, b0 = ks * nbw;          // this wave's blocks
    // descriptors: weight rows past n and activation rows past M read as zero
    const int nv = n - n0 <= 0 ? 0 : (n - n0 < ROWS ? (int)(n - n0) : ROWS);
    const auto rW = range_rsrc32(wq + (nv ? n0 * rowb : 0), nv * rowb);
    const auto rS = range_rsrc32(wd + (nv ? n0 * nb : 0), nv * nb * 2);
    const auto rX = range_rsrc32(x, M * k * 2);
    const int j = lane & 15, g = lane >> 4;          // fragment lane: row / column j, k group g
    const int cr = lane / LPR, cc = lane % LPR;      // copy lane: rows cr + RPI t, 16-byte chunk cc
    unsigned char* const sl = lds[wave];

    struct Step {
        i32x4 w[NLW];
        i32x4 xv[4];
        i32x2 s[RGW];
    };
    auto issue = [&](int c, Step& st) {
        const int bb = b0 + 4 * c;
#pragma unroll
        for (int t = 0; t < NLW; ++t)
            st.w[t] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rW, (cr + RPI * t) * rowb + cc * 16, bb * RB, NT ? kLoadNT : 0));
#pragma unroll
        for (int u = 0; u < 4; ++u)
            st.xv[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, j * k * 2 + 16 * g,
                                                                                        (bb + u) * 64, 0));
#pragma unroll
        for (int r = 0; r < RGW; ++r)
            st.s[r] = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(rS, (16 * r + j) * nb * 2,
                                                                                      bb * 2, 0));
    };
    f32x4 acc[RGW];
#pragma unroll
    for (int r = 0; r < RGW; ++r) acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Step& st) {
        // LDS operations of one wave run in order: the previous step's fragment
        // reads are done before this write
#pragma unroll
        for (int t = 0; t < NLW; ++t)
            if (ROWS % RPI == 0 || cr + RPI * t < ROWS)   // (an int4 half fragment copies with half the lanes)
                *reinterpret_cast<i32x4*>(sl + (cr + RPI * t) * PITCH + cc * 16) = st.w[t];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int r = 0; r < RGW; ++r) {
                const int frow = 16 * r + (HALF ? (j & 7) : j);
                i32x2 wv;
                if constexpr (Q4) {
                    // elements 8g .. 8g + 7: bytes 8 (g & 1) .. + 7, low nibbles for g < 2
                    wv = *reinterpret_cast<const i32x2*>(sl + frow * PITCH + 16 * u + 8 * (g & 1));
                    const uint32_t w0 = (uint32_t)wv[0], w1 = (uint32_t)wv[1];
                    wv[0] = (int)((g < 2 ? w0 << 4 : w0) & 0xF0F0F0F0u);
                    wv[1] = (int)((g < 2 ? w1 << 4 : w1) & 0xF0F0F0F0u);
                } else {
                    wv = *reinterpret_cast<const i32x2*>(sl + frow * PITCH + 32 * u + 8 * g);
                }
                if (HALF && j >= 8) wv = (i32x2){0, 0};
                uint32_t b[4];
                i8x4_to_bf16x4((uint32_t)wv[0], b[0], b[1]);
                i8x4_to_bf16x4((uint32_t)wv[1], b[2], b[3]);
                const i32x4 bw = {(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
                const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.xv[u]),
                                                                        __builtin_bit_cast(bf16x8, bw), z, 0, 0, 0);
                const uint32_t sv = (uint32_t)st.s[r][u >> 1];
                const float ws = half_bits_to_float((uint16_t)((u & 1) ? (sv >> 16) : (sv & 0xFFFFu))) *
                                 (Q4 ? 0.0625f : 1.0f);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[r][q] = fmaf(d[q], ws, acc[r][q]);
            }
        }
    };
    if constexpr (NSC > 0) {
        // the wave's whole K slice in flight at once
        Step st[NSC];
#pragma unroll
        for (int c = 0; c < NSC; ++c) issue(c, st[c]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NSC; ++c) {
            compute(st[c]);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        // two steps of registers: step c + 1 is loading while step c is multiplied
        const int NS = nbw / 4;
        Step s0, s1;
        issue(0, s0);
        for (int c = 0; c < NS; c += 2) {
            if (c + 1 < NS) issue(c + 1, s1);
            __builtin_amdgcn_sched_barrier(0);
            compute(s0);
            __builtin_amdgcn_sched_barrier(0);
            if (c + 1 >= NS) break;
            if (c + 2 < NS) issue(c + 2, s0);
            __builtin_amdgcn_sched_barrier(0);
            compute(s1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (KS > 1) {
        // the K slices of a row set, added in wave order through LDS (the
        // slices' staging bytes are consumed)
        __syncthreads();
        float* part = reinterpret_cast<float*>(&lds[0][0]);
#pragma unroll
        for (int r = 0; r < RGW; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) part[((wave * RGW + r) * 4 + q) * 64 + lane] = acc[r][q];
        __syncthreads();
        if (ks != 0) return;
#pragma unroll
        for (int s = 1; s < KS; ++s)
#pragma unroll
            for (int r = 0; r < RGW; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[r][q] += part[(((wave + s) * RGW + r) * 4 + q) * 64 + lane];
    }
#pragma unroll
    for (int r = 0; r < RGW; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * g + q;
            const int64_t row = n0 + 16 * r + j;
            if (m < M && row < n && (!HALF || j < 8)) y[(int64_t)m * n + row] = acc[r][q];
        }
}

template <int M, int RGW, int KS, int NT, int W, int NSC = 0, int HALF = 0, int Q4 = 0>
hipError_t launch_cfg(const int8_t* wq, const uint16_t* wd, int64_t n, int nb, const void* x, float* y,
                      hipStream_t stream) {
    if (NSC > 0 && nb != 4 * KS * NSC) return hipErrorInvalidValue;
    const int64_t rows = (HALF ? 8 : 16 * RGW) * (W / KS);
    const int64_t grid = (n + rows - 1) / rows;
    skinny_mfma_kernel<M, RGW, KS, NT, W, NSC, HALF, Q4><<<(unsigned)grid, 64 * W, 0, stream>>>(
        wq, wd, n, nb, static_cast<const uint16_t*>(x), y);
    return hipGetLastError();
}

template <int M>
hipError_t launch_m(const int8_t* wq, const uint16_t* wd, int64_t n, int nb, const void* x, float* y,
                    const SkinnyLayout& L, hipStream_t stream) {
    // K = 1536 (48 blocks): each wave's step count fixed at compile time, all
    // its steps in flight (lm_head batch 8 82.9 -> 76.5 us; qkv / o / gate_up
    // 2-3% less); other K take the two-step loop
    if (L.r == 2)
        return nb == 48 ? launch_cfg<M, 2, 4, 1, 4, 3>(wq, wd, n, nb, x, y, stream)
                        : launch_cfg<M, 2, 4, 1, 4>(wq, wd, n, nb, x, y, stream);
    if (L.cpl == 12)
        return nb == 48 ? launch_cfg<M, 1, 12, 0, 12, 1>(wq, wd, n, nb, x, y, stream)
                        : launch_cfg<M, 1, 12, 0, 12>(wq, wd, n, nb, x, y, stream);
    if (L.cpl == 8) return launch_cfg<M, 1, 8, 0, 8, 0, 1>(wq, wd, n, nb, x, y, stream);
    return launch_cfg<M, 1, 4, 0, 4>(wq, wd, n, nb, x, y, stream);
}

}  // namespace

// The matrix-core form is used for bf16 activations where it measured faster
// than the vector-ALU form (graph replay, weights rotated past the caches):
// every shape at batch 5..8, and at batch 2..4 only matrices of at least 64
// rows per compute unit (the lm_head, batch 2: 71.1 against 79.8 us), where
// the vector form's per-weight arithmetic shows (qkv and gate_up at batch 2..4
// measured faster alone on the matrix cores but level or slower inside the
// decode step: 2.25 against 2.17 ms at batch 3).  Q8 activations keep the
// vector form (on the int8 matrix cores the step measured slower at every
// batch).  It needs K a multiple of 512 (whole four-block steps in each of the
// four K slices).  Tall matrices (4 or more 32-row
// workgroups per compute unit) use two 16-row groups per wave and
// non-temporal weight loads; shorter ones one group with K split over the
// waves of a workgroup: twelve ways when the 32-element blocks are a multiple
// of 48 (K = 1536: one four-block step per wave; qkv / o / gate_up at batch 8
// 4.85 / 3.85 / 5.45 against 4.99 / 4.09 / 5.58 us with four), else eight
// ways for K a multiple of 1024 below 32 rows per compute unit (the down
// projection, whose 1536 rows make few workgroups: 8-row half fragments
// double them, and at batch 8 it takes 6.0 us against 6.5 with 16-row
// fragments and 7.4 with a four-way split), else four.
bool skinny_mfma_applies(int64_t n, int64_t k, int m, int cu_count) {
    if (m < 2 || m > 8 || k % 512 != 0) return false;
    if (m >= 5) return true;
    return (n + 31) / 32 >= 2 * (int64_t)cu_count;
}
SkinnyLayout skinny_mfma_layout(int64_t n, int64_t k, int cu_count) {
    if ((n + 31) / 32 >= 4 * (int64_t)cu_count) return SkinnyLayout{16, 2, 4, true};
    if (k % 1536 == 0) return SkinnyLayout{16, 1, 12, true};
    if (k % 1024 == 0 && (n + 31) / 32 < (int64_t)cu_count) return SkinnyLayout{8, 1, 8, true};
    return SkinnyLayout{16, 1, 4, true};
}

hipError_t launch_skinny_mfma(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m, const void* x,
                              float* y, const DeviceInfo& dev, hipStream_t stream) {
    (void)hipGetLastError();
    const int nb = (int)(k / 32);
    const SkinnyLayout L = skinny_mfma_layout(n, k, dev.cu_count);
    switch (m) {
        case 2: return launch_m<2>(wq, wd, n, nb, x, y, L, stream);
        case 3: return launch_m<3>(wq, wd, n, nb, x, y, L, stream);
        case 4: return launch_m<4>(wq, wd, n, nb, x, y, L, stream);
        case 5: return launch_m<5>(wq, wd, n, nb, x, y, L, stream);
        case 6: return launch_m<6>(wq, wd, n, nb, x, y, L, stream);
        case 7: return launch_m<7>(wq, wd, n, nb, x, y, L, stream);
        case 8: return launch_m<8>(wq, wd, n, nb, x, y, L, stream);
        default: return hipErrorInvalidValue;
    }
}

// int4 weights (bf16 activations): the same kernel on 16-byte blocks of
// nibble codes.  Layouts (same sweeps, int4 lm_head and Mimir shapes at batch
// 2, 4 and 8, against the vector-ALU int4 products): the tall and twelve-way
// forms as for Q8_0; the long-K short matrices (down) with full 16-row
// fragments and an eight-way split (an int4 row is half the bytes, so half
// fragments gain nothing: 6.15 against 6.17 us at batch 8); used from batch 2
// except on that down layout below batch 5 and on tall matrices at batch 2,
// where the vector form is level or faster (int4 lm_head batch 2: 50.8 against
// 56.4 us; the int4 decode step at batch 4: 2.18 against 2.33 ms with the
// vector form below batch 5).  Batch 8 against the vector form: lm_head 60.8 /
// 97.5 us, qkv 4.65 / 6.72, o 3.66 / 4.90, gate_up 4.85 / 7.01, down 6.15 /
// 8.35.
SkinnyLayout q4_mfma_layout(int64_t n, int64_t k, int cu_count) {
    if ((n + 31) / 32 >= 4 * (int64_t)cu_count) return SkinnyLayout{16, 2, 4, true};
    if (k % 1536 == 0) return SkinnyLayout{16, 1, 12, true};
    if (k % 1024 == 0 && (n + 31) / 32 < (int64_t)cu_count) return SkinnyLayout{16, 1, 8, true};
    return SkinnyLayout{16, 1, 4, true};
}
bool q4_mfma_applies(int64_t n, int64_t k, int m, int cu_count) {
    if (m < 2 || m > 8 || k % 512 != 0) return false;
    const SkinnyLayout L = q4_mfma_layout(n, k, cu_count);
    return !(L.cpl == 8 && m <= 4) && !(L.r == 2 && m == 2);
}

namespace {
template <int M>
hipError_t q4_launch_m(const uint8_t* wq8, const uint16_t* wd, int64_t n, int nb, const void* x, float* y,
                       const SkinnyLayout& L, hipStream_t stream) {
    const int8_t* wq = reinterpret_cast<const int8_t*>(wq8);
    // tall: cached weight loads (a step reads 64 bytes of a row, half a line;
    // with non-temporal loads the other half was fetched again: 7% more HBM
    // bytes, lm_head batch 8 63.0 against 58.0 us)
    if (L.r == 2)
        return nb == 48 ? launch_cfg<M, 2, 4, 0, 4, 3, 0, 1>(wq, wd, n, nb, x, y, stream)
                        : launch_cfg<M, 2, 4, 0, 4, 0, 0, 1>(wq, wd, n, nb, x, y, stream);
    if (L.cpl == 12)
        return nb == 48 ? launch_cfg<M, 1, 12, 0, 12, 1, 0, 1>(wq, wd, n, nb, x, y, stream)
                        : launch_cfg<M, 1, 12, 0, 12, 0, 0, 1>(wq, wd, n, nb, x, y, stream);
    if (L.cpl == 8) return launch_cfg<M, 1, 8, 0, 8, 0, 0, 1>(wq, wd, n, nb, x, y, stream);
    return launch_cfg<M, 1, 4, 0, 4, 0, 0, 1>(wq, wd, n, nb, x, y, stream);
}
}  // namespace

hipError_t launch_q4_mfma(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m, const void* x,
                          float* y, const DeviceInfo& dev, hipStream_t stream) {
    const int nb = (int)(k / 32);
    const SkinnyLayout L = q4_mfma_layout(n, k, dev.cu_count);
    (void)hipGetLastError();
    switch (m) {
        case 2: return q4_launch_m<2>(wq, wd, n, nb, x, y, L, stream);
        case 3: return q4_launch_m<3>(wq, wd, n, nb, x, y, L, stream);
        case 4: return q4_launch_m<4>(wq, wd, n, nb, x, y, L, stream);
        case 5: return q4_launch_m<5>(wq, wd, n, nb, x, y, L, stream);
        case 6: return q4_launch_m<6>(wq, wd, n, nb, x, y, L, stream);
        case 7: return q4_launch_m<7>(wq, wd, n, nb, x, y, L, stream);
        case 8: return q4_launch_m<8>(wq, wd, n, nb, x, y, L, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace q8
