// q8_attn.hip -- decode attention over a Q8_0 key/value cache.
//
//   s[j] = scale * sum_d q[h][d] * K[h][j][d],   w = softmax(s),
//   out[h][d] = sum_j w[j] * V[h][j][d],   j < t,
//
// one bf16 query row per head against t rows of a static cache slab
// [heads][t_cap][128] whose K and V are Q8_0 (int8 codes, one binary16 scale
// per 32 consecutive elements of a row) [Frigg README: "Masks" (the single
// decode query attends to every cached row unmasked), "Cache" (one static slab of
// [heads][4096][128] per virtual layer for K and for V), "The model, as
// verified" (12 heads of 128, multi-head attention), the bytes-per-token table
// (an int8 KV read per decoded token)].
//
// The cache read is the cost (2 x 136 bytes per row and head), so the kernel
// streams it once: up to 256 rows of context one workgroup takes all rows of a
// head (64, 128 or 256 of them) and writes the result itself; longer contexts
// are split into chunks of 64 rows of one head up to 512 rows, 128 up to 2048
// and 256 above (more, smaller workgroups measured faster at short contexts,
// fewer partials to combine at long ones);
// each of its four waves a quarter, lane l the 16-byte segment l % 8
// (dimensions 16 (l % 8) .. + 15, inside one Q8 block) of rows 8j + l / 8,
// j < RPL = 2, 4 or 8, for K and V alike, all loads issued before the first
// use.  A score is the bf16 dot of the query
// segment with the exactly converted codes, times the block scale, summed over
// the row's eight lanes by a fixed DPP tree.  The workgroup subtracts its
// maximum score, and writes (sum_j e^(s_j - m) V_j, m, sum_j e^(s_j - m)) to a
// caller-provided workspace; a second kernel combines the chunks of a head in
// chunk order (or the first kernel writes the result itself when one chunk
// covers the context).  Every reduction has a fixed order: results are
// bitwise reproducible.  Rows past t fall outside the buffer descriptors'
// range, read as zero and get weight zero.
#include "q8_device.hpp"
#include "q8_internal.hpp"

#include <mutex>

namespace q8 {

constexpr int kAttnD = 128;                    // head dimension
constexpr int64_t kAttnWholeTo = 256;          // contexts up to here: one chunk per head (64, 128 or 256 rows)
constexpr int64_t kAttnNarrowTo = 512;         // contexts up to here: 64-row chunks (two rows per lane)
constexpr int64_t kAttnWideFrom = 2048;        // above: 256-row chunks (eight); between: 128 (four)
constexpr int kAttnPart = kAttnPartFloats;      // floats per (head, chunk): o[128], m, l, 2 pad (16-byte records)
static_assert(kAttnPartFloats == kAttnD + 4, "partial record layout");

static int64_t attn_chunk_rows(int64_t t) {
    if (t <= kAttnWholeTo) return t <= 64 ? 64 : t <= 128 ? 128 : 256;
    return t <= kAttnNarrowTo ? 64 : t <= kAttnWideFrom ? 128 : 256;
}
// chunks the split uses for context t
int64_t attn_split_chunks(int64_t t) { return (t + attn_chunk_rows(t) - 1) / attn_chunk_rows(t); }
// the most chunks of any context up to t (1 up to 256 rows, 8 at 512, 16 at
// 2048), so a workspace sized for the longest context serves every shorter one
static int64_t attn_max_chunks(int64_t t) {
    int64_t c = attn_split_chunks(t);
    if (t > kAttnNarrowTo && c < attn_split_chunks(kAttnNarrowTo)) c = attn_split_chunks(kAttnNarrowTo);
    if (t > kAttnWideFrom && c < attn_split_chunks(kAttnWideFrom)) c = attn_split_chunks(kAttnWideFrom);
    return c;
}
int64_t attn_work_floats(int64_t heads, int64_t t) {
    const int64_t c = attn_max_chunks(t);
    return c > 1 ? heads * c * kAttnPart : 0;
}
int64_t attn_partial_floats(int64_t heads, int64_t t) { return heads * attn_max_chunks(t) * kAttnPart; }

// Maximum over each group of 32 lanes (exact in any order).
__device__ __forceinline__ float max32(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return xor16_max(v);
}

template <int RPL>
__global__ __launch_bounds__(256) void attn_split_kernel(const uint16_t* __restrict__ q,
                                                         int8_t* __restrict__ kq,
                                                         uint16_t* __restrict__ kd,
                                                         int8_t* __restrict__ vq,
                                                         uint16_t* __restrict__ vd,
                                                         int64_t t, int64_t t_cap, float scale,
                                                         int nchunks, float* __restrict__ work,
                                                         float* __restrict__ out,
                                                         const uint16_t* __restrict__ knew,
                                                         const uint16_t* __restrict__ vnew) {
    __shared__ float red[4][kAttnD + 2];
    const int h = (int)(blockIdx.x / (unsigned)nchunks), c = (int)(blockIdx.x % (unsigned)nchunks);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int seg = lane & 7, rsub = lane >> 3;

    // descriptors over the first t rows of head h (codes 128 B, scales 8 B per row)
    const int64_t hrow = (int64_t)h * t_cap;
    const auto rK = range_rsrc(kq + hrow * kAttnD, t * kAttnD);
    const auto rV = range_rsrc(vq + hrow * kAttnD, t * kAttnD);
    const auto rKs = range_rsrc(kd + hrow * (kAttnD / 32), t * (kAttnD / 32) * 2);
    const auto rVs = range_rsrc(vd + hrow * (kAttnD / 32), t * (kAttnD / 32) * 2);
    constexpr int WROWS = 8 * RPL;                                // rows per wave
    const int row0 = c * (4 * WROWS) + wave * WROWS + rsub;       // rows row0 + 8j, j < RPL

    // query segment: dimensions 16 seg .. 16 seg + 15 as eight bf16 pairs
    // (fetched first: small and cache resident)
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + (int64_t)h * kAttnD + 16 * seg);
    const u32x4 qa = qp[0], qb = qp[1];

    // A new row t - 1 (knew / vnew given) is appended by the workgroup of the
    // last chunk: thread i quantizes value i of [key row | value row] of head h
    // (its 32-value block is reduced over the 32 lanes that hold it; the
    // activation quantizer's rule), the codes meet in LDS, and the lanes of the
    // wave that covers row t - 1 write them into the cache and use them in place
    // of what the cache held there.  The bf16 value is fetched before the cache.
    const int rnew = (int)t - 1;
    const bool append = knew != nullptr && c == nchunks - 1;          // whole workgroup
    uint32_t nbits = 0;
    if (append) {
        const int i = threadIdx.x;
        nbits = (i < kAttnD ? knew : vnew)[(int64_t)h * kAttnD + (i & (kAttnD - 1))];
    }

    u32x4 kv[RPL], vv[RPL];
    uint32_t ks[RPL], vs[RPL];
    // keys and their scales first (the scores need only them), then values
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int row = row0 + 8 * j;
        kv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rK, row * kAttnD + 16 * seg, 0, kLoadNT));
        ks[j] = __builtin_amdgcn_raw_buffer_load_b16(rKs, row * 8 + 2 * (seg >> 1), 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);        // (the scheduler would group loads by type)
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int row = row0 + 8 * j;
        vv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rV, row * kAttnD + 16 * seg, 0, kLoadNT));
        vs[j] = __builtin_amdgcn_raw_buffer_load_b16(rVs, row * 8 + 2 * (seg >> 1), 0, 0);
    }
    if (append) {
        __shared__ __attribute__((aligned(16))) int8_t ncode[2 * kAttnD];
        __shared__ uint16_t nscale[2 * kAttnD / 32];
        pin(nbits);
        const float v = __uint_as_float(nbits << 16);
        const uint16_t sb = block_scale_bits(max32(fabsf(v)));
        ncode[threadIdx.x] = (int8_t)block_code(v, half_bits_to_float(sb));
        if ((threadIdx.x & 31) == 0) nscale[threadIdx.x >> 5] = sb;
        __syncthreads();
        if (wave == (rnew % (4 * WROWS)) / WROWS && rsub == (rnew & 7)) {
            const u32x4 kc = *reinterpret_cast<const u32x4*>(ncode + 16 * seg);
            const u32x4 vc = *reinterpret_cast<const u32x4*>(ncode + kAttnD + 16 * seg);
            const uint16_t ksb = nscale[seg >> 1], vsb = nscale[kAttnD / 32 + (seg >> 1)];
            const int jn = (rnew % WROWS) >> 3;
#pragma unroll
            for (int j = 0; j < RPL; ++j)
                if (j == jn) {
                    kv[j] = kc;
                    vv[j] = vc;
                    ks[j] = ksb;
                    vs[j] = vsb;
                }
            const int64_t crow = hrow + rnew;
            *reinterpret_cast<u32x4*>(kq + crow * kAttnD + 16 * seg) = kc;
            *reinterpret_cast<u32x4*>(vq + crow * kAttnD + 16 * seg) = vc;
            if ((seg & 1) == 0) {
                kd[crow * (kAttnD / 32) + (seg >> 1)] = ksb;
                vd[crow * (kAttnD / 32) + (seg >> 1)] = vsb;
            }
        }
    }

    const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};

    // ---- scores of the lane's four rows
    float s[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        uint32_t kb[8];
        i8x4_to_bf16x4(kv[j].x, kb[0], kb[1]);
        i8x4_to_bf16x4(kv[j].y, kb[2], kb[3]);
        i8x4_to_bf16x4(kv[j].z, kb[4], kb[5]);
        i8x4_to_bf16x4(kv[j].w, kb[6], kb[7]);
        float pa = 0.0f, pb = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pa = dot2_bf16(kb[e], qw[e], pa);
            pb = dot2_bf16(kb[4 + e], qw[4 + e], pb);
        }
        float v = (pa + pb) * half_bits_to_float((uint16_t)ks[j]);
        // sum over the row's eight lanes (xor 1, xor 2, half-row mirror)
        v += dpp_f<0xB1>(v);
        v += dpp_f<0x4E>(v);
        v += dpp_f<0x141>(v);
        s[j] = row0 + 8 * j < t ? v * scale : -INFINITY;
    }

    // ---- workgroup maximum
    float m = s[0];
#pragma unroll
    for (int j = 1; j < RPL; ++j) m = fmaxf(m, s[j]);
    m = fmaxf(m, dpp_f<0x128>(m));              // row_ror:8 = lane ^ 8 inside a row
    m = xor16_max(m);
    m = xor32_max(m);
    if (lane == 0) red[wave][kAttnD] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0][kAttnD], red[1][kAttnD]), fmaxf(red[2][kAttnD], red[3][kAttnD]));

    // ---- weights and the weighted value rows (lane: 16 dimensions)
    float o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.0f;
    float l = 0.0f;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const float p = expf(s[j] - m);                 // rows past t: exp(-inf) = 0
        l += p;
        const float pv = p * half_bits_to_float((uint16_t)vs[j]);
        const uint32_t w4[4] = {vv[j].x, vv[j].y, vv[j].z, vv[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[4 * e + 0] = fmaf(pv, (float)(int)(int8_t)(w4[e]), o[4 * e + 0]);
            o[4 * e + 1] = fmaf(pv, (float)(int)(int8_t)(w4[e] >> 8), o[4 * e + 1]);
            o[4 * e + 2] = fmaf(pv, (float)(int)(int8_t)(w4[e] >> 16), o[4 * e + 2]);
            o[4 * e + 3] = fmaf(pv, (float)((int)w4[e] >> 24), o[4 * e + 3]);
        }
    }
    // the eight row groups of the wave (lanes with equal seg), fixed tree
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        o[e] += dpp_f<0x128>(o[e]);
        o[e] = xor16_sum(o[e]);
        o[e] = xor32_sum(o[e]);
    }
    l += dpp_f<0x128>(l);
    l = xor16_sum(l);
    l = xor32_sum(l);
    if (rsub == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) red[wave][16 * seg + e] = o[e];
    }
    if (lane == 0) red[wave][kAttnD + 1] = l;   // every lane of a row group holds the same l
    __syncthreads();
    if (threadIdx.x < kAttnD) {
        const int d = threadIdx.x;
        const float od = ((red[0][d] + red[1][d]) + red[2][d]) + red[3][d];
        const float ls = ((red[0][kAttnD + 1] + red[1][kAttnD + 1]) + red[2][kAttnD + 1]) + red[3][kAttnD + 1];
        if (nchunks == 1 && out != nullptr) {
            out[(int64_t)h * kAttnD + d] = od / ls;
        } else {
            float* part = work + ((int64_t)h * nchunks + c) * kAttnPart;
            part[d] = od;
            if (d == 0) {
                part[kAttnD] = m;
                part[kAttnD + 1] = ls;
            }
        }
    }
}

// One workgroup per head, thread d: combine the chunks,
//   out = sum_c o_c e^(m_c - M) / sum_c l_c e^(m_c - M),  M = max_c m_c,
// every sum in chunk order.  Chunks are taken B at a time (4, 8, 16 or 32,
// the smallest that holds them; 32 per batch above that) with all loads of a
// batch in flight together: lane u (mod B) of each wave fetches
// chunk u's maximum and denominator and readlane hands them to every lane
// (uniform addresses would become scalar loads, of which few can be in
// flight); each thread fetches its own numerators.  Up to 32 chunks (4096
// rows) that is one round trip; longer contexts take the maximum over the
// batches first, then the sums.
constexpr int kCombBatch = 32;

template <int B>
struct CombBatch {
    float m[B], l[B], o[B];
};

template <int B>
__device__ __forceinline__ void load_batch(const float* w, int c0, int nchunks, int d, CombBatch<B>& b) {
    const int cu = c0 + (d & (B - 1)) < nchunks ? c0 + (d & (B - 1)) : nchunks - 1;   // in bounds; weight 0 below
    // (m, l) adjacent: one 8-byte load (kAttnPart is even, so it is aligned)
    const float2 ml = *reinterpret_cast<const float2*>(w + cu * kAttnPart + kAttnD);
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const int cc = c0 + u < nchunks ? c0 + u : nchunks - 1;
        b.o[u] = w[cc * kAttnPart + d];
    }
    __builtin_amdgcn_sched_barrier(0);        // every load of the batch before any use
#pragma unroll
    for (int u = 0; u < B; ++u) {
        b.m[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml.x), u));
        b.l[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml.y), u));
    }
}

template <int B>
__device__ __forceinline__ void sum_batch(const CombBatch<B>& b, int c0, int nchunks, float mx, float& num,
                                          float& den) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
        if (c0 + u < nchunks) {                 // uniform
            const float e = expf(b.m[u] - mx);
            num = fmaf(b.o[u], e, num);
            den = fmaf(b.l[u], e, den);
        }
    }
}

// nchunks <= B: one batch, one round trip
template <int B>
__device__ __forceinline__ float combine_one(const float* w, int nchunks, int d) {
    CombBatch<B> b;
    load_batch<B>(w, 0, nchunks, d, b);
    float mx = -INFINITY, num = 0.0f, den = 0.0f;
#pragma unroll
    for (int u = 0; u < B; ++u) mx = fmaxf(mx, b.m[u]);       // repeats of the last chunk change nothing
    sum_batch<B>(b, 0, nchunks, mx, num, den);
    return num / den;
}

__global__ __launch_bounds__(kAttnD) void attn_combine_kernel(const float* __restrict__ work,
                                                              int nchunks, float* __restrict__ out) {
    const int h = blockIdx.x, d = threadIdx.x;
    const float* w = work + (int64_t)h * nchunks * kAttnPart;
    float r;
    if (nchunks <= 4) {
        r = combine_one<4>(w, nchunks, d);
    } else if (nchunks <= 8) {
        r = combine_one<8>(w, nchunks, d);
    } else if (nchunks <= 16) {
        r = combine_one<16>(w, nchunks, d);
    } else if (nchunks <= kCombBatch) {
        r = combine_one<kCombBatch>(w, nchunks, d);
    } else {
        CombBatch<kCombBatch> b;
        float mx = -INFINITY, num = 0.0f, den = 0.0f;
        for (int c0 = 0; c0 < nchunks; c0 += kCombBatch) {
            load_batch<kCombBatch>(w, c0, nchunks, d, b);
#pragma unroll
            for (int u = 0; u < kCombBatch; ++u) mx = fmaxf(mx, b.m[u]);
        }
        for (int c0 = 0; c0 < nchunks; c0 += kCombBatch) {
            load_batch<kCombBatch>(w, c0, nchunks, d, b);
            sum_batch<kCombBatch>(b, c0, nchunks, mx, num, den);
        }
        r = num / den;
    }
    out[(int64_t)h * kAttnD + d] = r;
}

hipError_t launch_attn_decode(const uint16_t* q, int8_t* kq, uint16_t* kd, int8_t* vq, uint16_t* vd,
                              int64_t heads, int64_t t, int64_t t_cap, float scale, float* out,
                              float* work, const uint16_t* knew, const uint16_t* vnew,
                              const DeviceInfo& dev, hipStream_t stream) {
    (void)dev;
    const int64_t rows = attn_chunk_rows(t);
    const int nchunks = (int)attn_split_chunks(t);
    const unsigned grid = (unsigned)(heads * nchunks);
    (void)hipGetLastError();
    if (rows == 64)
        attn_split_kernel<2><<<grid, 256, 0, stream>>>(q, kq, kd, vq, vd, t, t_cap, scale, nchunks, work, out, knew,
                                                       vnew);
    else if (rows == 128)
        attn_split_kernel<4><<<grid, 256, 0, stream>>>(q, kq, kd, vq, vd, t, t_cap, scale, nchunks, work, out, knew,
                                                       vnew);
    else
        attn_split_kernel<8><<<grid, 256, 0, stream>>>(q, kq, kd, vq, vd, t, t_cap, scale, nchunks, work, out, knew,
                                                       vnew);
    if (nchunks > 1 && out != nullptr) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        attn_combine_kernel<<<(unsigned)heads, kAttnD, 0, stream>>>(work, nchunks, out);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ static scratch

// The chunk partials of the allocation-free entry point live here instead of a
// caller workspace.  Host code never passes this name to a kernel or a copy:
// on the host it only names the symbol, so its device address is looked up
// once per device (with that device current) and that address is used.
static __device__ __align__(256) float scratch[kAttnScratchFloats];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t attn_scratch(const DeviceInfo& dev, float** ptr) {
    if (dev.ordinal < 0 || dev.ordinal >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev.ordinal] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev.ordinal] = static_cast<float*>(p);
    }
    *ptr = g_scratch_ptr[dev.ordinal];
    return hipSuccess;
}

}  // namespace q8
