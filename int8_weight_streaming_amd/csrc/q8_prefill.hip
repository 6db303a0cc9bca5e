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
// rank-1 outer product, produced exactly by a matrix-core instruction with a
// single non-zero k term in the same register layout (a product of two
// binary16 numbers, subnormals included, needs at most 22 significant bits and
// lies in fp32's normal range).  The vector ALUs then only convert and
// accumulate: two operations per output and block.
//
// Work layout (both kernels).  A 32 x 32 output tile is computed by the four
// waves of a workgroup, each over a contiguous quarter of the K blocks, and the
// four partial tiles are added through LDS in a fixed order (wave 0 + 1 + 2 +
// 3), so results are bitwise reproducible and identical between the kernels.
// Operands are K-contiguous (codes [rows][K]); each wave copies its 32
// activation rows and 32 weight rows four blocks (128 bytes per row) at a time
// into its own LDS slice with full-cache-line 16-byte loads (eight lanes per
// row) and reads the MFMA operand slices from there (row pitch padded to 144
// bytes, so the 16-byte reads of 32 rows are bank-conflict free).  Gathering
// the operand slices straight from global memory touches 32 cache lines per
// instruction and measured 5-8x slower.
//
// prefill_stream_kernel (K a multiple of 512, every shape the model uses) is
// persistent: three workgroups per CU each walk a list of tiles, and the copy
// of the next four-block step (possibly the next tile's first) is in flight
// while the current one is multiplied, so the pipeline never drains between
// tiles.  Loads go through buffer descriptors built in scalar registers: the
// per-step advance is scalar arithmetic, rows past the matrix fall outside the
// descriptor's range and read as zero, and a step past the wave's last tile
// has an empty range and touches no memory.  The scale outer product is a
// v_mfma_f32_32x32x16_f16 on the raw binary16 scales (one operand holds the
// step's four activation scales in k = 0..3, the other one weight scale in
// the block's k slot), and the int8 product of
// the next block is issued before the fold of the current one, so the matrix
// core and the vector ALUs overlap.  Tiles are dealt so that the workgroups of
// one XCD (ids are dealt round-robin to the 8 XCDs) share its weight rows, so
// its L2 fetches each weight tile from HBM once.
//
// prefill_tile64_kernel (K a multiple of 256, enough tiles: the large-P
// kernel) computes a 64 x 64 tile per workgroup over all of K, below.
//
// prefill_kernel (any other K) computes one tile per workgroup, copies the
// tile's scales to LDS once, and uses v_mfma_f32_32x32x2_f32 for the outer
// product.
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

// ------------------------------------------------------------------ streaming

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kStreamSlice = 2 * 32 * kPitch;             // one wave's operand rows (scales stay in registers)
constexpr int kStreamLds = 4 * kStreamSlice;              // 36,864 B per workgroup
// three workgroups per CU: the kernel's 161 VGPRs leave room for three waves per
// SIMD (LDS would hold four workgroups: 4 x 36,864 B)
constexpr int kStreamWgPerCu = 3;
constexpr int64_t kStreamMaxK = int64_t(1) << 24;         // 32-bit buffer offsets

// One four-block step of one wave: 16 bytes of each of 4 + 4 copied rows, and
// the four binary16 scales of the lane's activation row and weight row.
struct StreamStage {
    i32x4 a[4], b[4];
    i32x2 sa, sb;
};

// gx workgroups per XCD; XCD x owns the weight tiles [ntn*x/8, ntn*(x+1)/8)
// and all activation tiles; workgroup j of an XCD takes its local tiles j,
// j + gx, j + 2 gx, ...  Requires nb % 16 == 0 (whole steps per wave).
__global__ __launch_bounds__(256) void prefill_stream_kernel(const int8_t* __restrict__ wq,
                                                             const uint16_t* __restrict__ wd,
                                                             int64_t n, int nb, int64_t p,
                                                             const int8_t* __restrict__ xq,
                                                             const uint16_t* __restrict__ xd,
                                                             float* __restrict__ y, int gx) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int ntn = (int)((n + 31) / 32), ntp = (int)((p + 31) / 32);
    const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
    const int tn_lo = (int)((int64_t)ntn * xcd / 8), tn_hi = (int)((int64_t)ntn * (xcd + 1) / 8);
    const int L = (tn_hi - tn_lo) * ntp;               // tiles of this XCD
    if (jw >= L) return;                               // whole workgroup leaves
    const int T = (L - jw + gx - 1) / gx;              // tiles of this workgroup
    const int S = nb / 16;                             // steps per wave and tile
    const int Q = T * S;
    const int64_t k = (int64_t)nb * 32;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // MFMA lanes: the 32x32 result layout gives lane (i, h) rows
    // 8*(r/4) + 4*h + r%4, r = 0..15; operand row i is taken from tile row pl(i)
    // so that the lane's 16 results are the 16 consecutive tile rows 16*h + r.
    const int i = lane & 31, h = lane >> 5;
    const int pl = 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    // copy lanes: lane l moves bytes 16*(l%8) of rows 8*j + l/8 (j = 0..3)
    const int cr = lane >> 3, cb = (lane & 7) * 16;
    unsigned char* slA = lds + wave * kStreamSlice;    // [32 rows][kPitch]
    unsigned char* slB = slA + 32 * kPitch;

    int voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) voff[j] = (8 * j + cr) * (int)k + cb;
    const int soffA = pl * nb * 2, soffB = i * nb * 2;

    // fetch cursor: the step whose loads are issued next (wave-uniform).  The
    // four buffer descriptors cover the cursor's tile (its rows of codes and
    // scales from column 0; an empty range once the workgroup's tiles are
    // done) and are rebuilt only when the cursor enters the next tile; a step
    // is addressed by the scalar offset of its first block, which stays below
    // the row length, so rows past the matrix read zero either way.
    int fs = 0, ft = 0, fm = jw;
    __amdgpu_buffer_rsrc_t rA, rB, rsA, rsB;
    auto enter_tile = [&]() {
        const bool live = ft < T;
        const int fp0 = (fm % ntp) * 32, fn0 = (tn_lo + fm / ntp) * 32;
        // ranges below 2^31 (rows <= 32, K <= 2^24): 32-bit range arithmetic
        const int pv = (int)(p - fp0 < 32 ? p - fp0 : 32);
        const int nv = (int)(n - fn0 < 32 ? n - fn0 : 32);
        const int kk = (int)k;
        rA = range_rsrc32(xq + (live ? (int64_t)fp0 * k : 0), live ? pv * kk : 0);
        rB = range_rsrc32(wq + (live ? (int64_t)fn0 * k : 0), live ? nv * kk : 0);
        rsA = range_rsrc32(xd + (live ? (int64_t)fp0 * nb : 0), live ? pv * nb * 2 : 0);
        rsB = range_rsrc32(wd + (live ? (int64_t)fn0 * nb : 0), live ? nv * nb * 2 : 0);
    };
    enter_tile();
    auto issue = [&](StreamStage& st) {
        const int blk0 = wave * 4 * S + 4 * fs;
        const int so = blk0 * 32, ss = blk0 * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            st.a[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, voff[j], so, 0));
            st.b[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, voff[j], so, 0));
        }
        st.sa = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(rsA, soffA, ss, 0));
        st.sb = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(rsB, soffB, ss, 0));
        if (++fs == S) {
            fs = 0;
            ++ft;
            fm += gx;
            enter_tile();
        }
    };

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const i32x16 zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const f32x16 zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int cs = 0, cm = jw;                               // compute cursor
    // scale operands: zero parts made opaque once, kept in registers
    i32x4 sta = {0, 0, 0, 0}, stb[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    asm volatile("" : "+v"(sta), "+v"(stb[0]), "+v"(stb[1]));

    // Step q: copy the staged step into the LDS slice, refill the stage with
    // step q + 1 (scheduling barriers keep every load in issue order, so the
    // compiler's counted waits stay exact), then multiply step q.  LDS
    // operations of one wave stay in order, so the previous step's reads are
    // done before this write.  (Two or three steps in flight measured slower
    // at every P: the kernel is not waiting on memory.)
    StreamStage st;
    issue(st);
    for (int q = 0; q < Q; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        // the lane's own scales (its operand rows) stay in registers
        const i32x2 ssa = st.sa, ssb = st.sb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<i32x4*>(slA + (8 * j + cr) * kPitch + cb) = st.a[j];
            *reinterpret_cast<i32x4*>(slB + (8 * j + cr) * kPitch + cb) = st.b[j];
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(st);
        __builtin_amdgcn_sched_barrier(0);

        // Scale outer product of block u: operand A holds the four blocks'
        // activation scales in k = 0..3 (k = 4..15 zero), operand B the weight
        // scale of block u in k = u only (zero on lanes 32..63, which carry
        // k = 8..15), so the single product is xs_u * ws_u.
        sta[0] = ssa[0];
        sta[1] = ssa[1];
        const int sb0 = h ? 0 : ssb[0], sb1 = h ? 0 : ssb[1];
        i32x4 av[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            av[u] = *reinterpret_cast<const i32x4*>(slA + pl * kPitch + u * 32 + 16 * h);
            bv[u] = *reinterpret_cast<const i32x4*>(slB + i * kPitch + u * 32 + 16 * h);
        }
        auto mm = [&](int u, i32x16& c, f32x16& t) {
            const int wb = (u >> 1) ? sb1 : sb0;
            const int half = (u & 1) ? (wb & (int)0xFFFF0000u) : (wb & 0xFFFF);
            stb[u & 1][0] = (u >> 1) ? 0 : half;
            stb[u & 1][1] = (u >> 1) ? half : 0;
            c = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[u], bv[u], zi, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, sta),
                                                        __builtin_bit_cast(f16x8, stb[u & 1]), zf, 0, 0, 0);
        };
        auto fold = [&](const i32x16& c, const f32x16& t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf((float)c[r], t[r], acc[r]);
        };
        // blocks 0..3, the matrix products of block u + 1 in flight while
        // block u is folded
        i32x16 c0, c1;
        f32x16 t0, t1;
        mm(0, c0, t0);
        __builtin_amdgcn_sched_barrier(0);
        mm(1, c1, t1);
        __builtin_amdgcn_sched_barrier(0);
        fold(c0, t0);
        __builtin_amdgcn_sched_barrier(0);
        mm(2, c0, t0);
        __builtin_amdgcn_sched_barrier(0);
        fold(c1, t1);
        __builtin_amdgcn_sched_barrier(0);
        mm(3, c1, t1);
        __builtin_amdgcn_sched_barrier(0);
        fold(c0, t0);
        __builtin_amdgcn_sched_barrier(0);
        fold(c1, t1);

        if (++cs == S) {
            // tile done: the four partial tiles go through the waves' own
            // slices (their operand data is consumed), each wave adds and
            // stores four of the sixteen result rows, wave 0 + 1 + 2 + 3
            cs = 0;
            float* mine = reinterpret_cast<float*>(slA);
#pragma unroll
            for (int r = 0; r < 16; ++r) mine[r * 64 + lane] = acc[r];
            __syncthreads();
            const int64_t p0 = (int64_t)(cm % ntp) * 32, n0 = (int64_t)(tn_lo + cm / ntp) * 32;
            const int64_t nout = n0 + i;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 4 * wave + rr;
                float v = reinterpret_cast<const float*>(lds)[r * 64 + lane];
#pragma unroll
                for (int w = 1; w < 4; ++w)
                    v += reinterpret_cast<const float*>(lds + w * kStreamSlice)[r * 64 + lane];
                const int64_t pout = p0 + 16 * h + r;
                if (nout < n && pout < p) y[pout * n + nout] = v;
            }
            __syncthreads();                           // slices free for the next step
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
            cm += gx;
        }
    }
}

// ------------------------------------------------------------------ 64 x 64 tiles

// prefill_tile64_kernel<KS>: a workgroup computes a 64 x 64 output tile with
// KS groups of four waves; each group takes a contiguous 1/KS of the K steps
// and its four waves the 2 x 2 subtiles of 32 x 32, so every staged operand
// row serves two waves.  With KS = 2 the groups' partial tiles are added in
// LDS in a fixed order (group 0 + group 1) at the end; it is for shapes with
// few tiles, where it halves each wave's chain of steps and puts twice as many
// waves on every SIMD.  A step is four blocks (128 bytes of each of the 64 +
// 64 rows plus their scales): each thread loads 4 x 16 bytes of rows t/8 and t/8 + 32 of
// both operands (8 threads per 128-byte row segment) and wave 0 / 1 load the
// 8 bytes of scales of one activation / weight row per lane, all through
// buffer descriptors (rows past the matrix read as zero; a step past K has an
// empty range).  Two steps are in flight in registers while a third is
// multiplied from one of two LDS buffers; one barrier per step.
constexpr int kT64Rows = 64;
constexpr int kT64Buf = 2 * kT64Rows * kPitch + 2 * kT64Rows * 8;   // one LDS buffer: 19,456 B
constexpr int kT64Lds = 2 * kT64Buf;               // per group of four waves

struct T64Stage {
    i32x4 a[2], b[2];
    i32x2 s;
};

// Register use is held to four waves per SIMD (128 VGPRs): measured faster
// than two or three waves with deeper per-wave overlap.
template <int KS>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(4, 4)))
void prefill_tile64_kernel(const int8_t* __restrict__ wq,
                           const uint16_t* __restrict__ wd,
                           int64_t n, int nb, int64_t p,
                           const int8_t* __restrict__ xq,
                           const uint16_t* __restrict__ xd,
                           float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int ntn = (int)((n + 63) / 64), ntp = (int)((p + 63) / 64);
    // id = xcd + 8 * (tp + ntp * c)  ->  weight tile tn = 8c + xcd, activation tile tp
    const int id = blockIdx.x;
    const int xcd = id & 7, rest = id >> 3;
    const int tp = rest % ntp, tn = 8 * (rest / ntp) + xcd;
    if (tn >= ntn) return;                             // whole padding workgroup leaves

    const int lane = threadIdx.x & 63;
    const int wg = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int grp = wg >> 2, wave = wg & 3;            // K group, wave inside the group
    const int64_t p0 = (int64_t)tp * 64, n0 = (int64_t)tn * 64;
    const int64_t k = (int64_t)nb * 32;
    const int64_t pv = p - p0 < 64 ? p - p0 : 64, nv = n - n0 < 64 ? n - n0 : 64;
    const int S = nb / (4 * KS);                       // steps of this group; even
    const int step0 = grp * S;                         // its first step over all of K
    unsigned char* const glds = lds + grp * kT64Lds;

    // copy lanes: thread t of the group moves bytes 16*(t%8) of rows t/8 and t/8 + 32
    const int tg = (int)(threadIdx.x & 255);
    const int cr = tg >> 3, cb = (tg & 7) * 16;
    const int voff0 = cr * (int)k + cb, voff1 = (cr + 32) * (int)k + cb;
    // scale lanes: wave 0 the activation rows, wave 1 the weight rows
    const int soff = lane * nb * 2;

    // Descriptor state of step 0 of this group; a step advances every base by
    // 128 code bytes (4 scales) and shrinks every range by as much.
    const int8_t* const a0 = xq + p0 * k + (int64_t)step0 * 128;
    const int8_t* const b0 = wq + n0 * k + (int64_t)step0 * 128;
    // (ranges below 2^31: rows <= 64, K <= 2^24)
    const int arec = (int)(pv * k - (int64_t)step0 * 128), brec = (int)(nv * k - (int64_t)step0 * 128);
    const uint16_t* const s0 = (wave == 0 ? xd + p0 * nb : wd + n0 * nb) + (int64_t)step0 * 4;
    const int srec = wave > 1 ? 0 : (int)(((wave == 0 ? pv : nv) * nb - (int64_t)step0 * 4) * 2);
    auto issue = [&](int lstep, T64Stage& st) {
        const bool live = lstep < S;
        const int adv = lstep * 128;
        const auto rA = range_rsrc32(a0 + adv, live ? arec - adv : 0);
        const auto rB = range_rsrc32(b0 + adv, live ? brec - adv : 0);
        const auto rS = range_rsrc32(s0 + lstep * 4, live ? srec - lstep * 8 : 0);
        st.a[0] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, voff0, 0, 0));
        st.a[1] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, voff1, 0, 0));
        st.b[0] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, voff0, 0, 0));
        st.b[1] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, voff1, 0, 0));
        st.s = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(rS, soff, 0, 0));
    };
    // LDS buffer: A rows [64][kPitch], B rows [64][kPitch], A scales [64][8 B], B scales [64][8 B]
    auto put = [&](int buf, const T64Stage& st) {
        unsigned char* base = glds + buf * kT64Buf;
        *reinterpret_cast<i32x4*>(base + cr * kPitch + cb) = st.a[0];
        *reinterpret_cast<i32x4*>(base + (cr + 32) * kPitch + cb) = st.a[1];
        *reinterpret_cast<i32x4*>(base + (64 + cr) * kPitch + cb) = st.b[0];
        *reinterpret_cast<i32x4*>(base + (96 + cr) * kPitch + cb) = st.b[1];
        if (wave < 2)
            *reinterpret_cast<i32x2*>(base + 128 * kPitch + (wave * 64 + lane) * 8) = st.s;
    };

    // MFMA lanes (same layout as the other kernels): lane (i, h) ends with the
    // 16 consecutive tile rows 16h + r of column i of its wave's subtile.
    const int i = lane & 31, h = lane >> 5;
    const int pl = 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    const int wp = wave & 1, wn = wave >> 1;
    const int arow = 32 * wp + pl, brow = 64 + 32 * wn + i;
    const int sa_off = 128 * kPitch + arow * 8, sb_off = 128 * kPitch + (64 + 32 * wn + i) * 8;

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const i32x16 zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const f32x16 zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // Scale outer product of block u: operand A holds the four blocks'
    // activation scales in k = 0..3 (the row's 8 raw bytes; k = 4..15 zero),
    // operand B the weight scale of block u in k = u only (zero on lanes
    // 32..63, which carry k = 8..15), so the single product is xs_u * ws_u.
    // The zero parts of both operands are set once and never written again.
    // (The zero halves are made opaque once, so the compiler keeps them in
    // registers instead of writing zeros again for every block.)
    i32x4 sta = {0, 0, 0, 0}, stb = {0, 0, 0, 0};
    asm volatile("" : "+v"(sta), "+v"(stb));
    auto compute = [&](int buf) {
        const unsigned char* base = glds + buf * kT64Buf;
        const i32x2 sa = *reinterpret_cast<const i32x2*>(base + sa_off);
        const i32x2 sb = *reinterpret_cast<const i32x2*>(base + sb_off);
        sta[0] = sa[0];
        sta[1] = sa[1];
        const int sb0 = h ? 0 : sb[0], sb1 = h ? 0 : sb[1];
        auto mm = [&](int u, i32x16& c, f32x16& t) {
            const i32x4 av = *reinterpret_cast<const i32x4*>(base + arow * kPitch + u * 32 + 16 * h);
            const i32x4 bv = *reinterpret_cast<const i32x4*>(base + brow * kPitch + u * 32 + 16 * h);
            const int wb = (u >> 1) ? sb1 : sb0;
            const int half = (u & 1) ? (wb & (int)0xFFFF0000u) : (wb & 0xFFFF);
            stb[0] = (u >> 1) ? 0 : half;
            stb[1] = (u >> 1) ? half : 0;
            c = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, zi, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, sta),
                                                        __builtin_bit_cast(f16x8, stb), zf, 0, 0, 0);
        };
        auto fold = [&](const i32x16& c, const f32x16& t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf((float)c[r], t[r], acc[r]);
        };
        // one block's products at a time: the other waves of the SIMD keep the
        // matrix core and the vector ALUs busy meanwhile
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            i32x16 c;
            f32x16 t;
            mm(u, c, t);
            fold(c, t);
        }
    };

    // The folds of a step are finished before its barrier (an empty asm that
    // takes the accumulators as operands), so the matrix products of different
    // steps are never live together.
    auto pin = [&]() {
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(acc[r]));
    };
    T64Stage ra, rb;
    issue(0, ra);
    issue(1, rb);
    put(0, ra);
    issue(2, ra);
    __syncthreads();
    for (int s0 = 0; s0 < S; s0 += 2) {
        put(1, rb);                                    // step s0 + 1 (S is even)
        issue(s0 + 3, rb);
        compute(0);                                    // step s0
        pin();
        __syncthreads();
        if (s0 + 2 < S) put(0, ra);                    // step s0 + 2
        issue(s0 + 4, ra);
        compute(1);                                    // step s0 + 1
        pin();
        __syncthreads();
    }

    if (KS > 1) {
        // groups 1.. leave their partial tiles in their own LDS (their operand
        // buffers are consumed); group 0 adds them in group order and stores
        if (grp > 0) {
            float* part = reinterpret_cast<float*>(glds) + wave * 16 * 64;
#pragma unroll
            for (int r = 0; r < 16; ++r) part[r * 64 + lane] = acc[r];
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int g = 1; g < KS; ++g) {
            const float* part = reinterpret_cast<const float*>(lds + g * kT64Lds) + wave * 16 * 64;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] += part[r * 64 + lane];
        }
    }
    // rows 16h + r of column i of subtile (wp, wn)
    const int64_t nout = n0 + 32 * wn + i;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t pout = p0 + 32 * wp + 16 * h + r;
        if (nout < n && pout < p) y[pout * n + nout] = acc[r];
    }
}

static bool use_stream(int64_t n, int64_t k, int64_t p) {
    const int64_t ntn = (n + 31) / 32, ntp = (p + 31) / 32;
    return k % 512 == 0 && k <= kStreamMaxK && ntn * ntp < (int64_t(1) << 31) &&
           32 * ntp < (int64_t(1) << 31) && 32 * ntn < (int64_t(1) << 31);
}

// Kernel choice, measured on the P = 256 .. 4096 Mimir products: the 64 x 64
// kernel with one group of waves from four 64 x 64 tiles per compute unit on
// (K a multiple of 256), with K split over two groups from 1.5 tiles per
// compute unit on (K a multiple of 512); below that the streaming kernel
// (K a multiple of 512) or the one-tile kernel.  Returns the number of groups,
// or 0 for the other kernels.
static int tile64_split(int64_t n, int64_t k, int64_t p, int cu_count) {
    const int64_t ntn = (n + 63) / 64, ntp = (p + 63) / 64;
    const int64_t grid = 8 * ntp * ((ntn + 7) / 8);
    if (k % 256 != 0 || k > kStreamMaxK || grid >= (int64_t(1) << 31)) return 0;
    const int64_t tiles = ntn * ntp;
    if (tiles >= 4 * (int64_t)cu_count) return 1;
    if (2 * tiles >= 3 * (int64_t)cu_count && k % 512 == 0) return 2;
    if (tiles >= (int64_t)cu_count && k % 512 != 0) return 1;
    return 0;
}

int prefill_kind(int64_t n, int64_t k, int64_t p, int cu_count) {
    if (const int ks = tile64_split(n, k, p, cu_count)) return ks == 1 ? kPrefillTile64x1 : kPrefillTile64x2;
    return use_stream(n, k, p) ? kPrefillStream : kPrefillTile32;
}

size_t prefill_lds_bytes(int64_t n, int64_t k, int64_t p, const DeviceInfo& dev) {
    if (const int ks = tile64_split(n, k, p, dev.cu_count)) return (size_t)ks * kT64Lds;
    if (k % 512 == 0 && k <= kStreamMaxK) return (size_t)kStreamLds;
    const size_t total_pad = ((size_t)64 * (size_t)(k / 32) + 255) & ~(size_t)255;
    return 4 * (size_t)kWaveSlice + (total_pad + 2) * 2;
}

hipError_t prefill_prepare(const DeviceInfo& dev) {
    const void* fns[2] = {reinterpret_cast<const void*>(&prefill_kernel),
                          reinterpret_cast<const void*>(&prefill_tile64_kernel<2>)};
    for (const void* f : fns) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_prefill(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t p,
                          const int8_t* xq, const uint16_t* xd, float* y,
                          const DeviceInfo& dev, hipStream_t stream) {
    const int nb = (int)(k / 32);
    const int64_t ntn = (n + 31) / 32, ntp = (p + 31) / 32;
    (void)hipGetLastError();
    if (const int ks = tile64_split(n, k, p, dev.cu_count)) {
        const int64_t ntn64 = (n + 63) / 64, ntp64 = (p + 63) / 64;
        const unsigned grid = (unsigned)(8 * ntp64 * ((ntn64 + 7) / 8));
        if (ks == 1)
            prefill_tile64_kernel<1><<<grid, 256, kT64Lds, stream>>>(wq, wd, n, nb, p, xq, xd, y);
        else
            prefill_tile64_kernel<2><<<grid, 512, 2 * kT64Lds, stream>>>(wq, wd, n, nb, p, xq, xd, y);
        return hipGetLastError();
    }
    if (use_stream(n, k, p)) {
        const int64_t per_xcd = ((ntn + 7) / 8) * ntp;          // most tiles of one XCD
        int64_t gx = (int64_t)(dev.cu_count / 8 > 0 ? dev.cu_count / 8 : 1) * kStreamWgPerCu;
        if (gx > per_xcd) gx = per_xcd;
        prefill_stream_kernel<<<(unsigned)(8 * gx), 256, kStreamLds, stream>>>(
            wq, wd, n, nb, p, xq, xd, y, (int)gx);
        return hipGetLastError();
    }
    const int64_t grid = 8 * ntp * ((ntn + 7) / 8);
    const size_t lds = prefill_lds_bytes(n, k, p, dev);
    prefill_kernel<<<(unsigned)grid, 256, lds, stream>>>(wq, wd, n, nb, p, xq, xd, y);
    return hipGetLastError();
}

}  // namespace q8
