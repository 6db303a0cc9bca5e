// q8_probe.hip -- measurement probes of the benchmark (libq8probe.so; not part
// of the q8stream library).
//
//  * HBM read probe.  Streams a buffer with the access pattern of the decode
//    product at its best: every workgroup reads one contiguous span of
//    256 x LPT x 16 bytes, each thread issues all of its LPT 16-byte
//    non-temporal loads before it uses any (the decode product issues a whole
//    K tile of a row group the same way), and the grid has one workgroup per
//    span, so the hardware keeps as many spans in flight as occupancy allows.
//    LPT (loads per thread) is a parameter; the benchmark sweeps it and takes
//    the fastest as the measured read peak.
//  * Grid-barrier probe: what one dependency edge would cost inside a single
//    persistent launch, against a graph-replayed launch boundary.
//  * int8 matrix-core probe: independent chains of v_mfma_i32_32x32x32_i8 per
//    wave, so the sustained int8 rate of the chip (at whatever clock it holds
//    under that load) can be quoted beside the published peak.
//  * Exact-fold probe: the arithmetic of a Q8 x Q8 block-tile (int8 block
//    sums, scale outer product, fp32 fold) with no memory traffic, the rate
//    any exact per-block prefill kernel is bounded by.
#include "q8probe.h"
#include "q8_device.hpp"

#include <hip/hip_runtime.h>

namespace {

// ---- HBM read probe

template <int LPT>
__global__ __launch_bounds__(256) void probe_read_kernel(const q8::u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * (256 * LPT) + threadIdx.x;
    q8::u32x4 v[LPT];
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int64_t i = base + 256 * j;
        v[j] = __builtin_nontemporal_load(src + (i < n16 ? i : n16 - 1));
    }
    q8::u32x4 acc = v[0];
#pragma unroll
    for (int j = 1; j < LPT; ++j) acc ^= v[j];
    const uint32_t s = acc.x ^ acc.y ^ acc.z ^ acc.w;
    // one word per workgroup keeps the loads live; lane 0 of wave 0 writes it
    // only if the xor of everything is a value no buffer here produces
    if (s == 0x9E3779B9u && threadIdx.x == 0) sink[0] = s;
}

// ---- grid-barrier probe

constexpr int kBarReplicas = 8;                // one flag array per XCD
constexpr int kBarStride = 1024;               // words per replica (>= workgroups)
constexpr unsigned kBarSpinLimit = 1u << 22;
constexpr int kBarErr = kBarReplicas * kBarStride;   // index of the error word

__device__ __forceinline__ unsigned coherent_load(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave per workgroup.  Epochs continue from the value this workgroup's own
// flag holds (every flag holds the same epoch between calls).
__global__ __launch_bounds__(64) void probe_barrier_kernel(unsigned* __restrict__ flags, int rounds) {
    const int g = blockIdx.x, lane = threadIdx.x, nwg = gridDim.x;
    const unsigned* mine = flags + (g % kBarReplicas) * kBarStride;
    unsigned epoch = coherent_load(flags + g);
    for (int r = 0; r < rounds; ++r) {
        ++epoch;
        if (lane < kBarReplicas) coherent_store(flags + lane * kBarStride + g, epoch);
        unsigned spins = 0;
        bool done = false;
        while (!done) {
            bool all = true;
            for (int i = lane; i < nwg; i += 64) all = all && (int)(coherent_load(mine + i) - epoch) >= 0;
            done = __all(all);
            if (!done && (coherent_load(flags + kBarErr) != 0u || ++spins > kBarSpinLimit)) {
                if (lane == 0) coherent_store(flags + kBarErr, 1u);
                return;                                 // every wave leaves
            }
        }
    }
}

// ---- int8 matrix-core probe

// Eight independent accumulation chains per wave, `iters` rounds of eight
// v_mfma_i32_32x32x32_i8 each (65,536 integer operations per instruction).
// The result is written only under a condition the operands never meet, so the
// chains stay live without a store per wave.
__global__ __launch_bounds__(256) void probe_mfma_i8_kernel(int iters, int* __restrict__ sink) {
    const int l = threadIdx.x;
    const q8::i32x4 a = {l, l + 1, l + 2, l + 3};
    q8::i32x16 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = (q8::i32x16){};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c[j], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s ^= c[j][0] ^ c[j][15];
    if (s == 0x7FEDCBA9 && l == 0) sink[0] = s;
}

// ---- exact-fold probe

typedef float f32x16p __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8p __attribute__((ext_vector_type(8)));

// A hash of 32-bit words for the probe's operands (an integer finalizer:
// xor-shift, multiply, xor-shift, multiply, xor-shift).
__device__ __forceinline__ uint32_t probe_mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

// Four int8 codes in [-127, 127] from one hash.
__device__ __forceinline__ int probe_codes(uint32_t seed) {
    uint32_t w = 0;
#pragma unroll
    for (int y = 0; y < 4; ++y) w |= (((probe_mix(seed * 4u + (uint32_t)y) % 255u) - 127u) & 0xFFu) << (8 * y);
    return (int)w;
}

// The arithmetic of one Q8 x Q8 prefill block-tile with nothing else, as the
// prefill kernel issues it: the exact int32 block sums (v_mfma_i32_32x32x32_i8,
// accumulating onto the bits of 1.5 * 2^23), the scale outer product
// (v_mfma_f32_32x32x16_f16, one nonzero k slot as in the kernel) and the fp32
// fold (16 exact subtractions + 16 FMAs per lane), the products of block u + 1
// issued before block u is folded.  Two operand sets of uniformly distributed
// codes and positive binary16 scales alternate, so successive products switch
// like real data (the matrix cores' power, and with it the clock, depends on
// the operand bits).  Each wave retires `iters` rounds of four block-tiles; the
// operands are made opaque every round so nothing is hoisted, and the result
// is written only in a case the operands never produce.  Timed with one to
// four workgroups per compute unit it gives the rate at which the chip can
// retire exact per-block folds -- the ceiling of any prefill kernel that keeps
// exact int32 block sums and folds them in fp32 one block at a time.
__global__ __launch_bounds__(256) void probe_fold_kernel(int iters, int* __restrict__ sink) {
    const int l = threadIdx.x & 63;
    const uint32_t g = (uint32_t)(blockIdx.x * 256 + threadIdx.x);
    q8::i32x4 a[2], b[2];
    f16x8p ha[2], hb;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[q][j] = probe_codes(g * 16u + (uint32_t)(q * 4 + j));
            b[q][j] = probe_codes(0x9E3779B9u ^ (g * 16u + (uint32_t)(q * 4 + j)));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ha[q][j] = (_Float16)0.0f;
        if (l < 32) ha[q][q] = (_Float16)(1.0f / (float)(1u + probe_mix(g * 2u + (uint32_t)q) % 1000u));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        hb[j] = j < 4 ? (_Float16)(1.0f / (float)(1u + probe_mix(0x85EBCA6Bu ^ (g * 8u + (uint32_t)j)) % 1000u))
                      : (_Float16)0.0f;
    q8::i32x16 cb;
#pragma unroll
    for (int r = 0; r < 16; ++r) cb[r] = 0x4B400000;
    asm volatile("" : "+v"(cb));
    const f32x16p zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    auto fold = [&](const q8::i32x16& c, const f32x16p& t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = fmaf(__int_as_float(c[r]) - 12582912.0f, t[r], acc[r]);
    };
    q8::i32x16 c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], cb, 0, 0, 0), c1;
    f32x16p t0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[0], hb, zf, 0, 0, 0), t1;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(ha[1]));
            c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[1], b[1], cb, 0, 0, 0);
            t1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[1], hb, zf, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            fold(c0, t0);
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" : "+v"(b[0]), "+v"(b[1]), "+v"(ha[0]));
            c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], cb, 0, 0, 0);
            t0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[0], hb, zf, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            fold(c1, t1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[r];
    if (__float_as_int(s) == 0x7FEDCBA9 && l == 0) sink[0] = c0[0];
}

int cu_count_current() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

template <int LPT>
hipError_t launch_read(const void* src, int64_t n16, uint32_t* sink, hipStream_t stream) {
    const int64_t grid = (n16 + 256 * LPT - 1) / (256 * LPT);
    probe_read_kernel<LPT><<<(unsigned)grid, 256, 0, stream>>>(reinterpret_cast<const q8::u32x4*>(src), n16,
                                                                sink);
    return hipGetLastError();
}

}  // namespace

extern "C" q8_status q8_probe_read(const void* src, int64_t bytes, int loads_per_thread, uint32_t* sink,
                                   hipStream_t stream) {
    if (bytes <= 0 || bytes % 16 != 0 || bytes > ((int64_t)1 << 40)) return Q8_ERR_SHAPE;
    if (loads_per_thread != 4 && loads_per_thread != 8 && loads_per_thread != 12 && loads_per_thread != 16)
        return Q8_ERR_SHAPE;
    if (!src || !sink) return Q8_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return Q8_ERR_ALIGN;
    if (cu_count_current() <= 0) return Q8_ERR_DEVICE;
    if ((bytes / 16 + 1023) / 1024 >= ((int64_t)1 << 31)) return Q8_ERR_SHAPE;
    (void)hipGetLastError();
    const int64_t n16 = bytes / 16;
    hipError_t e;
    switch (loads_per_thread) {
        case 4: e = launch_read<4>(src, n16, sink, stream); break;
        case 8: e = launch_read<8>(src, n16, sink, stream); break;
        case 12: e = launch_read<12>(src, n16, sink, stream); break;
        default: e = launch_read<16>(src, n16, sink, stream); break;
    }
    return e == hipSuccess ? Q8_OK : Q8_ERR_HIP;
}

extern "C" int64_t q8_probe_barrier_words(void) { return (int64_t)kBarErr + 1; }

extern "C" q8_status q8_probe_barrier(uint32_t* flags, int workgroups, int rounds, hipStream_t stream) {
    if (!flags) return Q8_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(flags) & 3u) return Q8_ERR_ALIGN;
    const int cus = cu_count_current();
    if (cus <= 0) return Q8_ERR_DEVICE;
    if (workgroups < 1 || workgroups > cus || workgroups > kBarStride || rounds < 0) return Q8_ERR_SHAPE;
    (void)hipGetLastError();
    probe_barrier_kernel<<<workgroups, 64, 0, stream>>>(flags, rounds);
    return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ERR_HIP;
}

extern "C" q8_status q8_probe_fold(int workgroups, int iters, int32_t* sink, hipStream_t stream) {
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24)) return Q8_ERR_SHAPE;
    if (!sink) return Q8_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(sink) & 3u) return Q8_ERR_ALIGN;
    if (cu_count_current() <= 0) return Q8_ERR_DEVICE;
    (void)hipGetLastError();
    probe_fold_kernel<<<workgroups, 256, 0, stream>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ERR_HIP;
}

extern "C" q8_status q8_probe_mfma_i8(int workgroups, int iters, int32_t* sink, hipStream_t stream) {
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24)) return Q8_ERR_SHAPE;
    if (!sink) return Q8_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(sink) & 3u) return Q8_ERR_ALIGN;
    if (cu_count_current() <= 0) return Q8_ERR_DEVICE;
    (void)hipGetLastError();
    probe_mfma_i8_kernel<<<workgroups, 256, 0, stream>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ERR_HIP;
}
