// q8_probe.hip -- HBM read-bandwidth probe (measurement utility).
//
// Each workgroup streams one contiguous span of the buffer with 16-byte
// non-temporal loads, four in flight per lane, and folds them into an xor
// checksum; one word per workgroup is written so the loads stay live.
// Contiguous spans per workgroup keep each DRAM page's reads together, which
// measured faster on MI355X than a grid-stride walk over the whole buffer.
#include "q8probe.h"
#include "q8_device.hpp"

#include <hip/hip_runtime.h>

namespace {

constexpr int kProbeBlocksPerCu = 16;

__global__ __launch_bounds__(256) void probe_read_kernel(const q8::u32x4* __restrict__ src,
                                                         int64_t n16, uint32_t* __restrict__ sink) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    q8::u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = b0 + threadIdx.x;
    for (; i + 3 * 256 < b1; i += 4 * 256) {
        const q8::u32x4 a = __builtin_nontemporal_load(src + i);
        const q8::u32x4 b = __builtin_nontemporal_load(src + i + 256);
        const q8::u32x4 c = __builtin_nontemporal_load(src + i + 512);
        const q8::u32x4 d = __builtin_nontemporal_load(src + i + 768);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(src + i);
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    __shared__ uint32_t red[256];
    red[threadIdx.x] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int t = 0; t < 256; ++t) s ^= red[t];
        sink[blockIdx.x] = s;
    }
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

int cu_count_current() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

}  // namespace

extern "C" int64_t q8_probe_sink_words(void) { return (int64_t)cu_count_current() * kProbeBlocksPerCu; }

extern "C" q8_status q8_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    if (bytes <= 0 || bytes % 16 != 0) return Q8_ERR_SHAPE;
    if (!src || !sink) return Q8_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return Q8_ERR_ALIGN;
    const int cus = cu_count_current();
    if (cus <= 0) return Q8_ERR_DEVICE;
    (void)hipGetLastError();
    probe_read_kernel<<<cus * kProbeBlocksPerCu, 256, 0, stream>>>(
        reinterpret_cast<const q8::u32x4*>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ERR_HIP;
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
