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
