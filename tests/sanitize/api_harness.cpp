// Host-only harness for the C-ABI layer (q8_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, built with g++ on the CPU: a fake HIP runtime
// (one gfx950 device with 256 compute units and 160 KiB of LDS per workgroup,
// or no device at all) and stand-ins for the kernel launchers that only record
// their arguments.  The driver calls every entry point with valid, boundary
// and invalid arguments, checks the status codes, and checks that a valid call
// reaches its launcher with the extents it was given and an invalid one never
// does.  Exit status 0 on success.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "q8_internal.hpp"
#include "q8stream.h"

// ---------------------------------------------------------------- fake runtime

static bool g_have_device = true;
static int g_launches = 0;
static int64_t g_last_n = -1, g_last_k = -1, g_last_rows = -1;

extern "C" hipError_t hipGetDevice(int* dev) {
    if (!g_have_device) return hipErrorNoDevice;
    *dev = 0;
    return hipSuccess;
}
extern "C" hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int dev) {
    if (!g_have_device || dev != 0) return hipErrorInvalidDevice;
    std::memset(prop, 0, sizeof *prop);
    std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
    prop->multiProcessorCount = 256;
    prop->sharedMemPerBlock = 160 * 1024;
    return hipSuccess;
}
extern "C" hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* dev) {
    *dev = 0;
    return hipSuccess;
}
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

// ---------------------------------------------------------------- launcher stand-ins

namespace q8 {
static hipError_t rec(int64_t n, int64_t k, int64_t rows) {
    ++g_launches;
    g_last_n = n;
    g_last_k = k;
    g_last_rows = rows;
    return hipSuccess;
}
hipError_t launch_quantize_f32(const float*, int64_t nblocks, int8_t*, uint16_t*, const DeviceInfo&, hipStream_t) {
    return rec(nblocks, 32, 0);
}
hipError_t launch_quantize_bf16(const uint16_t*, int64_t nblocks, int8_t*, uint16_t*, const DeviceInfo&,
                                hipStream_t) {
    return rec(nblocks, 32, 0);
}
hipError_t launch_skinny(const int8_t*, const uint16_t*, int64_t n, int64_t k, int m, int, const void*,
                         const uint16_t*, float*, const DeviceInfo&, hipStream_t) {
    return rec(n, k, m);
}
hipError_t launch_block_dots(const int8_t*, int64_t n, int64_t k, int m, const int8_t*, int32_t*,
                             const DeviceInfo&, hipStream_t) {
    return rec(n, k, m);
}
bool fused_combo_supported(int pro, int epi) { return !(pro == 0 && epi == 0); }
hipError_t launch_fused(const int8_t*, const uint16_t*, int64_t n, int64_t k, int m, int, const void*, int, void*,
                        int64_t, int64_t, const DeviceInfo&, hipStream_t) {
    return rec(n, k, m);
}
hipError_t launch_rmsnorm(const float*, int64_t m, int64_t k, float*, hipStream_t) { return rec(0, k, m); }
hipError_t launch_attn_residual(const int8_t*, const uint16_t*, int64_t n, int64_t k, const float*, int nchunks,
                                float*, const DeviceInfo&, hipStream_t) {
    return rec(n, k, nchunks);
}
hipError_t launch_act_prologue_quantize(const float*, int64_t m, int64_t k, int, int8_t*, uint16_t*,
                                        hipStream_t) {
    return rec(0, k, m);
}
hipError_t launch_act_prologue_quantize_frag(const float*, int64_t m, int64_t k, int, int8_t*, uint16_t*,
                                             hipStream_t) {
    return rec(0, k, m);
}
hipError_t launch_q4_quantize(const float*, int64_t nblocks, uint8_t*, uint16_t*, const DeviceInfo&,
                              hipStream_t) {
    return rec(nblocks, 32, 0);
}
hipError_t launch_q4_skinny(const uint8_t*, const uint16_t*, int64_t n, int64_t k, int m, int, const void*,
                            const uint16_t*, float*, const DeviceInfo&, hipStream_t) {
    return rec(n, k, m);
}
size_t prefill_lds_bytes(int64_t, int64_t k, int64_t, const DeviceInfo&) {
    return k % 256 == 0 ? 40960 : 36864 + (size_t)(k / 32) * 128;
}
hipError_t prefill_prepare(const DeviceInfo&) { return hipSuccess; }
hipError_t launch_prefill(const int8_t*, const uint16_t*, int64_t n, int64_t k, int64_t p, const int8_t*,
                          const uint16_t*, float*, const DeviceInfo&, hipStream_t) {
    return rec(n, k, p);
}
int prefill_kind(int64_t, int64_t k, int64_t, int) { return k % 512 == 0 ? kPrefillStream : kPrefillTile32; }
SkinnyLayout skinny_layout(int64_t, int64_t, int, int) { return {16, 2, 6, false}; }
bool skinny_mfma_applies(int64_t, int64_t k, int m, int) { return m >= 5 && k % 512 == 0; }
SkinnyLayout skinny_mfma_layout(int64_t, int64_t, int) { return {16, 1, 4, true}; }
hipError_t launch_skinny_mfma(const int8_t*, const uint16_t*, int64_t n, int64_t k, int m, const void*, float*,
                              const DeviceInfo&, hipStream_t) {
    return rec(n, k, m);
}
Q4Layout q4_layout(int64_t, int64_t, int, int, int) { return {16, 2, 3, 0}; }
bool q4_mfma_applies(int64_t, int64_t k, int m, int) { return m >= 5 && k % 512 == 0; }
SkinnyLayout q4_mfma_layout(int64_t, int64_t, int) { return {16, 1, 4, true}; }
int64_t frag_rows(int64_t rows) { return (rows + 63) / 64 * 64; }
int64_t frag_blocks(int64_t k) { return (k / 32 + 3) / 4 * 4; }
FragLayout prefill_frag_layout(int64_t n, int64_t p, int) {
    const int64_t tiles = ((n + 31) / 32) * ((p + 31) / 32);
    return FragLayout{1, 4, (tiles + 7) / 8 * 8, 1};
}
hipError_t launch_pack_frag(const int8_t*, const uint16_t*, int64_t rows, int64_t k, int8_t*, uint16_t*,
                            const DeviceInfo&, hipStream_t) {
    return rec(0, k, rows);
}
hipError_t launch_prefill_frag(const int8_t*, const uint16_t*, int64_t n, int64_t k, int64_t p, const int8_t*,
                               const uint16_t*, float*, const DeviceInfo&, hipStream_t) {
    return rec(n, k, p);
}
// attention sizes: 64-row chunks up to 512 rows, 128 up to 2048, 256 above
static int64_t chunk_rows(int64_t t) { return t <= 512 ? 64 : t <= 2048 ? 128 : 256; }
int64_t attn_split_chunks(int64_t t) { return (t + chunk_rows(t) - 1) / chunk_rows(t); }
static int64_t max_chunks(int64_t t) {
    int64_t c = attn_split_chunks(t);
    if (t > 512 && c < 8) c = 8;
    if (t > 2048 && c < 16) c = 16;
    return c;
}
int64_t attn_work_floats(int64_t heads, int64_t t) { return max_chunks(t) > 1 ? heads * max_chunks(t) * 132 : 0; }
int64_t attn_partial_floats(int64_t heads, int64_t t) { return heads * max_chunks(t) * 132; }
hipError_t launch_attn_decode(const uint16_t*, int8_t*, uint16_t*, int8_t*, uint16_t*, int64_t heads, int64_t t,
                              int64_t, float, float*, float*, const uint16_t*, const uint16_t*, const DeviceInfo&,
                              hipStream_t) {
    return rec(heads, 128, t);
}
static float g_scratch[16];
hipError_t attn_scratch(const DeviceInfo&, float** p) {
    *p = g_scratch;
    return hipSuccess;
}
}  // namespace q8

// ---------------------------------------------------------------- driver

static int g_fail = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                       \
        }                                                                   \
    } while (0)

// Calls `f`; expects status `want`, and a launch exactly when want == Q8_OK and
// `launches` says so.
template <typename F>
static void call(F f, int want, bool launches) {
    const int before = g_launches;
    const int got = f();
    if (got != want) {
        std::fprintf(stderr, "status %d, expected %d\n", got, want);
        ++g_fail;
    }
    EXPECT((g_launches != before) == launches);
}

int main() {
    alignas(16) static unsigned char buf[4096];
    void* A = buf;
    void* B = buf + 1024;
    void* MIS = buf + 4;
    auto i8 = [](void* p) { return static_cast<int8_t*>(p); };
    auto u16 = [](void* p) { return static_cast<uint16_t*>(p); };
    auto f32 = [](void* p) { return static_cast<float*>(p); };

    // status strings and version
    EXPECT(q8_abi_version() == Q8_ABI_VERSION);
    for (int s = -2; s < 10; ++s) EXPECT(q8_status_str(s) != nullptr);

    // quantizers
    call([&] { return q8_quantize_weights(f32(A), 4, 64, i8(A), u16(B), nullptr); }, Q8_OK, true);
    EXPECT(g_last_n == 8);
    call([&] { return q8_quantize_weights(f32(A), 4, 48, i8(A), u16(B), nullptr); }, Q8_ERR_SHAPE, false);
    call([&] { return q8_quantize_weights(f32(A), (int64_t)1 << 40, (int64_t)1 << 20, i8(A), u16(B), nullptr); },
         Q8_ERR_SHAPE, false);
    call([&] { return q8_quantize_weights(f32(A), (int64_t)1 << 30, (int64_t)1 << 16, i8(A), u16(B), nullptr); },
         Q8_OK, true);                                   // 2^46 codes: the largest accepted size
    EXPECT(g_last_n == ((int64_t)1 << 41));
    call([&] { return q8_quantize_act(u16(A), 3, 64, i8(A), u16(MIS), nullptr); }, Q8_ERR_ALIGN, false);
    call([&] { return q8_quantize_act(nullptr, 0, 64, nullptr, nullptr, nullptr); }, Q8_OK, false);

    // products
    for (int m = 0; m <= 9; ++m) {
        const int want = m > 8 ? Q8_ERR_BATCH : Q8_OK;
        call([&] { return q8_gemm_skinny(i8(A), u16(B), 100, 1536, m, Q8_ACT_BF16, A, nullptr, f32(A), nullptr); },
             want, m >= 1 && m <= 8);
    }
    EXPECT(g_last_n == 100 && g_last_k == 1536 && g_last_rows == 8);
    call([&] { return q8_gemm_skinny(i8(A), u16(B), 100, 1536, 2, Q8_ACT_Q8, A, nullptr, f32(A), nullptr); },
         Q8_ERR_ENUM, false);
    call([&] { return q8_gemv(i8(A), u16(B), (int64_t)1 << 31, 64, 0, A, nullptr, f32(A), nullptr); },
         Q8_ERR_SHAPE, false);
    call([&] { return q8_gemm_prefill(i8(A), u16(B), 4608, 1536, 256, i8(A), u16(B), f32(A), nullptr); },
         Q8_OK, true);
    EXPECT(g_last_rows == 256);
    call([&] { return q8_gemm_prefill(i8(A), u16(B), 10, 32 * 8001, 5, i8(A), u16(B), f32(A), nullptr); },
         Q8_ERR_SHAPE, false);                           // a K whose scales do not fit the LDS
    call([&] { return q8_gemm_prefill(i8(A), u16(B), 10, 64, 65535LL * 64 + 1, i8(A), u16(B), f32(A), nullptr); },
         Q8_ERR_SHAPE, false);
    call([&] { return q8_block_dots(i8(A), 7, 96, 3, i8(A), static_cast<int32_t*>(B), nullptr); }, Q8_OK, true);
    EXPECT(q8_frag_code_bytes(65, 96) == 128 * 4 * 32 && q8_frag_scale_bytes(65, 96) == 128 * 4 * 2);
    EXPECT(q8_frag_code_bytes(65, 95) == -1 && q8_frag_scale_bytes(-1, 96) == -1);
    call([&] { return q8_pack_frag(i8(A), u16(B), 65, 96, i8(A), u16(B), nullptr); }, Q8_OK, true);
    EXPECT(g_last_rows == 65 && g_last_k == 96);
    call([&] { return q8_pack_frag(i8(A), u16(MIS), 65, 96, i8(A), u16(B), nullptr); }, Q8_ERR_ALIGN, false);
    call([&] { return q8_pack_frag(nullptr, nullptr, 0, 96, nullptr, nullptr, nullptr); }, Q8_OK, false);
    call([&] { return q8_gemm_prefill_frag(i8(A), u16(B), 4608, 1536, 256, i8(A), u16(B), f32(A), nullptr); },
         Q8_OK, true);
    EXPECT(g_last_n == 4608 && g_last_rows == 256);
    call([&] { return q8_gemm_prefill_frag(i8(A), u16(B), (int64_t)1 << 30, 32, 65535LL * 64, i8(A), u16(B), f32(A),
                                           nullptr); }, Q8_ERR_SHAPE, false);   // grid beyond 2^31 - 1
    call([&] { return q8_gemm_prefill_frag(i8(A), nullptr, 46, 64, 3, i8(A), u16(B), f32(A), nullptr); },
         Q8_ERR_NULL, false);
    call([&] { return q8_gemm_fused(i8(A), u16(B), 10, 64, 1, 0, A, 0, A, 0, 0, nullptr); }, Q8_ERR_ENUM, false);
    call([&] { return q8_gemm_fused(i8(A), u16(B), 11, 64, 1, 2, A, 3, A, 0, 0, nullptr); }, Q8_ERR_SHAPE, false);
    call([&] { return q8_gemm_fused(i8(A), u16(B), 256, 128, 1, 2, A, 3, A, 128, 7, nullptr); }, Q8_OK, true);
    call([&] { return q8_rmsnorm(f32(A), 2, 1536, f32(A), nullptr); }, Q8_OK, true);
    call([&] { return q8_quantize_act_fused(f32(A), 2, 1536, 0, i8(A), u16(B), nullptr); }, Q8_ERR_ENUM, false);
    call([&] { return q8_quantize_act_fused_frag(f32(A), 37, 1536, 2, i8(A), u16(B), nullptr); }, Q8_OK, true);
    EXPECT(g_last_rows == 37 && g_last_k == 1536);
    call([&] { return q8_quantize_act_fused_frag(f32(A), 37, 1536, 3, i8(A), u16(B), nullptr); }, Q8_ERR_ENUM, false);
    call([&] { return q8_quantize_act_fused_frag(f32(A), 65535LL * 64 + 1, 64, 1, i8(A), u16(B), nullptr); },
         Q8_ERR_SHAPE, false);
    call([&] { return q4_quantize_weights(f32(A), 3, 64, static_cast<uint8_t*>(A), u16(B), nullptr); }, Q8_OK,
         true);
    call([&] { return q4_gemm_skinny(static_cast<uint8_t*>(A), u16(B), 3, 64, 9, 0, A, nullptr, f32(A), nullptr); },
         Q8_ERR_BATCH, false);

    // attention
    const int64_t need = q8_attn_work_words(12, 4096);
    EXPECT(need == 12 * 16 * 132);
    EXPECT(q8_attn_work_words(12, 0) == -1);
    call([&] { return q8_attn_decode(u16(A), i8(B), u16(A), i8(B), u16(A), 12, 4096, 4096, 128, 0.08f, f32(A),
                                     f32(B), need, nullptr); }, Q8_OK, true);
    call([&] { return q8_attn_decode(u16(A), i8(B), u16(A), i8(B), u16(A), 12, 4096, 4096, 128, 0.08f, f32(A),
                                     f32(B), need - 1, nullptr); }, Q8_ERR_SHAPE, false);
    call([&] { return q8_attn_decode_noalloc(u16(A), i8(B), u16(A), i8(B), u16(A), 12, 42240, 1 << 20, 128, 0.08f,
                                             f32(A), nullptr); }, Q8_OK, true);
    call([&] { return q8_attn_decode_noalloc(u16(A), i8(B), u16(A), i8(B), u16(A), 12, 42241, 1 << 20, 128, 0.08f,
                                             f32(A), nullptr); }, Q8_ERR_SHAPE, false);
    call([&] { return q8_attn_decode_append(u16(A), i8(B), u16(A), i8(B), u16(A), 2, 65, 128, 128, 0.08f, nullptr,
                                            u16(A), f32(A), f32(B), 1 << 20, nullptr); }, Q8_ERR_NULL, false);
    const int64_t pw = q8_attn_partial_words(12, 512);
    call([&] { return q8_attn_decode_append_partials(u16(A), i8(B), u16(A), i8(B), u16(A), 12, 512, 512, 128,
                                                     0.08f, u16(A), u16(A), f32(B), pw, nullptr); }, Q8_OK, true);
    call([&] { return q8_gemm_attn_residual(i8(A), u16(B), 1536, 1536, f32(B), pw, 512, f32(A), nullptr); }, Q8_OK,
         true);
    call([&] { return q8_gemm_attn_residual(i8(A), u16(B), 1536, 1536, f32(B), pw, 4097, f32(A), nullptr); },
         Q8_ERR_SHAPE, false);

    // diagnostics
    char name[96];
    call([&] { return q8_kernel_name(Q8_OP_SKINNY, 262144, 1536, 1, 0, name, sizeof name); }, Q8_OK, false);
    EXPECT(std::strcmp(name, "skinny_kernel<1,0,16,2,6>") == 0);
    call([&] { return q8_kernel_name(Q8_OP_SKINNY, 262144, 1536, 8, 0, name, sizeof name); }, Q8_OK, false);
    EXPECT(std::strcmp(name, "skinny_mfma_kernel<8,16,1,4,0>") == 0);
    call([&] { return q8_kernel_name(Q8_OP_SKINNY, 262144, 1536, 8, 1, name, sizeof name); }, Q8_OK, false);
    EXPECT(std::strcmp(name, "skinny_kernel<8,1,16,2,6>") == 0);
    call([&] { return q8_kernel_name(Q8_OP_PREFILL, 4608, 1536, 256, 9, name, sizeof name); }, Q8_OK, false);
    EXPECT(std::strcmp(name, "prefill_stream_kernel") == 0);
    call([&] { return q8_kernel_name(Q8_OP_PREFILL_FRAG, 4608, 1536, 256, 0, name, sizeof name); }, Q8_OK, false);
    EXPECT(std::strcmp(name, "prefill_frag_kernel<1,4>") == 0);
    call([&] { return q8_kernel_name(Q8_OP_SKINNY, 262144, 1536, 1, 0, name, 5); }, Q8_ERR_SHAPE, false);

    // without a device, valid calls are refused before any launch
    g_have_device = false;
    call([&] { return q8_gemv(i8(A), u16(B), 10, 64, 0, A, nullptr, f32(A), nullptr); }, Q8_ERR_DEVICE, false);
    std::printf("%s\n", g_fail ? "FAILED" : "api harness ok");
    return g_fail ? 1 : 0;
}
