// q8_api.cpp -- the extern "C" boundary of q8stream.
//
// Every entry point first checks its arguments without touching HIP (so a
// rejected call enqueues nothing and leaves every output untouched), then checks
// the device (a gfx950 device that owns the stream), then hands the validated
// arguments to the kernel launchers.
#include "q8stream.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "q8_internal.hpp"

namespace {

thread_local int t_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];          // 0 unknown, 1 gfx950, -1 unsupported
q8::DeviceInfo g_dev_info[kMaxDevices];

constexpr int64_t kMaxExtent = (int64_t)1 << 31;   // per-dimension limit
constexpr int64_t kMaxElems = (int64_t)1 << 46;    // n * k limit (64 TiB of codes)
constexpr int64_t kMaxPrefillRows = (int64_t)65535 * 64;
constexpr int64_t kMaxFragK = (int64_t)1 << 25;            // a tile's K range fits 32-bit buffer offsets
constexpr int64_t kMaxAttnHeads = (int64_t)1 << 16;
constexpr int64_t kMaxAttnRows = ((int64_t)1 << 24) - 128;   // cache rows per head

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

q8_status check_k(int64_t k) {
    if (k < 32 || k % 32 != 0 || k >= kMaxExtent) return Q8_ERR_SHAPE;
    return Q8_OK;
}

q8_status check_rows(int64_t rows, int64_t k) {
    if (rows < 0 || rows >= kMaxExtent) return Q8_ERR_SHAPE;
    if (rows > 0 && rows > kMaxElems / k) return Q8_ERR_SHAPE;
    return Q8_OK;
}

q8_status hip_fail(hipError_t e) {
    t_last_hip_error = (int)e;
    return Q8_ERR_HIP;
}

// The device that will run the call: the current device, which must be a gfx950
// and must own `stream`.
q8_status device_for(hipStream_t stream, const q8::DeviceInfo** info) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        t_last_hip_error = (int)e;
        return Q8_ERR_DEVICE;
    }
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (g_dev_state[dev] == 0) {
            hipDeviceProp_t prop;
            e = hipGetDeviceProperties(&prop, dev);
            if (e != hipSuccess) {
                t_last_hip_error = (int)e;
                return Q8_ERR_DEVICE;
            }
            const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                            (prop.gcnArchName[6] == 0 || prop.gcnArchName[6] == ':');
            g_dev_info[dev].cu_count = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
            g_dev_info[dev].max_lds = prop.sharedMemPerBlock > 0 ? (size_t)prop.sharedMemPerBlock : 65536;
            g_dev_info[dev].ordinal = dev;
            if (ok && g_dev_info[dev].max_lds > 65536 &&
                q8::prefill_prepare(g_dev_info[dev]) != hipSuccess) {
                (void)hipGetLastError();
                g_dev_info[dev].max_lds = 65536;   // the default every kernel may use
            }
            g_dev_state[dev] = ok ? 1 : -1;
        }
        if (g_dev_state[dev] != 1) {
            t_last_hip_error = 0;
            return Q8_ERR_DEVICE;
        }
    }
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) {
            t_last_hip_error = (int)e;
            return Q8_ERR_DEVICE;
        }
        if ((int)sdev != dev) {
            t_last_hip_error = 0;
            return Q8_ERR_DEVICE;
        }
    }
    *info = &g_dev_info[dev];
    return Q8_OK;
}

#define Q8_TRY(expr)                       \
    do {                                   \
        const q8_status st_ = (expr);      \
        if (st_ != Q8_OK) return st_;      \
    } while (0)

q8_status finish(hipError_t e) {
    if (e != hipSuccess) return hip_fail(e);
    return Q8_OK;
}

q8_status check_act(int act, const void* xd) {
    if (act != Q8_ACT_BF16 && act != Q8_ACT_Q8) return Q8_ERR_ENUM;
    if (act == Q8_ACT_BF16 && xd != nullptr) return Q8_ERR_ENUM;
    if (act == Q8_ACT_Q8 && xd == nullptr) return Q8_ERR_ENUM;
    return Q8_OK;
}

}  // namespace

extern "C" {

int q8_abi_version(void) { return Q8_ABI_VERSION; }

const char* q8_status_str(int status) {
    switch (status) {
        case Q8_OK: return "Q8_OK";
        case Q8_ERR_NULL: return "Q8_ERR_NULL";
        case Q8_ERR_SHAPE: return "Q8_ERR_SHAPE";
        case Q8_ERR_BATCH: return "Q8_ERR_BATCH";
        case Q8_ERR_ALIGN: return "Q8_ERR_ALIGN";
        case Q8_ERR_ENUM: return "Q8_ERR_ENUM";
        case Q8_ERR_DEVICE: return "Q8_ERR_DEVICE";
        case Q8_ERR_HIP: return "Q8_ERR_HIP";
        default: return "unknown";
    }
}

int q8_last_hip_error(void) { return t_last_hip_error; }

q8_status q8_quantize_weights(const float* w, int64_t n, int64_t k, int8_t* wq, uint16_t* wd,
                              hipStream_t stream) {
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    if (n == 0) return Q8_OK;
    if (!w || !wq || !wd) return Q8_ERR_NULL;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(wd)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_quantize_f32(w, n * (k / 32), wq, wd, *dev, stream));
}

q8_status q8_quantize_act(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                          hipStream_t stream) {
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(m, k));
    if (m == 0) return Q8_OK;
    if (!x || !xq || !xd) return Q8_ERR_NULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(xd)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_quantize_bf16(x, m * (k / 32), xq, xd, *dev, stream));
}

q8_status q8_gemm_skinny(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t m,
                         int act, const void* x, const uint16_t* xd, float* y,
                         hipStream_t stream) {
    Q8_TRY(check_act(act, xd));
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    if (m < 0 || m > Q8_MAX_BATCH) return Q8_ERR_BATCH;
    if (n == 0 || m == 0) return Q8_OK;
    if (!wq || !wd || !x || !y) return Q8_ERR_NULL;
    if (!aligned16(wq) || !aligned16(wd) || !aligned16(x) || !aligned16(y) ||
        (xd && !aligned16(xd)))
        return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_skinny(wq, wd, n, k, (int)m, act, x, xd, y, *dev, stream));
}

q8_status q8_gemv(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int act,
                  const void* x, const uint16_t* xd, float* y, hipStream_t stream) {
    return q8_gemm_skinny(wq, wd, n, k, 1, act, x, xd, y, stream);
}

q8_status q8_gemm_prefill(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t p,
                          const int8_t* xq, const uint16_t* xd, float* y, hipStream_t stream) {
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    Q8_TRY(check_rows(p, k));
    if (p > kMaxPrefillRows) return Q8_ERR_SHAPE;
    if (n == 0 || p == 0) return Q8_OK;
    if (!wq || !wd || !xq || !xd || !y) return Q8_ERR_NULL;
    if (!aligned16(wq) || !aligned16(wd) || !aligned16(xq) || !aligned16(xd) || !aligned16(y))
        return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    if (q8::prefill_lds_bytes(n, k, p, *dev) > dev->max_lds) return Q8_ERR_SHAPE;
    return finish(q8::launch_prefill(wq, wd, n, k, p, xq, xd, y, *dev, stream));
}

int64_t q8_frag_code_bytes(int64_t rows, int64_t k) {
    if (check_k(k) != Q8_OK || check_rows(rows, k) != Q8_OK) return -1;
    return q8::frag_rows(rows) * q8::frag_blocks(k) * 32;
}

int64_t q8_frag_scale_bytes(int64_t rows, int64_t k) {
    if (check_k(k) != Q8_OK || check_rows(rows, k) != Q8_OK) return -1;
    return q8::frag_rows(rows) * q8::frag_blocks(k) * 2;
}

q8_status q8_pack_frag(const int8_t* q, const uint16_t* d, int64_t rows, int64_t k, int8_t* qf, uint16_t* df,
                       hipStream_t stream) {
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(rows, k));
    if (rows == 0) return Q8_OK;
    if (!q || !d || !qf || !df) return Q8_ERR_NULL;
    if (!aligned16(q) || !aligned16(d) || !aligned16(qf) || !aligned16(df)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_pack_frag(q, d, rows, k, qf, df, *dev, stream));
}

q8_status q8_gemm_prefill_frag(const int8_t* wf, const uint16_t* wdf, int64_t n, int64_t k, int64_t p,
                               const int8_t* xf, const uint16_t* xdf, float* y, hipStream_t stream) {
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    Q8_TRY(check_rows(p, k));
    if (p > kMaxPrefillRows || k > kMaxFragK) return Q8_ERR_SHAPE;
    if (n == 0 || p == 0) return Q8_OK;
    if (!wf || !wdf || !xf || !xdf || !y) return Q8_ERR_NULL;
    if (!aligned16(wf) || !aligned16(wdf) || !aligned16(xf) || !aligned16(xdf) || !aligned16(y))
        return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    if (q8::prefill_frag_layout(n, p, dev->cu_count).grid > (int64_t)INT32_MAX) return Q8_ERR_SHAPE;
    return finish(q8::launch_prefill_frag(wf, wdf, n, k, p, xf, xdf, y, *dev, stream));
}

q8_status q8_block_dots(const int8_t* wq, int64_t n, int64_t k, int64_t m, const int8_t* xq,
                        int32_t* isum, hipStream_t stream) {
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    if (m < 0 || m > Q8_MAX_BATCH) return Q8_ERR_BATCH;
    if (n == 0 || m == 0) return Q8_OK;
    if (!wq || !xq || !isum) return Q8_ERR_NULL;
    if (!aligned16(wq) || !aligned16(xq) || !aligned16(isum)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_block_dots(wq, n, k, (int)m, xq, isum, *dev, stream));
}

q8_status q8_gemm_fused(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t m,
                        int prologue, const void* x, int epilogue, void* out, int64_t rope_rows,
                        int64_t pos, hipStream_t stream) {
    if (prologue < Q8_PRO_BF16 || prologue > Q8_PRO_RMSNORM || epilogue < Q8_EPI_F32 ||
        epilogue > Q8_EPI_ROPE || !q8::fused_combo_supported(prologue, epilogue))
        return Q8_ERR_ENUM;
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    if (m < 0 || m > Q8_MAX_BATCH) return Q8_ERR_BATCH;
    if ((epilogue == Q8_EPI_SWIGLU || epilogue == Q8_EPI_ROPE) && n % 2 != 0) return Q8_ERR_SHAPE;
    if (epilogue == Q8_EPI_ROPE &&
        (rope_rows < 0 || rope_rows > n || rope_rows % 128 != 0 || pos < 0 || pos >= kMaxExtent))
        return Q8_ERR_SHAPE;
    if (n == 0 || m == 0) return Q8_OK;
    if (!wq || !wd || !x || !out) return Q8_ERR_NULL;
    if (!aligned16(wq) || !aligned16(wd) || !aligned16(x) || !aligned16(out)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_fused(wq, wd, n, k, (int)m, prologue, x, epilogue, out, rope_rows, pos, *dev,
                                   stream));
}

q8_status q8_rmsnorm(const float* x, int64_t m, int64_t k, float* y, hipStream_t stream) {
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(m, k));
    if (m == 0) return Q8_OK;
    if (!x || !y) return Q8_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_rmsnorm(x, m, k, y, stream));
}

q8_status q8_quantize_act_fused(const float* x, int64_t m, int64_t k, int prologue, int8_t* xq,
                                uint16_t* xd, hipStream_t stream) {
    if (prologue != Q8_PRO_F32 && prologue != Q8_PRO_RMSNORM) return Q8_ERR_ENUM;
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(m, k));
    if (m == 0) return Q8_OK;
    if (!x || !xq || !xd) return Q8_ERR_NULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(xd)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_act_prologue_quantize(x, m, k, prologue, xq, xd, stream));
}

q8_status q8_quantize_act_fused_frag(const float* x, int64_t m, int64_t k, int prologue, int8_t* xqf,
                                     uint16_t* xdf, hipStream_t stream) {
    if (prologue != Q8_PRO_F32 && prologue != Q8_PRO_RMSNORM) return Q8_ERR_ENUM;
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(m, k));
    if (m > kMaxPrefillRows) return Q8_ERR_SHAPE;
    if (m == 0) return Q8_OK;
    if (!x || !xqf || !xdf) return Q8_ERR_NULL;
    if (!aligned16(x) || !aligned16(xqf) || !aligned16(xdf)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_act_prologue_quantize_frag(x, m, k, prologue, xqf, xdf, stream));
}

q8_status q4_quantize_weights(const float* w, int64_t n, int64_t k, uint8_t* wq, uint16_t* wd,
                              hipStream_t stream) {
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    if (n == 0) return Q8_OK;
    if (!w || !wq || !wd) return Q8_ERR_NULL;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(wd)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_q4_quantize(w, n * (k / 32), wq, wd, *dev, stream));
}

q8_status q4_gemm_skinny(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t m,
                         int act, const void* x, const uint16_t* xd, float* y,
                         hipStream_t stream) {
    Q8_TRY(check_act(act, xd));
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    if (m < 0 || m > Q8_MAX_BATCH) return Q8_ERR_BATCH;
    if (n == 0 || m == 0) return Q8_OK;
    if (!wq || !wd || !x || !y) return Q8_ERR_NULL;
    if (!aligned16(wq) || !aligned16(wd) || !aligned16(x) || !aligned16(y) ||
        (xd && !aligned16(xd)))
        return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_q4_skinny(wq, wd, n, k, (int)m, act, x, xd, y, *dev, stream));
}

q8_status q8_kernel_name(int op, int64_t n, int64_t k, int64_t rows, int act, char* buf, int64_t buf_len) {
    if (op != Q8_OP_SKINNY && op != Q8_OP_PREFILL && op != Q8_OP_Q4_SKINNY && op != Q8_OP_PREFILL_FRAG)
        return Q8_ERR_ENUM;
    const bool prefill = op == Q8_OP_PREFILL || op == Q8_OP_PREFILL_FRAG;
    if (!prefill && act != Q8_ACT_BF16 && act != Q8_ACT_Q8) return Q8_ERR_ENUM;
    Q8_TRY(check_k(k));
    Q8_TRY(check_rows(n, k));
    if (prefill) {
        Q8_TRY(check_rows(rows, k));
        if (rows > kMaxPrefillRows) return Q8_ERR_SHAPE;
    } else if (rows < 0 || rows > Q8_MAX_BATCH) {
        return Q8_ERR_BATCH;
    }
    if (!buf) return Q8_ERR_NULL;
    if (buf_len < 1) return Q8_ERR_SHAPE;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(nullptr, &dev));
    char name[96];
    if (n == 0 || rows == 0) {
        std::snprintf(name, sizeof name, "none");
    } else if (op == Q8_OP_SKINNY && act == Q8_ACT_BF16 &&
               q8::skinny_mfma_applies(n, k, (int)rows, dev->cu_count)) {
        const q8::SkinnyLayout L = q8::skinny_mfma_layout(n, k, dev->cu_count);
        std::snprintf(name, sizeof name, "skinny_mfma_kernel<%d,%d,%d,%d,%d>", (int)rows, L.g, L.r, L.cpl,
                      L.r == 2 ? 1 : 0);
    } else if (op == Q8_OP_SKINNY) {
        const q8::SkinnyLayout L = q8::skinny_layout(n, k, (int)rows, dev->cu_count);
        std::snprintf(name, sizeof name, "skinny_kernel<%d,%d,%d,%d,%d>", (int)rows, act, L.g, L.r, L.cpl);
    } else if (op == Q8_OP_Q4_SKINNY && act == Q8_ACT_BF16 &&
               q8::q4_mfma_applies(n, k, (int)rows, dev->cu_count)) {
        const q8::SkinnyLayout L = q8::q4_mfma_layout(n, k, dev->cu_count);
        std::snprintf(name, sizeof name, "q4_skinny_mfma_kernel<%d,%d,%d,%d,0>", (int)rows, L.g, L.r, L.cpl);
    } else if (op == Q8_OP_Q4_SKINNY) {
        const q8::Q4Layout L = q8::q4_layout(n, k, (int)rows, act, dev->cu_count);
        std::snprintf(name, sizeof name, "q4_skinny_kernel<%d,%d,%d,%d,%d,%d>", (int)rows, act, L.g, L.r, L.cpl,
                      L.xl);
    } else if (op == Q8_OP_PREFILL_FRAG) {
        const q8::FragLayout L = q8::prefill_frag_layout(n, rows, dev->cu_count);
        if (L.wp == 2)
            std::snprintf(name, sizeof name, "prefill_frag64_kernel<%d>", L.ks);
        else
            std::snprintf(name, sizeof name, "prefill_frag_kernel<%d,%d>", L.wn, L.ks);
    } else {
        static const char* const kinds[] = {"prefill_tile64_kernel<1>", "prefill_tile64_kernel<2>",
                                            "prefill_stream_kernel", "prefill_kernel"};
        std::snprintf(name, sizeof name, "%s", kinds[q8::prefill_kind(n, k, rows, dev->cu_count)]);
    }
    const size_t len = std::strlen(name);
    if ((int64_t)len + 1 > buf_len) return Q8_ERR_SHAPE;
    std::memcpy(buf, name, len + 1);
    return Q8_OK;
}

int64_t q8_attn_work_words(int64_t heads, int64_t t) {
    if (heads < 0 || heads > kMaxAttnHeads || t < 1 || t > kMaxAttnRows) return -1;
    return q8::attn_work_floats(heads, t);
}

q8_status q8_attn_decode(const uint16_t* q, const int8_t* kq, const uint16_t* kd, const int8_t* vq,
                         const uint16_t* vd, int64_t heads, int64_t t, int64_t t_cap,
                         int64_t head_dim, float scale, float* out, float* work, int64_t work_words,
                         hipStream_t stream) {
    if (head_dim != 128) return Q8_ERR_SHAPE;
    if (heads < 0 || heads > kMaxAttnHeads || t < 1 || t > t_cap || t_cap > kMaxAttnRows)
        return Q8_ERR_SHAPE;
    if (!(scale == scale) || scale - scale != 0.0f) return Q8_ERR_SHAPE;   // NaN or infinite
    if (heads == 0) return Q8_OK;
    const int64_t need = q8::attn_work_floats(heads, t);
    if (work_words < need) return Q8_ERR_SHAPE;
    if (!q || !kq || !kd || !vq || !vd || !out || (need > 0 && !work)) return Q8_ERR_NULL;
    if (!aligned16(q) || !aligned16(kq) || !aligned16(kd) || !aligned16(vq) || !aligned16(vd) ||
        !aligned16(out) || (need > 0 && !aligned16(work)))
        return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    // the cache is only read on this path (knew == NULL)
    return finish(q8::launch_attn_decode(q, const_cast<int8_t*>(kq), const_cast<uint16_t*>(kd),
                                         const_cast<int8_t*>(vq), const_cast<uint16_t*>(vd), heads, t,
                                         t_cap, scale, out, work, nullptr, nullptr, *dev, stream));
}

q8_status q8_attn_decode_append(const uint16_t* q, int8_t* kq, uint16_t* kd, int8_t* vq, uint16_t* vd,
                                int64_t heads, int64_t t, int64_t t_cap, int64_t head_dim, float scale,
                                const uint16_t* knew, const uint16_t* vnew, float* out, float* work,
                                int64_t work_words, hipStream_t stream) {
    if (head_dim != 128) return Q8_ERR_SHAPE;
    if (heads < 0 || heads > kMaxAttnHeads || t < 1 || t > t_cap || t_cap > kMaxAttnRows)
        return Q8_ERR_SHAPE;
    if (!(scale == scale) || scale - scale != 0.0f) return Q8_ERR_SHAPE;
    if (heads == 0) return Q8_OK;
    const int64_t need = q8::attn_work_floats(heads, t);
    if (work_words < need) return Q8_ERR_SHAPE;
    if (!q || !kq || !kd || !vq || !vd || !knew || !vnew || !out || (need > 0 && !work)) return Q8_ERR_NULL;
    if (!aligned16(q) || !aligned16(kq) || !aligned16(kd) || !aligned16(vq) || !aligned16(vd) ||
        !aligned16(knew) || !aligned16(vnew) || !aligned16(out) || (need > 0 && !aligned16(work)))
        return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_attn_decode(q, kq, kd, vq, vd, heads, t, t_cap, scale, out, work, knew, vnew,
                                         *dev, stream));
}

q8_status q8_attn_decode_noalloc(const uint16_t* q, const int8_t* kq, const uint16_t* kd, const int8_t* vq,
                                 const uint16_t* vd, int64_t heads, int64_t t, int64_t t_cap, int64_t head_dim,
                                 float scale, float* out, hipStream_t stream) {
    if (head_dim != 128) return Q8_ERR_SHAPE;
    if (heads < 0 || heads > kMaxAttnHeads || t < 1 || t > t_cap || t_cap > kMaxAttnRows)
        return Q8_ERR_SHAPE;
    if (!(scale == scale) || scale - scale != 0.0f) return Q8_ERR_SHAPE;
    if (heads == 0) return Q8_OK;
    const int64_t need = q8::attn_work_floats(heads, t);
    if (need > q8::kAttnScratchFloats) return Q8_ERR_SHAPE;
    if (!q || !kq || !kd || !vq || !vd || !out) return Q8_ERR_NULL;
    if (!aligned16(q) || !aligned16(kq) || !aligned16(kd) || !aligned16(vq) || !aligned16(vd) ||
        !aligned16(out))
        return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    float* work = nullptr;
    if (need > 0) {
        const hipError_t e = q8::attn_scratch(*dev, &work);
        if (e != hipSuccess) return hip_fail(e);
    }
    return finish(q8::launch_attn_decode(q, const_cast<int8_t*>(kq), const_cast<uint16_t*>(kd),
                                         const_cast<int8_t*>(vq), const_cast<uint16_t*>(vd), heads, t,
                                         t_cap, scale, out, work, nullptr, nullptr, *dev, stream));
}

int64_t q8_attn_partial_words(int64_t heads, int64_t t) {
    if (heads < 0 || heads > kMaxAttnHeads || t < 1 || t > kMaxAttnRows) return -1;
    return q8::attn_partial_floats(heads, t);
}

q8_status q8_attn_decode_append_partials(const uint16_t* q, int8_t* kq, uint16_t* kd, int8_t* vq, uint16_t* vd,
                                         int64_t heads, int64_t t, int64_t t_cap, int64_t head_dim, float scale,
                                         const uint16_t* knew, const uint16_t* vnew, float* work,
                                         int64_t work_words, hipStream_t stream) {
    if (head_dim != 128) return Q8_ERR_SHAPE;
    if (heads < 0 || heads > kMaxAttnHeads || t < 1 || t > t_cap || t_cap > kMaxAttnRows)
        return Q8_ERR_SHAPE;
    if (!(scale == scale) || scale - scale != 0.0f) return Q8_ERR_SHAPE;
    if (heads == 0) return Q8_OK;
    if (work_words < q8::attn_partial_floats(heads, t)) return Q8_ERR_SHAPE;
    if (!q || !kq || !kd || !vq || !vd || !knew || !vnew || !work) return Q8_ERR_NULL;
    if (!aligned16(q) || !aligned16(kq) || !aligned16(kd) || !aligned16(vq) || !aligned16(vd) ||
        !aligned16(knew) || !aligned16(vnew) || !aligned16(work))
        return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_attn_decode(q, kq, kd, vq, vd, heads, t, t_cap, scale, nullptr, work, knew, vnew,
                                         *dev, stream));
}

q8_status q8_gemm_attn_residual(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, const float* work,
                                int64_t work_words, int64_t t, float* h, hipStream_t stream) {
    if (k < 128 || k % 128 != 0 || k > 2048) return Q8_ERR_SHAPE;
    Q8_TRY(check_rows(n, k));
    if (t < 1 || t > 4096) return Q8_ERR_SHAPE;
    const int64_t chunks = q8::attn_split_chunks(t);       // <= 16
    if (work_words < q8::attn_partial_floats(k / 128, t)) return Q8_ERR_SHAPE;
    if (n == 0) return Q8_OK;
    if (!wq || !wd || !work || !h) return Q8_ERR_NULL;
    if (!aligned16(wq) || !aligned16(wd) || !aligned16(work) || !aligned16(h)) return Q8_ERR_ALIGN;
    const q8::DeviceInfo* dev = nullptr;
    Q8_TRY(device_for(stream, &dev));
    return finish(q8::launch_attn_residual(wq, wd, n, k, work, (int)chunks, h, *dev, stream));
}

}  // extern "C"
