// q8_internal.hpp -- host-side launchers shared between the C ABI layer and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

struct DeviceInfo {
    int cu_count;
    size_t max_lds;   // largest LDS allocation of one workgroup, bytes
    int ordinal;      // HIP device index
};

// Each launcher enqueues on `stream` and returns the launch's hipError_t.
hipError_t launch_quantize_f32(const float* w, int64_t nblocks, int8_t* q, uint16_t* d,
                               const DeviceInfo& dev, hipStream_t stream);
hipError_t launch_quantize_bf16(const uint16_t* x, int64_t nblocks, int8_t* q, uint16_t* d,
                                const DeviceInfo& dev, hipStream_t stream);

// Lane-group layout of the decode product kernel for (n, k, m) on a device
// with cu_count compute units: G lanes per group, R rows per group, CPL
// 16-byte chunks per lane per K tile.  For the matrix-core form (mfma): G rows
// per fragment (16, or 8 for a half fragment), R fragments of rows per wave, K
// split over CPL waves (workgroups of max(4, CPL) waves).
struct SkinnyLayout {
    int g, r, cpl;
    bool mfma;
};
SkinnyLayout skinny_layout(int64_t n, int64_t k, int m, int cu_count);
// The batch 2..8 W8A16 product on the matrix cores (bf16 activations only):
// whether it is used for (n, k, m), its layout, and its launch.
bool skinny_mfma_applies(int64_t n, int64_t k, int m, int cu_count);
SkinnyLayout skinny_mfma_layout(int64_t n, int64_t k, int cu_count);
hipError_t launch_skinny_mfma(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m, const void* x,
                              float* y, const DeviceInfo& dev, hipStream_t stream);
// The same for int4 weights (q4_gemm_skinny with bf16 activations).
bool q4_mfma_applies(int64_t n, int64_t k, int m, int cu_count);
SkinnyLayout q4_mfma_layout(int64_t n, int64_t k, int cu_count);
hipError_t launch_q4_mfma(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m, const void* x,
                          float* y, const DeviceInfo& dev, hipStream_t stream);

hipError_t launch_skinny(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m,
                         int act, const void* x, const uint16_t* xd, float* y,
                         const DeviceInfo& dev, hipStream_t stream);

hipError_t launch_block_dots(const int8_t* wq, int64_t n, int64_t k, int m, const int8_t* xq,
                             int32_t* isum, const DeviceInfo& dev, hipStream_t stream);

// W8A16 products with a fused prologue / epilogue (codes of q8_prologue and
// q8_epilogue), and the standalone weightless RMSNorm.
bool fused_combo_supported(int pro, int epi);
hipError_t launch_fused(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m, int pro,
                        const void* x, int epi, void* out, int64_t rope_rows, int64_t pos,
                        const DeviceInfo& dev, hipStream_t stream);
hipError_t launch_rmsnorm(const float* x, int64_t m, int64_t k, float* y, hipStream_t stream);
// y[n] += W * bf16(a): a = the attention output combined from the partials in
// `work` (heads = k / 128, nchunks <= 8 of them per head).
hipError_t launch_attn_residual(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, const float* work,
                                int nchunks, float* y, const DeviceInfo& dev, hipStream_t stream);
hipError_t launch_act_prologue_quantize(const float* x, int64_t m, int64_t k, int pro, int8_t* xq,
                                        uint16_t* xd, hipStream_t stream);
// The same writing fragment order (q8_prefill_frag.hip's layout), padding
// rows and blocks included.
hipError_t launch_act_prologue_quantize_frag(const float* x, int64_t m, int64_t k, int pro, int8_t* xqf,
                                             uint16_t* xdf, hipStream_t stream);

// int4 weights (two codes per byte, binary16 scale per 32-element block).
hipError_t launch_q4_quantize(const float* w, int64_t nblocks, uint8_t* q, uint16_t* d,
                              const DeviceInfo& dev, hipStream_t stream);
hipError_t launch_q4_skinny(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int m,
                            int act, const void* x, const uint16_t* xd, float* y,
                            const DeviceInfo& dev, hipStream_t stream);

// The prefill kernel chosen for (n, k, p) on a device with cu_count compute
// units: prefill_tile64_kernel<1> / <2>, prefill_stream_kernel, prefill_kernel.
enum { kPrefillTile64x1 = 0, kPrefillTile64x2 = 1, kPrefillStream = 2, kPrefillTile32 = 3 };
int prefill_kind(int64_t n, int64_t k, int64_t p, int cu_count);

// Layout of the int4 product kernel: as SkinnyLayout, plus whether the
// activation tile is staged in LDS.
struct Q4Layout {
    int g, r, cpl, xl;
};
Q4Layout q4_layout(int64_t n, int64_t k, int m, int act, int cu_count);

// LDS the prefill kernel chosen for this shape needs, and the one-time
// per-device setup that lets it use up to dev.max_lds.
size_t prefill_lds_bytes(int64_t n, int64_t k, int64_t p, const DeviceInfo& dev);
hipError_t prefill_prepare(const DeviceInfo& dev);

hipError_t launch_prefill(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t p,
                          const int8_t* xq, const uint16_t* xd, float* y,
                          const DeviceInfo& dev, hipStream_t stream);

// The prefill product on operands in the int8 matrix core's fragment order
// (q8_prefill_frag.hip): rows rounded up to 64 and K/32 rounded up to 4 in
// that layout; the tile shape (wn weight tiles of 32 rows per wave), K split
// over ks waves and grid chosen for (n, p); the packing of a row-major Q8_0
// matrix; the product.
int64_t frag_rows(int64_t rows);
int64_t frag_blocks(int64_t k);
struct FragLayout {
    int wn, ks;
    int64_t grid;
    int wp;        // token tiles per wave: 2 selects the 64 x 64 kernel (wn = 2, ks = 1)
};
FragLayout prefill_frag_layout(int64_t n, int64_t p, int cu_count);
hipError_t launch_pack_frag(const int8_t* q, const uint16_t* d, int64_t rows, int64_t k, int8_t* qf,
                            uint16_t* df, const DeviceInfo& dev, hipStream_t stream);
hipError_t launch_prefill_frag(const int8_t* wf, const uint16_t* wsf, int64_t n, int64_t k, int64_t p,
                               const int8_t* xf, const uint16_t* xsf, float* y, const DeviceInfo& dev,
                               hipStream_t stream);

// Decode attention over a Q8_0 key/value cache (head dimension 128): the
// workspace floats the chunk partials of any context up to t need (0 when one
// chunk covers every such context).
int64_t attn_work_floats(int64_t heads, int64_t t);
// The chunks the split uses for context t, and the floats of the partials of
// any context up to t: per (head, chunk) a record of kAttnPartFloats floats
// (numerator [128], max, denominator, padding), heads outer.
int64_t attn_split_chunks(int64_t t);
int64_t attn_partial_floats(int64_t heads, int64_t t);
constexpr int kAttnPartFloats = 132;
// With knew / vnew (bf16 [heads][128]) the key and value rows t - 1 are first
// quantized into the cache; NULL leaves the cache untouched.  With out == NULL
// the per-chunk partials are left in `work` (also for a single chunk) and not
// combined.
hipError_t launch_attn_decode(const uint16_t* q, int8_t* kq, uint16_t* kd, int8_t* vq, uint16_t* vd,
                              int64_t heads, int64_t t, int64_t t_cap, float scale, float* out,
                              float* work, const uint16_t* knew, const uint16_t* vnew,
                              const DeviceInfo& dev, hipStream_t stream);

// The library's static attention scratch (kAttnScratchFloats floats, a
// file-scope device array, one copy per GPU): its device address on dev,
// looked up once per device with that device current and kept.
constexpr int64_t kAttnScratchFloats = 262144;          // 1 MiB
hipError_t attn_scratch(const DeviceInfo& dev, float** ptr);

}  // namespace q8
