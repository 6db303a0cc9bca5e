/*
 * q8stream.h -- C ABI of the Q8_0 weight-streaming library for MI355X (gfx950).
 *
 * The library computes the int8 weight-streaming hot path of LLM decode and
 * prefill: block quantization of weights and activations, the batch-1..8
 * matrix-vector / skinny products over int8 weights, the Q8 x Q8 prefill
 * product, decode attention over a Q8_0 key/value cache, the int4-weight
 * variant of the quantizer and the batch-1..8 products, and the glue of a
 * decode block fused into those calls (RMSNorm, rotary embedding, SwiGLU and
 * residual prologues/epilogues; attention that appends its key/value row; the
 * attention combine inside the output projection; the prefill activation side
 * in one launch).  Every call is a hand-written HIP kernel enqueued on the
 * caller's stream.
 *
 * Format (Q8_0) [fak MODEL-BASELINE-RESULTS, ACT 3, "How it was closed",
 * item 1]: a row of K values (K % 32 == 0) is cut into K/32 blocks of 32
 * consecutive elements along the reduction axis.  Each block stores 32 int8
 * codes and one scale d = maxabs / 127.  The scale is stored as IEEE binary16
 * (2 bytes, so 34 bytes per 32 weights = 1.0625 B/weight, the page's "~1.06
 * B/weight").  d is the fp32 quotient maxabs / 127 rounded to binary16 (nearest,
 * ties to even).  Codes are clamp(round_half_away(v / d), -127, 127), the
 * quotient being the correctly rounded fp32 division by the STORED scale; a block
 * whose stored scale is zero has all-zero codes [ACT 4, "Correctness": rounding
 * equal to math.Round, never add-0.5-and-truncate].
 *
 * Conventions shared by every call:
 *  - Pointers are device pointers on the current HIP device.  bf16 and binary16
 *    values travel as uint16_t bit patterns.  Arrays are dense and row-major:
 *      int8 codes  [rows][K]     (row pitch K bytes)
 *      scales      [rows][K/32]  (row pitch K/16 bytes)
 *      bf16 values [rows][K]     (row pitch 2K bytes)
 *      fp32 output [m][N]        (row pitch 4N bytes)
 *  - Every pointer passed for a non-empty call must be 16-byte aligned.
 *  - Ownership: the caller allocates and frees every buffer.  The library never
 *    allocates, frees or caches device memory and keeps no per-call state, so
 *    calls may be made from several host threads and may be captured into a
 *    HIP graph.  (One exception: q8_attn_decode_noalloc keeps its partials in a
 *    fixed static array per GPU, see there.)  Outputs must not alias inputs.
 *  - Asynchrony: a call validates its arguments, enqueues kernels on `stream`
 *    (NULL = the current device's null stream) and returns.  Results are valid
 *    once the stream has been synchronized.  Calls never synchronize.
 *  - Errors: arguments are checked on the host before any HIP call; on a
 *    validation error nothing is enqueued and no output is touched.  A failed
 *    launch returns Q8_ERR_HIP (the HIP error code is kept per host thread, see
 *    q8_last_hip_error()).  Faults inside kernels surface, as in HIP, at the next
 *    synchronization.
 *  - Empty calls: a zero row count (n, m or p == 0) is a valid no-op that
 *    returns Q8_OK without touching any pointer.  K must be a positive multiple
 *    of 32.
 *  - Inputs must be finite.  Non-finite inputs give unspecified results.
 *  - Determinism: identical inputs and shapes give bitwise identical outputs on
 *    every call and on graph replay (fixed reduction order, no atomics).
 */
#ifndef Q8STREAM_H
#define Q8STREAM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q8_ABI_VERSION 1

/* Largest batch of the decode products. */
#define Q8_MAX_BATCH 8

typedef enum {
    Q8_OK = 0,
    Q8_ERR_NULL = 1,   /* a required pointer is NULL                              */
    Q8_ERR_SHAPE = 2,  /* negative extent, K < 32, K % 32 != 0, size overflow     */
    Q8_ERR_BATCH = 3,  /* m outside [0, Q8_MAX_BATCH] for gemv / skinny           */
    Q8_ERR_ALIGN = 4,  /* a pointer is not 16-byte aligned                        */
    Q8_ERR_ENUM = 5,   /* unknown q8_act, or xd given (or missing) against act    */
    Q8_ERR_DEVICE = 6, /* no HIP device, device is not gfx950, or the stream
                          belongs to another device than the current one          */
    Q8_ERR_HIP = 7     /* a HIP launch failed; see q8_last_hip_error()            */
} q8_status;

typedef enum {
    Q8_ACT_BF16 = 0,   /* activations are bf16 [m][K]: W8A16                      */
    Q8_ACT_Q8 = 1      /* activations are Q8_0: int8 codes [m][K] + binary16 [m][K/32] */
} q8_act;

/* Version of this ABI (Q8_ABI_VERSION). */
int q8_abi_version(void);

/* Static, NUL-terminated name of a status code ("Q8_OK", ...); "unknown" for
 * values outside the enum. */
const char* q8_status_str(int status);

/* The hipError_t behind the most recent Q8_ERR_HIP or Q8_ERR_DEVICE returned
 * on this host thread; 0 when that failure was not a HIP error (wrong
 * architecture, stream of another device) or when no such failure happened. */
int q8_last_hip_error(void);

/* Quantize fp32 weights W [n][k] into codes wq [n][k] and binary16 scales
 * wd [n][k/32], following the Q8_0 rule above [fak MODEL-BASELINE-RESULTS,
 * ACT 3 item 1; ACT 4 "Correctness"].  Offline work, done once per weight. */
q8_status q8_quantize_weights(const float* w, int64_t n, int64_t k,
                              int8_t* wq, uint16_t* wd, hipStream_t stream);

/* Quantize bf16 activations X [m][k] into codes xq [m][k] and binary16 scales
 * xd [m][k/32] with the same rule [fak MODEL-BASELINE-RESULTS, ACT 5 "What
 * moved" item 3: the round-half-away activation quantizer, exact on zeros,
 * denormals and exact halves].  Any m >= 0. */
q8_status q8_quantize_act(const uint16_t* x, int64_t m, int64_t k,
                          int8_t* xq, uint16_t* xd, hipStream_t stream);

/* Batch-1 product y[n] = sum_b d[n][b] * sum_{i<32} q[n][32b+i] * x[32b+i],
 * fp32 accumulation [Frigg README, "The machine": at batch 1 every decode GEMM
 * is this matrix-vector shape, and its speed is bytes / bandwidth].
 *   act == Q8_ACT_BF16: x is bf16 [k], xd must be NULL.
 *   act == Q8_ACT_Q8:   x is int8 codes [k], xd is binary16 [k/32]; each block
 *                       contributes wd * xd * (exact int32 sum of code products)
 *                       [fak MODEL-BASELINE-RESULTS, ACT 3 item 3].
 * y is fp32 [n].  Same as q8_gemm_skinny with m = 1. */
q8_status q8_gemv(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k,
                  int act, const void* x, const uint16_t* xd,
                  float* y, hipStream_t stream);

/* Skinny product for m = 0..8 activation rows, reading every weight byte once
 * for all rows [Frigg README, Finding 8: looping the GEMV re-reads the weights
 * per row; a batched kernel costs nearly the same at every batch size].
 * x is bf16 [m][k] (act BF16) or int8 [m][k] with xd [m][k/32] (act Q8);
 * y is fp32 [m][n].  Row t of y depends on row t of x only, bit for bit; for a
 * given (n, k, m, act) results are bitwise reproducible, but a row's last bits
 * may differ between batch sizes (each may take another kernel and fp32
 * summation order; bf16 activations take the matrix cores at batch 5-8, and
 * at batch 2-4 on matrices of at least 64 rows per compute unit). */
q8_status q8_gemm_skinny(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k,
                         int64_t m, int act, const void* x, const uint16_t* xd,
                         float* y, hipStream_t stream);

/* Q8 x Q8 prefill product for p activation rows (0 <= p <= 4,194,240).  For K
 * a multiple of 512 (and K a multiple of 256 with at least as many 64 x 64
 * output tiles as compute units) the kernels use a fixed 36-80 KiB of LDS per
 * workgroup, for K up to 2^24.  For any other K a workgroup keeps the binary16
 * scales of its rows for the whole of K in LDS: 36 KiB + 128 bytes per
 * 32-element block must fit the device's per-workgroup LDS (K <= 7168 with 64
 * KiB, K <= 31744 with 160 KiB); a larger K returns Q8_ERR_SHAPE, checked after
 * the device check, with nothing enqueued.
 * y[t][j] = sum_b wd[j][b] * xd[t][b] * sum_{i<32} wq[j][32b+i] * xq[t][32b+i],
 * the int32 block sums taken on the int8 matrix cores, each block folded into an
 * fp32 accumulator with its two scales [fak MODEL-BASELINE-RESULTS, ACT 4,
 * "How the GEMM was closed": deferred per-block reduction, register-blocked
 * output tile].  y is fp32 [p][n]. */
q8_status q8_gemm_prefill(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k,
                          int64_t p, const int8_t* xq, const uint16_t* xd,
                          float* y, hipStream_t stream);

/* Fragment order: a second layout of a Q8_0 matrix, the one the int8 matrix
 * core reads.  For a matrix of `rows` rows and K columns (nb = K/32 blocks) let
 * rows64 = rows rounded up to a multiple of 64 and nbp = nb rounded up to a
 * multiple of 4; then
 *   codes  int8   [rows64 / 32][nbp][64][16]: entry (t, b, l, j) is code
 *          32b + 16 (l / 32) + j of row 32t + l % 32;
 *   scales uint16 [rows64 / 32][nbp / 4][32][4]: entry (t, g, i, u) is the
 *          binary16 scale of row 32t + i, block 4g + u;
 * rows >= `rows` and blocks >= nb hold zero codes and zero scales.  Every
 * (32-row tile, block) is one contiguous kilobyte, loaded by a wave with one
 * 16-byte load per lane into the registers the matrix core reads.  The byte
 * counts are those of the row-major matrix plus the padding:
 * q8_frag_code_bytes = rows64 * nbp * 32, q8_frag_scale_bytes = rows64 * nbp * 2
 * (-1 for an invalid K or rows; host-only, no device needed). */
int64_t q8_frag_code_bytes(int64_t rows, int64_t k);
int64_t q8_frag_scale_bytes(int64_t rows, int64_t k);

/* Rewrite a row-major Q8_0 matrix (codes q [rows][k], scales d [rows][k/32])
 * into fragment order (qf, df of the sizes above, padding included).  Weights
 * are packed once, next to their row-major copy; activation rows per call,
 * after quantization.  rows = 0 is a no-op; pointers 16-byte aligned. */
q8_status q8_pack_frag(const int8_t* q, const uint16_t* d, int64_t rows, int64_t k,
                       int8_t* qf, uint16_t* df, hipStream_t stream);

/* The Q8 x Q8 prefill product of q8_gemm_prefill on fragment-order operands:
 * wf / wdf the n weight rows, xf / xdf the p activation rows (both as written
 * by q8_pack_frag with the same K), 0 <= p <= 4,194,240, K <= 2^25; y fp32 [p][n]
 * row-major.  The same arithmetic [fak MODEL-BASELINE-RESULTS, ACT 4, "How the
 * GEMM was closed": every block's int32 sum taken exactly (here on the int8
 * matrix cores) and folded once into an fp32 accumulator with the product of
 * its two scales; register-blocked output tiles], with the operands loaded
 * straight from memory into the matrix core's registers instead of through
 * LDS.  fp32 summation order: blocks in order within each of up to 8 contiguous
 * K ranges, the ranges' partial sums added in order; results are bitwise
 * reproducible for a given (n, k, p) and exact whenever every partial sum is
 * (e.g. power-of-two scales).  A grid beyond 2^31 - 1 workgroups (a product of
 * more than ~2^35 32 x 32 output tiles) returns Q8_ERR_SHAPE after the device
 * check. */
q8_status q8_gemm_prefill_frag(const int8_t* wf, const uint16_t* wdf, int64_t n, int64_t k,
                               int64_t p, const int8_t* xf, const uint16_t* xdf,
                               float* y, hipStream_t stream);

/* The exact int32 block sums of the Q8 x Q8 product, exported so that they can
 * be compared bit for bit: isum[t][j][b] = sum_{i<32} wq[j][32b+i] * xq[t][32b+i]
 * for t < m (m = 0..8), j < n, b < k/32 [fak MODEL-BASELINE-RESULTS, ACT 3
 * item 3: signed x signed int8 block dot].  Uses the same block-dot routine as
 * the Q8-activation decode products (each half block on its own lane with
 * v_dot4_i32_i8, the two halves added across the lane pair); the prefill
 * product takes its block sums from the int8 matrix cores instead.  isum is
 * int32 [m][n][k/32]. */
q8_status q8_block_dots(const int8_t* wq, int64_t n, int64_t k, int64_t m,
                        const int8_t* xq, int32_t* isum, hipStream_t stream);

/* Diagnostics: the kernel (with its compile-time layout) that a product call
 * with these extents launches on the current device, so that a test can show
 * which code path a shape exercises.  op Q8_OP_SKINNY: q8_gemm_skinny with
 * m = rows and activation type act (also q8_gemv at rows = 1); Q8_OP_PREFILL:
 * q8_gemm_prefill with p = rows (act ignored); Q8_OP_Q4_SKINNY: q4_gemm_skinny;
 * Q8_OP_PREFILL_FRAG: q8_gemm_prefill_frag with p = rows (act ignored).
 * Writes a NUL-terminated name such as "skinny_kernel<1,0,16,2,6>" (batch,
 * activation type, lanes per group, rows per group, chunks per lane) or
 * "prefill_tile64_kernel<2>" or "prefill_frag_kernel<2,2>" (weight tiles per wave,
 * waves per K split) or "prefill_frag64_kernel<1>" (two token tiles and two
 * weight tiles per wave, long prompts; waves per K split) into buf, "none" for
 * an empty call.  Extents are
 * validated as by those calls (Q8_ERR_ENUM, Q8_ERR_SHAPE, Q8_ERR_BATCH); buf
 * NULL gives Q8_ERR_NULL, a name longer than buf_len - 1 bytes Q8_ERR_SHAPE;
 * no device gives Q8_ERR_DEVICE.  Enqueues nothing. */
typedef enum { Q8_OP_SKINNY = 0, Q8_OP_PREFILL = 1, Q8_OP_Q4_SKINNY = 2, Q8_OP_PREFILL_FRAG = 3 } q8_op;
q8_status q8_kernel_name(int op, int64_t n, int64_t k, int64_t rows, int act, char* buf, int64_t buf_len);

/* Decode attention over a Q8_0 key/value cache, one query row per head and no
 * mask [Frigg README: "Masks" (the single decode query attends to every cached
 * row unmasked), "Cache" (one static slab [heads][4096][128] per virtual layer
 * for K and for V), "The model, as verified" (12 heads of head_dim 128,
 * multi-head attention: one key/value head per query head)]:
 *
 *   s[j] = scale * sum_d q[h][d] * K[h][j][d]   for the cache rows j < t,
 *   out[h][d] = sum_j softmax(s)[j] * V[h][j][d],
 *
 * with K and V dequantized (codes times their block's binary16 scale; the
 * pages name an int8 cache without its layout, which is read as the same Q8_0
 * format: blocks of 32 along head_dim, e.g. as written by q8_quantize_act).
 * q: bf16 [heads][128]; kq, vq: int8 codes [heads][t_cap][128]; kd, vd:
 * binary16 scales [heads][t_cap][4] (row h * t_cap + j of the slab); out: fp32
 * [heads][128].  head_dim must be 128 (Q8_ERR_SHAPE otherwise); 1 <= t <= t_cap
 * <= 2^24 - 128; heads <= 65536 (0 is a no-op); scale finite.
 * `work`: caller-owned fp32 workspace of at least q8_attn_work_words(heads, t)
 * words (0 when t <= 256, and then `work` may be NULL); its contents on entry
 * do not matter and are overwritten.  Rows past t are never read.  fp32
 * accumulation; results are bitwise reproducible for a given (heads, t). */
q8_status q8_attn_decode(const uint16_t* q, const int8_t* kq, const uint16_t* kd,
                         const int8_t* vq, const uint16_t* vd, int64_t heads, int64_t t,
                         int64_t t_cap, int64_t head_dim, float scale, float* out,
                         float* work, int64_t work_words, hipStream_t stream);

/* For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): q8_attn_decode with the chunk partials kept in a static scratch
 * array of Q8_ATTN_SCRATCH_WORDS fp32 words (1 MiB) that the library holds on
 * each GPU it runs on until the process ends.  The call allocates and frees
 * nothing.  Arguments, results and errors are those of q8_attn_decode without
 * `work`; a (heads, t) whose q8_attn_work_words exceeds Q8_ATTN_SCRATCH_WORDS
 * returns Q8_ERR_SHAPE (checked before any HIP call, nothing enqueued), e.g.
 * 12 heads fit contexts up to 42,240 rows.  Every call on one GPU shares that
 * GPU's scratch and keeps no state in it between calls (each call writes the
 * partials it reads), but calls that overlap on one GPU -- on different
 * streams, or from several host threads without ordering -- race on it and
 * must not be issued. */
#define Q8_ATTN_SCRATCH_WORDS 262144
q8_status q8_attn_decode_noalloc(const uint16_t* q, const int8_t* kq, const uint16_t* kd,
                                 const int8_t* vq, const uint16_t* vd, int64_t heads, int64_t t,
                                 int64_t t_cap, int64_t head_dim, float scale, float* out,
                                 hipStream_t stream);

/* Workspace words q8_attn_decode needs for (heads, t), enough for every context
 * up to t (the count never decreases with t, so a workspace sized for t_cap
 * serves every call on that cache); -1 when out of range. */
int64_t q8_attn_work_words(int64_t heads, int64_t t);

/* Decode attention that first appends the token's own key and value: knew and
 * vnew are bf16 [heads][128] (the key already rotated); each 32-wide block is
 * quantized with the q8_quantize_act rule and written into row t - 1 of the
 * caches (kq, vq codes; kd, vd scales), then the attention of q8_attn_decode
 * runs over rows [0, t) with those rows.  The launch that computes it writes
 * row t - 1 and reads nothing else it writes.  Same arguments, workspace and
 * errors as q8_attn_decode otherwise; knew and vnew must be non-NULL and
 * 16-byte aligned (Q8_ERR_NULL / Q8_ERR_ALIGN). */
q8_status q8_attn_decode_append(const uint16_t* q, int8_t* kq, uint16_t* kd, int8_t* vq, uint16_t* vd,
                                int64_t heads, int64_t t, int64_t t_cap, int64_t head_dim, float scale,
                                const uint16_t* knew, const uint16_t* vnew, float* out, float* work,
                                int64_t work_words, hipStream_t stream);

/* The attention of q8_attn_decode_append without its combine step, for
 * q8_gemm_attn_residual: the token's key and value rows are appended as there,
 * and the per-chunk partials -- per head and chunk of cache rows, a record of
 * 132 floats: the numerator sum_j e^(s_j - m) V_j [128], the chunk's largest
 * score m, the denominator sum_j e^(s_j - m), 2 unused -- are left in `work`
 * (also when one chunk covers the context); nothing else is written.  work:
 * fp32, at least q8_attn_partial_words(heads, t) words (-1 when out of range;
 * like q8_attn_work_words it covers every context up to t).
 * Other arguments and errors as q8_attn_decode_append, without `out`. */
int64_t q8_attn_partial_words(int64_t heads, int64_t t);
q8_status q8_attn_decode_append_partials(const uint16_t* q, int8_t* kq, uint16_t* kd, int8_t* vq,
                                         uint16_t* vd, int64_t heads, int64_t t, int64_t t_cap,
                                         int64_t head_dim, float scale, const uint16_t* knew,
                                         const uint16_t* vnew, float* work, int64_t work_words,
                                         hipStream_t stream);

/* The attention output projection with its residual add, reading the
 * attention partials directly [Frigg README, Findings 3 and 8: every launch of a
 * batch-1 step costs; this one saves the combine launch]:
 *   h[j] += sum_i W[j][i] * bf16(a[i]),   a = the attention output [k/128][128],
 * where a is combined from the partials q8_attn_decode_append_partials left in
 * `work` for the same (heads = k / 128, t), exactly as q8_attn_decode combines
 * them (bit for bit).  wq/wd Q8_0 [n][k]; h fp32 [n], read and written.  k a
 * multiple of 128 with 128 <= k <= 2048 (the row is combined once per
 * workgroup); 1 <= t <= 4096 (at most 16 chunks of cache rows); work_words at
 * least q8_attn_partial_words(k / 128, t); Q8_ERR_SHAPE otherwise.  Other
 * conventions as q8_gemm_fused with Q8_EPI_ADD at m = 1. */
q8_status q8_gemm_attn_residual(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, const float* work,
                                int64_t work_words, int64_t t, float* h, hipStream_t stream);

/* ---- decode-step glue fused into the W8A16 products ---------------------------
 *
 * A decode block [Frigg README, "The model, as verified": pre-norm blocks,
 * RMSNorm without a learnable weight (eps 1e-6) and a final norm per module run;
 * rotary embedding with theta 10,000, default rotation; SwiGLU MLP; 12 heads of
 * 128] needs glue between its products.  q8_gemm_fused runs a W8A16 product
 * (Q8_0 weights, fp32 accumulation, m = 0..8 rows) with one prologue on its
 * activations and one epilogue on its outputs, so a block is its four product
 * launches plus attention.
 *
 * Prologues (x, row-major [m][k]):
 *   Q8_PRO_BF16     x is bf16, used as is.
 *   Q8_PRO_F32      x is fp32, rounded to bf16 (nearest, ties to even).
 *   Q8_PRO_RMSNORM  x is fp32; each row is scaled by 1 / sqrt(mean(x^2) + 1e-6)
 *                   (fp32 arithmetic, the reduction of q8_rmsnorm) and rounded
 *                   to bf16.
 * Epilogues (y[t][j] = the product, fp32):
 *   Q8_EPI_F32      out fp32 [m][n] = y.
 *   Q8_EPI_ADD      out fp32 [m][n] += y (the residual stream; read and written).
 *   Q8_EPI_SWIGLU   n even; rows 2j and 2j + 1 are gate_j and up_j; out bf16
 *                   [m][n/2]: out[t][j] = bf16(g / (1 + exp(-g)) * u).
 *   Q8_EPI_ROPE     n even; rows [0, rope_rows) (rope_rows a multiple of 128)
 *                   hold heads of 128 in pair order: row 2(64h + i) is dimension
 *                   i of head h and the next row dimension i + 64; each pair
 *                   (a, b) turns by the angle pos * 10000^(-i/64) (computed in
 *                   fp64): out[t][128h + i] = bf16(a cos - b sin),
 *                   out[t][128h + i + 64] = bf16(b cos + a sin).  Rows from
 *                   rope_rows on are copied: out[t][j] = bf16(y[t][j]).  out bf16
 *                   [m][n] in natural dimension order.
 * Supported pairs (others return Q8_ERR_ENUM): RMSNORM+ROPE (qkv), F32+ADD (o),
 * RMSNORM+SWIGLU (gate/up), BF16+ADD (down), F32+F32 and RMSNORM+F32 (lm_head).
 * `out` must not overlap x, wq or wd.  rope_rows and pos are read only by the
 * ROPE epilogue (0 <= rope_rows <= n, 0 <= pos < 2^31).  Other conventions are
 * those of the Q8_0 products. */
typedef enum { Q8_PRO_BF16 = 0, Q8_PRO_F32 = 1, Q8_PRO_RMSNORM = 2 } q8_prologue;
typedef enum { Q8_EPI_F32 = 0, Q8_EPI_ADD = 1, Q8_EPI_SWIGLU = 2, Q8_EPI_ROPE = 3 } q8_epilogue;

q8_status q8_gemm_fused(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t m,
                        int prologue, const void* x, int epilogue, void* out,
                        int64_t rope_rows, int64_t pos, hipStream_t stream);

/* Weightless RMSNorm of m fp32 rows of length k (the final norm of a module
 * run): y = x / sqrt(mean(x^2) + 1e-6), fp32, with the same reduction as the
 * RMSNORM prologue.  y may be x (in place).  k a multiple of 32 (the K of the
 * products it feeds), 32 <= k < 2^31; 0 <= m < 2^31, m * k <= 2^46. */
q8_status q8_rmsnorm(const float* x, int64_t m, int64_t k, float* y, hipStream_t stream);

/* The activation side of a Q8 x Q8 prefill product in one launch: the fp32
 * rows x [m][k] go through the prologue -- Q8_PRO_F32: rounded to bf16;
 * Q8_PRO_RMSNORM: scaled by 1 / sqrt(mean(x^2) + 1e-6) (the reduction of
 * q8_rmsnorm) and rounded to bf16 -- and the bf16 rows are quantized exactly
 * as q8_quantize_act would (xq int8 [m][k], xd binary16 [m][k/32]) [Frigg
 * README, "The model, as verified": the norm before every product that reads
 * the residual stream; fak MODEL-BASELINE-RESULTS, ACT 5 "What moved" item 3:
 * the activation quantizer].  Bit-identical to q8_rmsnorm, bf16 rounding and
 * q8_quantize_act in sequence.  Other prologues return Q8_ERR_ENUM; k and m as
 * for q8_rmsnorm; outputs must not overlap x. */
q8_status q8_quantize_act_fused(const float* x, int64_t m, int64_t k, int prologue, int8_t* xq,
                                uint16_t* xd, hipStream_t stream);

/* q8_quantize_act_fused writing fragment order: the same codes and scales, in
 * the layout of q8_pack_frag (xqf of q8_frag_code_bytes(m, k) bytes, xdf of
 * q8_frag_scale_bytes(m, k)), padding rows and blocks written as zeros, so the
 * activation side of q8_gemm_prefill_frag is one launch.  Bit-identical to
 * q8_quantize_act_fused followed by q8_pack_frag.  0 <= m <= 4,194,240;
 * otherwise as q8_quantize_act_fused. */
q8_status q8_quantize_act_fused_frag(const float* x, int64_t m, int64_t k, int prologue, int8_t* xqf,
                                     uint16_t* xdf, hipStream_t stream);

/* ---- int4 weights ----------------------------------------------------------
 *
 * The pages price and measure an "int4 core + int8 vocab" build (Frigg README:
 * bytes-per-token table, benchmark matrix row "int4 W / int8 vocab"; "Known
 * limits" reports int4 as slower and less accurate than int8 there) but give no
 * int4 layout.  It is read as the Q8_0 rule above with 7 in place of 127:
 * blocks of 32 along K, one binary16 scale d = maxabs / 7 (fp32 quotient
 * rounded to binary16, nearest-even), codes clamp(round_half_away(w / d), -7, 7)
 * against the stored d, all-zero codes for a zero scale.  Codes are packed two
 * per byte as 4-bit two's complement: byte j of a block's 16 bytes holds element
 * j in bits 0-3 and element j + 16 in bits 4-7.
 *   int4 codes [rows][K/2] bytes (row pitch K/2), scales [rows][K/32] binary16;
 *   18 bytes per 32 weights (0.5625 B/weight).
 * Conventions (pointers, alignment, ownership, asynchrony, errors, empty calls,
 * determinism) are those of the Q8_0 calls. */

/* Quantize fp32 weights W [n][k] into packed int4 codes wq [n][k/2] and
 * binary16 scales wd [n][k/32] with the rule above.  Offline work. */
q8_status q4_quantize_weights(const float* w, int64_t n, int64_t k,
                              uint8_t* wq, uint16_t* wd, hipStream_t stream);

/* Batch 0..8 product over int4 weights, reading every weight byte once for all
 * m rows [Frigg README, Finding 8; "The machine": at batch 1 the time is weight
 * bytes / bandwidth]:
 *   y[t][j] = sum_b wd[j][b] * sum_{i<32} c[j][32b+i] * x[t][32b+i],
 * c the unpacked codes.  act Q8_ACT_BF16: x is bf16 [m][k], xd NULL, fp32
 * accumulation.  act Q8_ACT_Q8: x is int8 codes [m][k] with binary16 xd
 * [m][k/32]; each block contributes wd * xd * (exact int32 sum of code
 * products).  y is fp32 [m][n].  Batch behaviour as q8_gemm_skinny (bf16
 * activations at batch 2-8 go to the matrix cores on most shapes). */
q8_status q4_gemm_skinny(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k,
                         int64_t m, int act, const void* x, const uint16_t* xd,
                         float* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8STREAM_H */
