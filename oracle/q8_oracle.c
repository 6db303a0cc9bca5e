/*
 * q8_oracle.c -- plain, slow CPU oracle for the Q8_0 weight-streaming path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no source with the HIP library.
 *
 * What it computes, and where the pages define it:
 *
 *  - Q8_0 block format [fak MODEL-BASELINE-RESULTS, ACT 3, "How it was closed",
 *    item 1]: weights and activations are cut into blocks of 32 consecutive
 *    elements along the reduction axis; each block keeps int8 codes and one
 *    scale d = maxabs / 127.  The page calls the scale f32 but prices the
 *    format at about 1.06 bytes per weight, i.e. a 2-byte scale; the scale is
 *    stored here as IEEE binary16.  The division by 127 is done in fp32 (the
 *    page's scale precision), then rounded to binary16, nearest-even.
 *  - Codes are round-half-away-from-zero of w / s, in fp32, with s the STORED
 *    binary16 scale [fak MODEL-BASELINE-RESULTS, ACT 4, "Correctness": the
 *    rounding must equal math.Round over the whole code range, and adding 0.5
 *    then truncating is wrong because 0.49999997 + 0.5 rounds up to 1 in fp32;
 *    ACT 5, "What moved", item 3: zeros, denormals and exact halves].
 *    Codes are clamped to [-127, 127]; a block whose scale is zero gets all-zero
 *    codes with no division.
 *  - W8A16 product: y[m][n] = sum_k q[n][k] * s[n][k/32] * x[m][k], every term
 *    and the sum in fp64 (dequantize, then matmul).  This is the batch-1 decode
 *    GEMV of the Frigg README ("The machine", bench vram table: the lm_head
 *    shape [1,1536] x [1536,262144]) and its batched form (Finding 8).
 *  - Q8 x Q8 product: isum[m][n][b] = sum_{i<32} wq[n][32b+i] * xq[m][32b+i] in
 *    exact integers, y[m][n] = sum_b wd[n][b] * xd[m][b] * isum[m][n][b] in
 *    fp64 [fak MODEL-BASELINE-RESULTS, ACT 3 item 3 (signed x signed int8 block
 *    dot) and ACT 4, "How the GEMM was closed" (per-block int32 sum folded into
 *    a float accumulator with the block's scales)].
 *
 *  - The glue of a decode step [Frigg README, "The model, as verified": RMSNorm
 *    with no learnable weight, eps 1e-6, pre-norm and a final norm per module;
 *    RoPE with theta 10,000 and the default rotation; SwiGLU MLP; residual
 *    stream]: rmsnorm(x)_i = x_i / sqrt(mean_j x_j^2 + 1e-6); the default
 *    rotation pairs dimension i with i + 64 of a 128-wide head and turns the
 *    pair by pos * 10000^(-i/64); swiglu(g, u) = g / (1 + e^-g) * u.  All in
 *    fp64 from fp32 inputs.
 *
 *  - int4 weights [Frigg README, bytes-per-token table ("int4 core + int8
 *    vocab") and benchmark matrix ("int4 W / int8 vocab"); "Known limits":
 *    int4 is implemented there but slower and less accurate than int8].  The
 *    pages give no int4 layout; it is read as the Q8_0 rule with the largest
 *    4-bit magnitude in place of 127: blocks of 32 along the reduction axis,
 *    d = maxabs / 7 (fp32 division, then binary16), codes
 *    clamp(round_half_away(w / d), -7, 7) against the stored d, zero codes for
 *    a zero scale.  Two codes share a byte as 4-bit two's complement: byte j of
 *    a block holds element j in bits 0-3 and element j + 16 in bits 4-7, so a
 *    block is 16 bytes of codes plus its 2-byte scale (0.5625 B/weight).  The
 *    products over int4 weights are the W8A16 and Q8 x Q8 products above with
 *    the unpacked codes (values in [-7, 7]) in place of the int8 codes.
 *
 *  - Decode attention over a Q8_0 key/value cache [Frigg README, "The model, as
 *    verified": hidden 1536 = 12 heads x head_dim 128, multi-head attention
 *    with 12 key/value heads; "Masks": the single decode query attends to
 *    every cached row unmasked; "Cache": one static slab [heads][4096][128] per
 *    virtual layer for K and for V; the bytes-per-token table counts an int8
 *    KV read per token].  The pages name int8 KV without its block layout; it
 *    is read here as the same Q8_0 format (blocks of 32 along head_dim, one
 *    binary16 scale each).  For head h over the first t cache rows:
 *    s[j] = scale * sum_d q[h][d] * K[h][j][d],  w = softmax(s),
 *    out[h][d] = sum_j w[j] * V[h][j][d], in fp64 with K and V dequantized.
 *
 * Threading: output rows are split over OpenMP threads; each output is computed
 * by one thread in a fixed order, so results do not depend on the thread count
 * [fak MODEL-BASELINE-RESULTS, ACT 1, "Parity lane": row-parallel matmul].
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int oracle_get_threads(void) { return g_threads; }

/* ---------- binary16 and bfloat16 ---------- */

/* Value of an IEEE binary16 bit pattern. */
double oracle_half_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a finite value v >= 0 to binary16, nearest with ties to even; returns
 * the bit pattern (0x7C00 on overflow).  The value is scaled by the binary16
 * quantum of its binade (a power of two, so exactly), rounded to an integer
 * with rint() in the default round-to-nearest-even mode, and scaled back. */
uint16_t oracle_half_from_double(double v) {
    if (!(v > 0.0)) return 0;
    int ex;
    frexp(v, &ex);                   /* v in [2^(ex-1), 2^ex) */
    int unit = ex - 1;               /* exponent of the leading bit */
    int qexp = unit < -14 ? -24 : unit - 10;   /* quantum 2^qexp */
    double r = rint(ldexp(v, -qexp));          /* integer, exact scaling */
    double hv = ldexp(r, qexp);
    if (hv >= 65520.0) return 0x7C00;
    if (hv < ldexp(1.0, -14))
        return (uint16_t)r;                    /* subnormal: mantissa = r */
    frexp(hv, &ex);
    unit = ex - 1;
    double mant = ldexp(hv, -(unit - 10)) - 1024.0;   /* 0..1023 */
    return (uint16_t)(((unit + 15) << 10) | (int)mant);
}

float oracle_bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ---------- the quantizer ---------- */

/* Round half away from zero of a float, exactly: sign(t) * floor(|t| + 1/2).
 * |t| + 1/2 is formed in fp64; for |t| >= 2^-30 the sum is exact, and below
 * that floor() gives 0 either way. */
double oracle_rhaway(float t) {
    double a = fabs((double)t);
    double r = floor(a + 0.5);
    return t < 0.0f ? -r : r;
}

void oracle_rhaway_array(const float* t, int64_t n, int32_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)oracle_rhaway(t[i]);
}

/* Scale of one block from its largest magnitude: fp32 amax / 127, to binary16. */
uint16_t oracle_block_scale(float amax) {
    float d = amax / 127.0f;                    /* fp32 division, correctly rounded */
    return oracle_half_from_double((double)d);
}

/* Quantize one 32-element block of fp32 values. */
static void quantize_block(const float* v, int8_t* q, uint16_t* d) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    uint16_t s16 = oracle_block_scale(amax);
    *d = s16;
    float s = (float)oracle_half_to_double(s16);
    for (int i = 0; i < 32; ++i) {
        if (s == 0.0f) { q[i] = 0; continue; }
        float t = v[i] / s;                     /* fp32 division by the stored scale */
        double c = oracle_rhaway(t);
        if (c > 127.0) c = 127.0;
        if (c < -127.0) c = -127.0;
        q[i] = (int8_t)c;
    }
}

/* fp32 W [n][k] -> codes [n][k], binary16 scales [n][k/32].  k % 32 == 0. */
void oracle_quantize_f32(const float* w, int64_t n, int64_t k, int8_t* q, uint16_t* d) {
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b)
            quantize_block(w + r * k + 32 * b, q + r * k + 32 * b, d + r * nb + b);
}

/* bf16 X [m][k] -> codes [m][k], binary16 scales [m][k/32].  k % 32 == 0. */
void oracle_quantize_bf16(const uint16_t* x, int64_t m, int64_t k, int8_t* q, uint16_t* d) {
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t r = 0; r < m; ++r) {
        float v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 32; ++i) v[i] = oracle_bf16_to_float(x[r * k + 32 * b + i]);
            quantize_block(v, q + r * k + 32 * b, d + r * nb + b);
        }
    }
}

/* ---------- decode-step glue ---------- */

/* Weightless RMSNorm of each of m rows of length k: y = x / sqrt(mean(x^2) + eps). */
void oracle_rmsnorm(const float* x, int64_t m, int64_t k, double eps, double* y) {
    for (int64_t r = 0; r < m; ++r) {
        double ss = 0.0;
        for (int64_t i = 0; i < k; ++i) ss += (double)x[r * k + i] * (double)x[r * k + i];
        const double inv = 1.0 / sqrt(ss / (double)k + eps);
        for (int64_t i = 0; i < k; ++i) y[r * k + i] = (double)x[r * k + i] * inv;
    }
}

/* Rotary embedding of `heads` heads of width d (even) at position pos, in place
 * on fp64 values: dimension i < d/2 pairs with i + d/2 and the pair turns by
 * pos * theta^(-2i/d). */
void oracle_rope(double* v, int64_t heads, int64_t d, int64_t pos, double theta) {
    const int64_t half = d / 2;
    for (int64_t h = 0; h < heads; ++h)
        for (int64_t i = 0; i < half; ++i) {
            const double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
            const double c = cos(ang), sn = sin(ang);
            double* a = v + h * d + i;
            double* b = v + h * d + i + half;
            const double x0 = *a, x1 = *b;
            *a = x0 * c - x1 * sn;
            *b = x1 * c + x0 * sn;
        }
}

/* SwiGLU: s_j = g_j / (1 + exp(-g_j)) * u_j, n values. */
void oracle_swiglu(const double* g, const double* u, int64_t n, double* s) {
    for (int64_t j = 0; j < n; ++j) s[j] = g[j] / (1.0 + exp(-g[j])) * u[j];
}

/* ---------- int4 weights ---------- */

/* Scale of one int4 block: fp32 amax / 7, to binary16. */
uint16_t oracle_q4_block_scale(float amax) {
    float d = amax / 7.0f;                      /* fp32 division, correctly rounded */
    return oracle_half_from_double((double)d);
}

/* Codes in [-7, 7] of one 32-element block of fp32 values, and its scale. */
static void q4_codes_block(const float* v, int* c, uint16_t* d) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    uint16_t s16 = oracle_q4_block_scale(amax);
    *d = s16;
    float s = (float)oracle_half_to_double(s16);
    for (int i = 0; i < 32; ++i) {
        if (s == 0.0f) { c[i] = 0; continue; }
        float t = v[i] / s;                     /* fp32 division by the stored scale */
        double r = oracle_rhaway(t);
        if (r > 7.0) r = 7.0;
        if (r < -7.0) r = -7.0;
        c[i] = (int)r;
    }
}

/* Low 4 bits of a code in two's complement (-7 -> 9, -1 -> 15, 3 -> 3). */
static unsigned q4_nibble(int c) { return (unsigned)(c < 0 ? c + 16 : c); }

/* fp32 W [n][k] -> packed codes [n][k/2], binary16 scales [n][k/32]; k % 32 == 0. */
void oracle_q4_quantize_f32(const float* w, int64_t n, int64_t k, uint8_t* q, uint16_t* d) {
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            int c[32];
            q4_codes_block(w + r * k + 32 * b, c, d + r * nb + b);
            uint8_t* out = q + r * (k / 2) + 16 * b;
            for (int j = 0; j < 16; ++j)
                out[j] = (uint8_t)(q4_nibble(c[j]) | (q4_nibble(c[j + 16]) << 4));
        }
}

/* Packed codes [n][k/2] -> one int8 per code [n][k]. */
void oracle_q4_unpack(const uint8_t* q, int64_t n, int64_t k, int8_t* codes) {
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 32; ++b) {
            const uint8_t* in = q + r * (k / 2) + 16 * b;
            int8_t* out = codes + r * k + 32 * b;
            for (int j = 0; j < 16; ++j) {
                int lo = in[j] & 15, hi = in[j] >> 4;
                out[j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
                out[j + 16] = (int8_t)(hi >= 8 ? hi - 16 : hi);
            }
        }
}

/* ---------- products ---------- */

/* W8A16: y[mi][r] = sum_k q[r][k] * s[r][k/32] * x[mi][k] in fp64, for the
 * output rows r in rows[0..nrows) (all rows when rows == NULL, nrows == n).
 * y is [m][nrows]. */
void oracle_w8a16(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k,
                  int64_t m, const uint16_t* x, const int64_t* rows, int64_t nrows,
                  double* y) {
    int64_t nb = k / 32;
    (void)n;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t r = rows ? rows[j] : j;
        for (int64_t mi = 0; mi < m; ++mi) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) {
                double wv = (double)wq[r * k + kk] * oracle_half_to_double(wd[r * nb + kk / 32]);
                acc += wv * (double)oracle_bf16_to_float(x[mi * k + kk]);
            }
            y[mi * nrows + j] = acc;
        }
    }
}

/* Exact int32 block dots: isum[mi][r][b] = sum_{i<32} wq[r][32b+i] * xq[mi][32b+i]. */
void oracle_block_dots(const int8_t* wq, int64_t n, int64_t k, const int8_t* xq,
                       int64_t m, int32_t* isum) {
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t mi = 0; mi < m; ++mi)
            for (int64_t b = 0; b < nb; ++b) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i)
                    s += (int32_t)wq[r * k + 32 * b + i] * (int32_t)xq[mi * k + 32 * b + i];
                isum[(mi * n + r) * nb + b] = s;
            }
}

/* Q8 x Q8: y[mi][r] = sum_b wd[r][b] * xd[mi][b] * isum[mi][r][b] in fp64, rows
 * as in oracle_w8a16; y is [m][nrows]. */
void oracle_q8q8(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k,
                 int64_t m, const int8_t* xq, const uint16_t* xd,
                 const int64_t* rows, int64_t nrows, double* y) {
    int64_t nb = k / 32;
    (void)n;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t r = rows ? rows[j] : j;
        for (int64_t mi = 0; mi < m; ++mi) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i)
                    s += (int32_t)wq[r * k + 32 * b + i] * (int32_t)xq[mi * k + 32 * b + i];
                acc += oracle_half_to_double(wd[r * nb + b]) *
                       oracle_half_to_double(xd[mi * nb + b]) * (double)s;
            }
            y[mi * nrows + j] = acc;
        }
    }
}

/* Decode attention, one bf16 query row per head against t rows of a Q8_0 key
 * and value cache laid out [heads][t_cap][d] (codes) and [heads][t_cap][d/32]
 * (binary16 scales).  Softmax with the maximum subtracted first (the value is
 * that of the plain definition; the subtraction only keeps exp in range).
 * out is fp64 [heads][d]. */
void oracle_attn_decode(const uint16_t* q, const int8_t* kq, const uint16_t* kd,
                        const int8_t* vq, const uint16_t* vd, int64_t heads, int64_t t,
                        int64_t t_cap, int64_t d, double scale, double* out) {
    int64_t nb = d / 32;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int64_t h = 0; h < heads; ++h) {
        double* s = (double*)malloc(sizeof(double) * (size_t)(t > 0 ? t : 1));
        double smax = -INFINITY;
        for (int64_t j = 0; j < t; ++j) {
            const int64_t row = h * t_cap + j;
            double acc = 0.0;
            for (int64_t e = 0; e < d; ++e)
                acc += (double)oracle_bf16_to_float(q[h * d + e]) *
                       ((double)kq[row * d + e] * oracle_half_to_double(kd[row * nb + e / 32]));
            s[j] = scale * acc;
            if (s[j] > smax) smax = s[j];
        }
        double sum = 0.0;
        for (int64_t j = 0; j < t; ++j) {
            s[j] = exp(s[j] - smax);
            sum += s[j];
        }
        for (int64_t e = 0; e < d; ++e) {
            double o = 0.0;
            for (int64_t j = 0; j < t; ++j) {
                const int64_t row = h * t_cap + j;
                o += s[j] * ((double)vq[row * d + e] * oracle_half_to_double(vd[row * nb + e / 32]));
            }
            out[h * d + e] = o / sum;
        }
        free(s);
    }
}
