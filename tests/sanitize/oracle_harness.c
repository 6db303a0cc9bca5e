/* Harness for the oracle (q8_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every exported function on small inputs with the
 * edge cases the pins use (zero and negative-zero blocks, binary16-subnormal
 * scales, exact halves, K = 32, ragged shapes, one-row caches), plus a few
 * closed-form checks so that a sanitizer build that computed garbage would
 * also fail.  Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_set_threads(int n);
double oracle_half_to_double(uint16_t h);
uint16_t oracle_half_from_double(double v);
double oracle_rhaway(float t);
void oracle_rhaway_array(const float* t, int64_t n, int32_t* out);
uint16_t oracle_block_scale(float amax);
void oracle_quantize_f32(const float* w, int64_t n, int64_t k, int8_t* q, uint16_t* d);
void oracle_quantize_bf16(const uint16_t* x, int64_t m, int64_t k, int8_t* q, uint16_t* d);
void oracle_rmsnorm(const float* x, int64_t m, int64_t k, double eps, double* y);
void oracle_rope(double* v, int64_t heads, int64_t d, int64_t pos, double theta);
void oracle_swiglu(const double* g, const double* u, int64_t n, double* s);
uint16_t oracle_q4_block_scale(float amax);
void oracle_q4_quantize_f32(const float* w, int64_t n, int64_t k, uint8_t* q, uint16_t* d);
void oracle_q4_unpack(const uint8_t* q, int64_t n, int64_t k, int8_t* codes);
void oracle_w8a16(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t m, const uint16_t* x,
                  const int64_t* rows, int64_t nrows, double* y);
void oracle_block_dots(const int8_t* wq, int64_t n, int64_t k, const int8_t* xq, int64_t m, int32_t* out);
void oracle_q8q8(const int8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t m, const int8_t* xq,
                 const uint16_t* xd, const int64_t* rows, int64_t nrows, double* y);
void oracle_attn_decode(const uint16_t* q, const int8_t* kq, const uint16_t* kd, const int8_t* vq,
                        const uint16_t* vd, int64_t heads, int64_t t, int64_t t_cap, int64_t d, double scale,
                        double* out);

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static uint16_t bf16(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)((u + 0x7FFF + ((u >> 16) & 1)) >> 16); }

int main(void) {
    enum { N = 7, K = 96, M = 3 };
    oracle_set_threads(3);
    EXPECT(oracle_rhaway(0.49999997f) == 0.0 && oracle_rhaway(2.5f) == 3.0 && oracle_rhaway(-0.5f) == -1.0);
    float ts[5] = {0.5f, -1.5f, 126.5f, -0.0f, 3.2f};
    int32_t r[5];
    oracle_rhaway_array(ts, 5, r);
    EXPECT(r[0] == 1 && r[1] == -2 && r[2] == 127 && r[3] == 0 && r[4] == 3);
    EXPECT(oracle_half_to_double(0x3C00) == 1.0 && oracle_half_from_double(1.0) == 0x3C00);
    EXPECT(oracle_block_scale(127.0f) == 0x3C00 && oracle_block_scale(0.0f) == 0);

    float w[N * K];
    srand(7);
    for (int i = 0; i < N * K; ++i) w[i] = ((float)rand() / RAND_MAX - 0.5f) * 0.04f;
    for (int i = 0; i < 32; ++i) { w[i] = 0.0f; w[K + i] = -0.0f; w[2 * K + i] = 1e-6f * (i - 16); }
    w[3 * K] = 127.0f; w[3 * K + 1] = 0.5f;                          /* exact half */
    int8_t wq[N * K]; uint16_t wd[N * K / 32];
    oracle_quantize_f32(w, N, K, wq, wd);
    EXPECT(wd[0] == 0 && wd[K / 32] == 0 && wq[0] == 0 && wq[K] == 0);
    EXPECT(wd[3 * K / 32] == 0x3C00 && wq[3 * K] == 127 && wq[3 * K + 1] == 1);

    uint16_t x[M * K];
    for (int i = 0; i < M * K; ++i) x[i] = bf16(((float)rand() / RAND_MAX - 0.5f) * 4.0f);
    int8_t xq[M * K]; uint16_t xd[M * K / 32];
    oracle_quantize_bf16(x, M, K, xq, xd);
    double y[M * N], yq[M * N];
    oracle_w8a16(wq, wd, N, K, M, x, NULL, N, y);
    int64_t rows[2] = {6, 0};
    double ys[M * 2];
    oracle_w8a16(wq, wd, N, K, M, x, rows, 2, ys);
    EXPECT(ys[0] == y[6] && ys[1] == y[0]);
    int32_t isum[M * N * (K / 32)];
    oracle_block_dots(wq, N, K, xq, M, isum);
    oracle_q8q8(wq, wd, N, K, M, xq, xd, NULL, N, yq);
    for (int t = 0; t < M; ++t)
        for (int j = 0; j < N; ++j) {
            double s = 0.0;
            for (int b = 0; b < K / 32; ++b)
                s += oracle_half_to_double(wd[j * (K / 32) + b]) * oracle_half_to_double(xd[t * (K / 32) + b]) *
                     isum[(t * N + j) * (K / 32) + b];
            EXPECT(fabs(s - yq[t * N + j]) <= 1e-12 * (1.0 + fabs(s)));
        }

    double hx[2 * 64], hy[2 * 64];
    float hf[2 * 64];
    for (int i = 0; i < 128; ++i) hf[i] = (float)(i % 5) - 2.0f;
    oracle_rmsnorm(hf, 2, 64, 1e-6, hy);
    for (int i = 0; i < 128; ++i) hx[i] = hy[i];
    oracle_rope(hx, 1, 128, 5, 10000.0);
    double g[4] = {0.0, 1.0, -40.0, 40.0}, u[4] = {1, 1, 1, 1}, s4[4];
    oracle_swiglu(g, u, 4, s4);
    EXPECT(s4[0] == 0.0 && fabs(s4[3] - 40.0) < 1e-9);

    uint8_t q4[N * K / 2]; uint16_t d4[N * K / 32]; int8_t c4[N * K];
    EXPECT(oracle_q4_block_scale(7.0f) == 0x3C00);
    oracle_q4_quantize_f32(w, N, K, q4, d4);
    oracle_q4_unpack(q4, N, K, c4);
    for (int i = 0; i < N * K; ++i) EXPECT(c4[i] >= -7 && c4[i] <= 7);

    /* attention: 2 heads, a cache of capacity 3 with one row used, then all */
    int8_t kq[2 * 3 * 128], vq[2 * 3 * 128]; uint16_t kd[2 * 3 * 4], vd[2 * 3 * 4], q[2 * 128];
    for (int i = 0; i < 2 * 3 * 128; ++i) { kq[i] = (int8_t)(i % 255 - 127); vq[i] = (int8_t)((i * 7) % 255 - 127); }
    for (int i = 0; i < 2 * 3 * 4; ++i) { kd[i] = 0x2000; vd[i] = 0x3C00; }
    for (int i = 0; i < 2 * 128; ++i) q[i] = bf16((float)(i % 9) - 4.0f);
    double out[2 * 128];
    oracle_attn_decode(q, kq, kd, vq, vd, 2, 1, 3, 128, 0.088, out);
    EXPECT(out[0] == (double)vq[0] && out[128] == (double)vq[3 * 128]);   /* one row: its value row */
    oracle_attn_decode(q, kq, kd, vq, vd, 2, 3, 3, 128, 0.088, out);
    printf("%s\n", fails ? "FAILED" : "oracle harness ok");
    return fails ? 1 : 0;
}
