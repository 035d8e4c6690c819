/* Drives every function of the CPU oracle (oracle/moe_oracle.c) on small
 * inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * any out-of-range access, use after free, signed overflow or misaligned
 * load aborts the run.  Also checks a few invariants of the results so the
 * run cannot pass by skipping work.  Exit status 0 = clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_exp_spec(float y);
float oracle_sigmoid_spec(float x);
double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float x);
void oracle_sigmoid_spec_n(const float* x, int64_t n, float* out);
void oracle_exp_spec_n(const float* x, int64_t n, float* out);
void oracle_e4m3_encode_n(const float* x, int64_t n, uint8_t* out);
void oracle_router_scores(const uint16_t* u, const uint16_t* e, int64_t T, int d, int E, float* s);
void oracle_topk_from_scores(const float* s, const float* bias, int64_t T, int E, int K, int32_t* idx, float* gate);
void oracle_topk_grouped_from_scores(const float* s, const float* bias, int64_t T, int E, int K, int n_groups,
                                     int topk_groups, int32_t* idx, float* gate);
void oracle_seq_balance_loss(const float* s, const int32_t* idx, int64_t T, int E, int K, int L, double alpha,
                             double* loss);
int oracle_dispatch(const int32_t* idx, int64_t T, int K, int E, int include_shared, int32_t* count,
                    int32_t* group_offset, int32_t* row_token, int32_t* slot_row);
void oracle_quant_1x128(const float* x, int64_t rows, int cols, uint8_t* q, float* scale);
void oracle_quant_128x128(const float* w, int64_t rows, int cols, uint8_t* q, float* scale);
void oracle_gemm_blockscaled(const uint8_t* qa, const float* sa, const int32_t* a_rows, int64_t M, const uint8_t* qb,
                             const float* sb, int N, int K, double* out);
void oracle_swiglu(const double* zg, const double* zu, int64_t n, double* h);
void oracle_combine(const uint16_t* u, const double* y, int64_t shared_row0, const float* gate,
                    const int32_t* slot_row, int64_t T, int K, int d, double* out);
void oracle_bias_update(float* bias, const int32_t* count, int E, int64_t total_assignments, float gamma);
void oracle_set_threads(int n);
int oracle_max_threads(void);

static uint64_t rng_state = 88172645463325252ull;
static uint32_t rnd(void) {            /* xorshift64 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 32);
}
static float unif(void) { return (float)(rnd() >> 8) / 16777216.0f * 2.0f - 1.0f; }
static uint16_t bf16(float x) {        /* truncation is enough for test data */
    uint32_t b;
    memcpy(&b, &x, 4);
    return (uint16_t)(b >> 16);
}

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                   \
        }                                                               \
    } while (0)

int main(void) {
    enum { T = 37, D = 256, E = 16, K = 4, I = 256, NG = 4, MG = 2 };
    const int64_t R = (int64_t)T * K + T;
    oracle_set_threads(2);
    CHECK(oracle_max_threads() >= 1);
    /* scalars and codec */
    for (int c = 0; c < 256; ++c) {
        double v = oracle_e4m3_decode((uint8_t)c);
        if (!isnan(v)) CHECK(oracle_e4m3_encode((float)v) == (uint8_t)c || v == 0.0);
    }
    float xs[1000], ys[1000];
    uint8_t cs[1000];
    for (int i = 0; i < 1000; ++i) xs[i] = unif() * 100.0f;
    oracle_sigmoid_spec_n(xs, 1000, ys);
    oracle_exp_spec_n(xs, 1000, ys);
    oracle_e4m3_encode_n(xs, 1000, cs);
    CHECK(oracle_sigmoid_spec(0.0f) == 0.5f && oracle_exp_spec(0.0f) == 1.0f);
    /* router, top-K (plain and group-limited), balance loss */
    uint16_t* u = malloc(sizeof(uint16_t) * T * D);
    uint16_t* e = malloc(sizeof(uint16_t) * E * D);
    float* uf = malloc(sizeof(float) * T * D);
    for (int i = 0; i < T * D; ++i) {
        u[i] = bf16(unif() * 2.0f);
        uint32_t b = (uint32_t)u[i] << 16;
        memcpy(&uf[i], &b, 4);
    }
    for (int i = 0; i < E * D; ++i) e[i] = bf16(unif() * 0.06f);
    float bias[E], s[T * E], gate[T * K];
    int32_t idx[T * K];
    for (int i = 0; i < E; ++i) bias[i] = unif() * 0.05f;
    oracle_router_scores(u, e, T, D, E, s);
    oracle_topk_grouped_from_scores(s, bias, T, E, K, NG, MG, idx, gate);
    oracle_topk_from_scores(s, bias, T, E, K, idx, gate);
    for (int t = 0; t < T; ++t) {
        float g = 0.0f;
        for (int k = 0; k < K; ++k) g += gate[t * K + k];
        CHECK(fabsf(g - 1.0f) < 1e-5f);
    }
    double loss[1];
    oracle_seq_balance_loss(s, idx, T, E, K, T, 1e-4, loss);
    CHECK(loss[0] > 0.0);
    /* dispatch */
    int32_t count[E], go[E + 2], *row_token = malloc(sizeof(int32_t) * R), slot_row[T * K];
    CHECK(oracle_dispatch(idx, T, K, E, 1, count, go, row_token, slot_row) == 0);
    int64_t total = 0;
    for (int i = 0; i < E; ++i) total += count[i];
    CHECK(total == (int64_t)T * K && go[E] == T * K && go[E + 1] == R);
    /* quantisers, GEMMs, SwiGLU, combine, bias update */
    uint8_t* uq = malloc((size_t)T * D);
    float* us = malloc(sizeof(float) * T * (D / 128));
    oracle_quant_1x128(uf, T, D, uq, us);
    float* w = malloc(sizeof(float) * 2 * I * D);
    uint8_t* wq = malloc((size_t)2 * I * D);
    float* ws = malloc(sizeof(float) * (2 * I / 128) * (D / 128));
    for (int i = 0; i < 2 * I * D; ++i) w[i] = unif() * 0.06f;
    oracle_quant_128x128(w, 2 * I, D, wq, ws);
    const int64_t rows = go[1] - go[0];
    double* z = malloc(sizeof(double) * (rows + 1) * 2 * I);
    oracle_gemm_blockscaled(uq, us, row_token + go[0], rows, wq, ws, 2 * I, D, z);
    double* h = malloc(sizeof(double) * (rows + 1) * I);
    double* zg = malloc(sizeof(double) * (rows + 1) * I);
    double* zu = malloc(sizeof(double) * (rows + 1) * I);
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < I; ++c) {
            zg[r * I + c] = z[r * 2 * I + c];
            zu[r * I + c] = z[r * 2 * I + I + c];
        }
    oracle_swiglu(zg, zu, rows * I, h);
    double* y = calloc((size_t)R * D, sizeof(double));
    double* out = malloc(sizeof(double) * T * D);
    oracle_combine(u, y, (int64_t)T * K, gate, slot_row, T, K, D, out);
    for (int i = 0; i < T * D; ++i) CHECK(out[i] == (double)uf[i]);     /* zero FFN outputs give u */
    oracle_bias_update(bias, count, E, (int64_t)T * K, 1e-3f);
    free(u); free(e); free(uf); free(row_token); free(uq); free(us); free(w); free(wq); free(ws);
    free(z); free(h); free(zg); free(zu); free(y); free(out);
    printf("oracle driver: clean\n");
    return 0;
}
