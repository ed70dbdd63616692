/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every function on small ragged inputs (single rows and columns, the
 * smallest K, padded rows of the other formats, the extremes of int8), with
 * a few results checked by hand. Exit 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) {
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state >> 8;
}
static float rndf(void) { return ((float)(rnd() % 20001) - 10000.0f) / 10000.0f; }
static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void run_shape(int64_t M, int64_t N, int64_t K) {
    float* W = malloc(sizeof(float) * N * K);
    int8_t* q = malloc(N * K);
    int8_t* q2 = malloc(N * K);
    uint32_t* packed = malloc(sizeof(uint32_t) * N * (K / 16));
    uint16_t* x = malloc(sizeof(uint16_t) * M * K);
    uint16_t* gain = malloc(sizeof(uint16_t) * K);
    int8_t* xq = malloc(M * K);
    float* sc = malloc(sizeof(float) * M);
    double* rms = malloc(sizeof(double) * M);
    int32_t* acc = malloc(sizeof(int32_t) * M * N);
    int32_t* acc2 = malloc(sizeof(int32_t) * M * N);
    float* y = malloc(sizeof(float) * M * N);
    double* R = malloc(sizeof(double) * N);
    for (int64_t i = 0; i < N * K; ++i) W[i] = 0.02f * rndf();
    for (int64_t i = 0; i < M * K; ++i) x[i] = bf16(rndf() * (i % 7 == 0 ? 20.0f : 1.0f));
    for (int64_t k = 0; k < K; ++k) gain[k] = bf16(1.0f + 0.1f * rndf());

    oracle_absmean_rowsums(W, N, K, R);
    const float gamma = oracle_absmean_gamma(W, N, K);
    oracle_ternarize(W, N, K, gamma, 1e-5f, q);
    oracle_pack(q, N, K, packed);
    oracle_unpack(packed, N, K, q2);
    CHECK(memcmp(q, q2, N * K) == 0);
    oracle_act_quant(x, M, K, NULL, 1e-5f, xq, sc, NULL);
    oracle_act_quant(x, M, K, gain, 1e-5f, xq, sc, rms);
    oracle_int_matmul(xq, M, K, q, N, acc);
    oracle_addsub_matmul(xq, M, K, q, N, acc2);
    CHECK(memcmp(acc, acc2, sizeof(int32_t) * M * N) == 0);
    oracle_epilogue(acc, M, N, sc, gamma, y);

    float* gt = malloc(sizeof(float) * M * N);
    float* up = malloc(sizeof(float) * M * N);
    uint16_t* hh = malloc(sizeof(uint16_t) * M * N);
    for (int64_t i = 0; i < M * N; ++i) {
        gt[i] = rndf() * 3.0f;
        up[i] = rndf();
    }
    gt[0] = -800.0f; /* exp overflow path of SiLU */
    oracle_relu2_glu(gt, up, M * N, hh);
    oracle_swiglu(gt, up, M * N, hh);

    const int64_t rw = 4 * ((K + 127) / 128), rb3 = 16 * (((K + 4) / 5 + 15) / 16);
    uint32_t* pb = malloc(sizeof(uint32_t) * N * rw);
    uint8_t* p3 = malloc(N * rb3);
    oracle_binarize(W, N, K, q2);
    oracle_pack_binary(q2, N, K, rw, pb);
    oracle_unpack_binary(pb, N, K, rw, q2);
    oracle_pack_base3(q, N, K, rb3, p3);
    oracle_unpack_base3(p3, N, K, rb3, q2);
    CHECK(memcmp(q, q2, N * K) == 0);

    const int64_t rbt = 16 * (((N + 3) / 4 + 15) / 16);
    uint8_t* qT = malloc(K * rbt);
    oracle_pack_ste_t(q, N, K, rbt, qT);
    uint16_t* dy = malloc(sizeof(uint16_t) * M * N);
    for (int64_t i = 0; i < M * N; ++i) dy[i] = bf16(rndf());
    float* dx = malloc(sizeof(float) * M * K);
    float* dW = malloc(sizeof(float) * N * K);
    oracle_ste_dx(dy, M, N, q, K, gamma, dx);
    for (int64_t i = 0; i < M * K; ++i) xq[i] = (int8_t)((int)(rnd() % 256) - 128);
    oracle_ste_dw(dy, M, N, xq, sc, K, dW);

    free(W); free(q); free(q2); free(packed); free(x); free(gain); free(xq); free(sc); free(rms);
    free(acc); free(acc2); free(y); free(R); free(gt); free(up); free(hh); free(pb); free(p3);
    free(qT); free(dy); free(dx); free(dW);
}

int main(void) {
    /* Hand values: the act quant of the tie token (codes 62, 0, 2, 2, -2). */
    uint16_t tok[16] = {0};
    const float vals[6] = {127.0f, 62.5f, 0.5f, 1.5f, 2.5f, -2.5f};
    for (int i = 0; i < 6; ++i) tok[i] = bf16(vals[i]);
    int8_t codes[16];
    float s;
    oracle_act_quant(tok, 1, 16, NULL, 1e-5f, codes, &s, NULL);
    CHECK(codes[0] == 127 && codes[1] == 62 && codes[2] == 0 && codes[3] == 2 &&
          codes[4] == 2 && codes[5] == -2 && s == 1.0f);
    /* Extremes: int8 -128 and +127 in the product. */
    int8_t xa[16], qa[16];
    int32_t a;
    for (int i = 0; i < 16; ++i) {
        xa[i] = (i % 2) ? -128 : 127;
        qa[i] = (int8_t)((i % 3) - 1);
    }
    oracle_int_matmul(xa, 1, 16, qa, 1, &a);
    int32_t want = 0;
    for (int i = 0; i < 16; ++i) want += xa[i] * qa[i];
    CHECK(a == want);

    const int64_t shapes[][3] = {{1, 1, 16}, {3, 5, 64}, {2, 17, 80}, {7, 3, 128}, {1, 33, 320}};
    for (unsigned i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        run_shape(shapes[i][0], shapes[i][1], shapes[i][2]);
    if (failures) return 1;
    puts("oracle sanitizer checks: ok");
    return 0;
}
