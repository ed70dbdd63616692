/*
 * CPU oracle for the BitNet b1.58 BitLinear forward pass.
 * TEST INFRASTRUCTURE ONLY -- see oracle.h for the sources and the readings.
 *
 * Plain single-threaded C11, built with -O3 -ffp-contract=off and without
 * -ffast-math, so every fp32 operation below is one IEEE-754 round-to-nearest
 * operation in the order written (no contraction; without -ffast-math the
 * compiler may not reassociate floating-point sums). nearbyintf runs under
 * the default FE_TONEAREST mode, i.e. ties go to the even integer.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

#ifndef ORACLE_SOURCE_SHA256
#define ORACLE_SOURCE_SHA256 "unknown"
#endif
/* Digest of the sources and flags this copy was built from, behind a marker
 * that a loader can find in the file's bytes. */
const char* oracle_source_sha256 = "oracle-source-sha256:" ORACLE_SOURCE_SHA256;

static float bf16_bits_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round an fp32 value to bf16 bits, nearest with ties to even (finite input). */
static uint16_t float_to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Mean absolute value of the whole matrix [P3a]: fp64 row sums in order. */
void oracle_absmean_rowsums(const float* W, int64_t N, int64_t K, double* R) {
    for (int64_t n = 0; n < N; ++n) {
        const float* row = W + n * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += (double)fabsf(row[k]);
        R[n] = s;
    }
}

float oracle_absmean_gamma(const float* W, int64_t N, int64_t K) {
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const float* row = W + n * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += (double)fabsf(row[k]);
        total += s;
    }
    return (float)(total / (double)(N * K));
}

/* Scale by the (eps-guarded) mean, take the nearest integer, clip to
 * {-1, 0, +1} [P3a]. */
void oracle_ternarize(const float* W, int64_t N, int64_t K, float gamma,
                      float eps, int8_t* q) {
    const float s = gamma + eps;
    for (int64_t i = 0; i < N * K; ++i) {
        float r = W[i] / s;
        float t = nearbyintf(r);
        if (t > 1.0f) t = 1.0f;
        if (t < -1.0f) t = -1.0f;
        q[i] = (int8_t)t;
    }
}

/* Two bits per ternary weight [P3b]: code c = q + 1. */
void oracle_pack(const int8_t* q, int64_t N, int64_t K, uint32_t* packed) {
    const int64_t words = K / 16;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < words; ++j) {
            uint32_t w = 0;
            for (int i = 0; i < 16; ++i) {
                uint32_t c = (uint32_t)(q[n * K + 16 * j + i] + 1);
                int shift = 8 * (i % 4) + 2 * (i / 4);
                w |= c << shift;
            }
            packed[n * words + j] = w;
        }
    }
}

void oracle_unpack(const uint32_t* packed, int64_t N, int64_t K, int8_t* q) {
    const int64_t words = K / 16;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < words; ++j) {
            uint32_t w = packed[n * words + j];
            for (int i = 0; i < 16; ++i) {
                int shift = 8 * (i % 4) + 2 * (i / 4);
                q[n * K + 16 * j + i] = (int8_t)((int)((w >> shift) & 3u) - 1);
            }
        }
    }
}

/* Binary weights, the original BitNet's {-1, +1} [P3d]: sign of the latent
 * weight, with W >= 0 (both zeros included) giving +1. */
void oracle_binarize(const float* W, int64_t N, int64_t K, int8_t* q) {
    for (int64_t i = 0; i < N * K; ++i) q[i] = (int8_t)(W[i] >= 0.0f ? 1 : -1);
}

/* One bit per weight: bit 1 for +1, 0 for -1. Row n is row_words uint32
 * words; weight k sits in word k/32 at bit 8*(i%4) + i/4, i = k%32. Bits at
 * k >= K are 0. */
void oracle_pack_binary(const int8_t* q, int64_t N, int64_t K, int64_t row_words,
                        uint32_t* packed) {
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < row_words; ++j) {
            uint32_t w = 0;
            for (int i = 0; i < 32; ++i) {
                int64_t k = 32 * j + i;
                if (k < K && q[n * K + k] > 0) w |= 1u << (8 * (i % 4) + i / 4);
            }
            packed[n * row_words + j] = w;
        }
    }
}

void oracle_unpack_binary(const uint32_t* packed, int64_t N, int64_t K, int64_t row_words,
                          int8_t* q) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int i = (int)(k % 32);
            uint32_t bit = (packed[n * row_words + k / 32] >> (8 * (i % 4) + i / 4)) & 1u;
            q[n * K + k] = (int8_t)(bit ? 1 : -1);
        }
}

/* Five ternary weights per byte, near the log2(3) bound [P3b]: byte j of row
 * n is the base-3 number sum_{i<5} c_i * 3^i with c_i = q[n][5j+i] + 1 (the
 * least significant digit first); positions k >= K count as weight 0 (c = 1).
 * A row is row_bytes bytes; bytes past ceil(K/5) are 121 (five zeros). */
void oracle_pack_base3(const int8_t* q, int64_t N, int64_t K, int64_t row_bytes,
                       uint8_t* packed) {
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < row_bytes; ++j) {
            int v = 0, p3 = 1;
            for (int i = 0; i < 5; ++i) {
                int64_t k = 5 * j + i;
                int c = k < K ? q[n * K + k] + 1 : 1;
                v += c * p3;
                p3 *= 3;
            }
            packed[n * row_bytes + j] = (uint8_t)v;
        }
    }
}

void oracle_unpack_base3(const uint8_t* packed, int64_t N, int64_t K, int64_t row_bytes,
                         int8_t* q) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; 5 * j < K; ++j) {
            int v = packed[n * row_bytes + j];
            for (int i = 0; i < 5 && 5 * j + i < K; ++i) {
                q[n * K + 5 * j + i] = (int8_t)(v % 3 - 1);
                v /= 3;
            }
        }
}

/* Backward-layout packing of the ternary codes for the straight-through
 * estimator [P5b]: row k of qT holds q[n][k] for n = 0..N-1, four codes per
 * byte, code c = q + 1 of n = 4j + i at bits 2i of byte j; positions n >= N
 * are code 1 (weight 0). Rows are row_bytes bytes (padding bytes 0x55). */
void oracle_pack_ste_t(const int8_t* q, int64_t N, int64_t K, int64_t row_bytes,
                       uint8_t* qT) {
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < row_bytes; ++j) {
            unsigned v = 0;
            for (int i = 0; i < 4; ++i) {
                int64_t n = 4 * j + i;
                unsigned c = n < N ? (unsigned)(q[n * K + k] + 1) : 1u;
                v |= c << (2 * i);
            }
            qT[k * row_bytes + j] = (uint8_t)v;
        }
}

/* Straight-through estimator, gradient with respect to the layer input
 * [P5b]: the forward's rounding is treated as the identity, so
 * dx[m][k] = gamma * sum_n dy[m][n] * q[n][k] (the transpose of the ternary
 * product, rescaled by the weight scale). dy is bf16 [M][N]; the sum is taken
 * in fp64 with n increasing, multiplied by gamma in fp64 and rounded once to
 * fp32. */
void oracle_ste_dx(const uint16_t* dy, int64_t M, int64_t N, const int8_t* q, int64_t K,
                   float gamma, float* dx) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                int8_t w = q[n * K + k];
                if (w) s += (double)w * (double)bf16_bits_to_float(dy[m * N + n]);
            }
            dx[m * K + k] = (float)(s * (double)gamma);
        }
}

/* Straight-through estimator, gradient with respect to the latent weights
 * [P5b]: the forward multiplies the dequantised activations x~ = x_q * s_x by
 * the weights, and the backward treats the weights' rounding as the
 * identity, so dW[n][k] = sum_m dy[m][n] * x_q[m][k] * s_x[m]. Each product
 * is exact in fp64 (8 + 24 + 8 significant bits); the sum is taken in fp64
 * with m increasing and rounded once to fp32. */
void oracle_ste_dw(const uint16_t* dy, int64_t M, int64_t N, const int8_t* x_q,
                   const float* x_scale, int64_t K, float* dW) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                int8_t x = x_q[m * K + k];
                if (x)
                    s += (double)bf16_bits_to_float(dy[m * N + n]) * (double)x_scale[m] *
                         (double)x;
            }
            dW[n * K + k] = (float)s;
        }
}

/* 8-bit activations [P1], per token by absmax into [-127, 127]. */
void oracle_act_quant(const uint16_t* x, int64_t M, int64_t K,
                      const uint16_t* gain, float rms_eps,
                      int8_t* x_q, float* scale, double* rms_out) {
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * K;
        /* z = x * g is exact in fp32: two 8-bit significands. */
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float z = bf16_bits_to_float(row[k]);
            if (gain) z = z * bf16_bits_to_float(gain[k]);
            float mag = fabsf(z);
            if (mag > a) a = mag;
        }
        if (!(a > 1e-5f)) a = 1e-5f;
        const float inv = 127.0f / a;
        for (int64_t k = 0; k < K; ++k) {
            float z = bf16_bits_to_float(row[k]);
            if (gain) z = z * bf16_bits_to_float(gain[k]);
            float t = nearbyintf(z * inv);
            if (t > 127.0f) t = 127.0f;
            if (t < -127.0f) t = -127.0f;
            x_q[m * K + k] = (int8_t)t;
        }
        if (gain) {
            /* RMSNorm [P1]: rms = sqrt(mean(x^2) + eps); the normalised
             * token's absmax is a / rms. */
            double ss = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double v = (double)bf16_bits_to_float(row[k]);
                ss += v * v;
            }
            double rms = sqrt(ss / (double)K + (double)rms_eps);
            scale[m] = (float)((double)a / (127.0 * rms));
            if (rms_out) rms_out[m] = rms;
        } else {
            scale[m] = a / 127.0f;
        }
    }
}

/* Integer product of int8 activations and ternary weights [P3c], [P5]. */
void oracle_int_matmul(const int8_t* x_q, int64_t M, int64_t K,
                       const int8_t* q, int64_t N, int32_t* acc) {
    for (int64_t m = 0; m < M; ++m) {
        const int8_t* xr = x_q + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* wr = q + n * K;
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int32_t)xr[k] * (int32_t)wr[k];
            acc[m * N + n] = s;
        }
    }
}

void oracle_addsub_matmul(const int8_t* x_q, int64_t M, int64_t K,
                          const int8_t* q, int64_t N, int32_t* acc) {
    for (int64_t m = 0; m < M; ++m) {
        const int8_t* xr = x_q + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* wr = q + n * K;
            int32_t plus = 0, minus = 0;
            for (int64_t k = 0; k < K; ++k) {
                if (wr[k] == 1) plus += xr[k];
                else if (wr[k] == -1) minus += xr[k];
            }
            acc[m * N + n] = plus - minus;
        }
    }
}

/* Rescale of the integer result [P1]. */
void oracle_epilogue(const int32_t* acc, int64_t M, int64_t N,
                     const float* scale, float gamma, float* y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (float)((double)acc[m * N + n] * (double)scale[m] *
                                   (double)gamma);
}

void oracle_relu2_glu(const float* g, const float* u, int64_t count,
                      uint16_t* h) {
    for (int64_t i = 0; i < count; ++i) {
        float r = g[i] > 0.0f ? g[i] : 0.0f;
        float sq = r * r;
        h[i] = float_to_bf16_bits(sq * u[i]);
    }
}

/* SwiGLU gating: the SiLU (swish) of the gate, g * sigmoid(g), times up.
 * The SiLU is evaluated in fp64 from the definition and rounded once to
 * fp32; the product with up is one fp32 multiply, then bf16 rounding. */
void oracle_swiglu(const float* g, const float* u, int64_t count, uint16_t* h) {
    for (int64_t i = 0; i < count; ++i) {
        double gd = (double)g[i];
        float s = (float)(gd / (1.0 + exp(-gd)));
        h[i] = float_to_bf16_bits(s * u[i]);
    }
}
