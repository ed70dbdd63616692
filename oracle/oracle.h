/*
 * CPU oracle for the BitNet b1.58 BitLinear forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, single-threaded reference
 * that the GPU library is checked against. Only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it; the product library
 * never calls, links or includes anything here, and nothing here is shared with
 * the GPU path (no common headers, tables or helpers).
 *
 * Sources (the pages give prose only, no formulas or listings):
 *   [P1] comrad404.com, "BitNet b1.58: что показала работа Microsoft об «эре
 *        1-битных LLM»", section «Метод: как устроен BitNet b1.58»: ternary
 *        {-1,0,1} weights by absmean quantisation, 8-bit activations,
 *        RMSNorm, no biases, and the four-step forward (normalise, quantise
 *        activations, ternary weights, low-bit matmul then rescale).
 *   [P3a] inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
 *        "„Trenowany od zera” — i czemu to nie jest zwykła kwantyzacja":
 *        the whole weight matrix is scaled by its mean absolute value, then
 *        every entry goes to the nearest integer in {-1,0,+1}.
 *   [P3b] same page, section "Skąd te 1,58 bita": log2(3) is the information
 *        bound; practical storage puts a ternary value in two bits.
 *   [P3c] same page, section "Mnożenie? Jakie mnożenie": times +1 is an add,
 *        times -1 a subtract, times 0 is skipped.
 *   [P3d] same page, section "Dlaczego akurat ternarne, a nie czyste
 *        zero-jeden" (the paragraph after the 1.58-bit count): the original
 *        BitNet used binary weights, only -1 and +1.
 *   [P5b] juhe.plus (Habr repost), the section on training that follows
 *        BinaryConnect: sign() has no useful derivative, so the forward
 *        uses the rounding and the backward passes the gradient straight
 *        through as if there were none (straight-through estimator).
 *   [P5] juhe.plus (Habr repost), section «Когда - три лучше двух»: with
 *        ternary weights y = W·x reduces to sums of the inputs where the
 *        weight is +1 minus sums where it is -1.
 *
 * Readings where the pages are silent (all shared with the GPU library by
 * specification, never by code):
 *   - weight epsilon 1e-5: s = gamma + 1e-5f (fp32 add); rescale uses gamma.
 *   - gamma = (float)(S / (N*K)) with S an fp64 sum: per-row sums in
 *     increasing k, then the row sums in increasing n.
 *   - rounding to nearest uses ties-to-even, on an fp32 correctly rounded
 *     quotient / product.
 *   - activations: per token absmax into [-127, 127]; absmax floored at 1e-5;
 *     the returned scale is the dequantisation multiplier (x ~ x_q * scale).
 *   - fused RMSNorm: codes of RMSNorm(x) are taken as the codes of x*g (a
 *     positive per-token factor cancels in absmax quantisation); the scale
 *     carries 1/rms with rms = sqrt(mean(x^2) + eps) in fp64.
 *   - 2-bit packing: c = q + 1 in {0,1,2}; row n is K/16 little-endian uint32
 *     words; weight k sits in word k/16 at bits 8*(i%4) + 2*(i/4), i = k%16.
 *   - epilogue y = acc * scale * gamma evaluated in fp64, rounded to fp32.
 *   - FFN glue h = bf16_rne((relu(g)*relu(g)) * u) in fp32.
 *   - binary weights: q = +1 where W >= 0, else -1, with the same absmean
 *     gamma; 1 bit per weight (word k/32, bit 8*(i%4) + i/4), rows padded to
 *     16 bytes with 0 bits.
 *   - 1.6-bit storage: five weights per byte as a base-3 number, least
 *     significant digit first (c = q + 1), rows padded to 16 bytes with 121.
 *   - straight-through backward: dx = gamma * dy . q with dy in bf16, the
 *     sum exact in fp64, rounded once to fp32; the transposed codes are
 *     stored four per byte along n, rows padded to 16 bytes with 0x55. The
 *     latent weights' gradient is dW = dy^T . x~ with x~ = x_q * s_x, the
 *     dequantised activations the forward multiplied (fp64, one rounding).
 */
#ifndef BITLINEAR_ORACLE_H
#define BITLINEAR_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* "oracle-source-sha256:" followed by the SHA-256 (hex) of oracle.c, oracle.h
 * and the compile flags this copy was built from. */
extern const char* oracle_source_sha256;

/* Per-row sums R[n] = sum_k |W[n][k]| in fp64, k increasing. W fp32 [N][K]. */
void oracle_absmean_rowsums(const float* W, int64_t N, int64_t K, double* R);

/* gamma = (float)((sum_n R[n], n increasing, fp64) / (N*K)).  [P3a] */
float oracle_absmean_gamma(const float* W, int64_t N, int64_t K);

/* q[n][k] = clamp(rne(W[n][k] / (gamma + eps)), -1, 1) as int8.  [P3a] */
void oracle_ternarize(const float* W, int64_t N, int64_t K, float gamma,
                      float eps, int8_t* q);

/* 2-bit packing of ternary codes, K % 16 == 0.  [P3b] */
void oracle_pack(const int8_t* q, int64_t N, int64_t K, uint32_t* packed);
void oracle_unpack(const uint32_t* packed, int64_t N, int64_t K, int8_t* q);

/* Per-token absmax int8 quantisation of bf16 x [M][K] (raw bits).
 * gain == NULL: plain; else fused RMSNorm with gain bf16 [K] and rms_eps.
 * Writes x_q int8 [M][K] and scale fp32 [M]. Optional rms_out fp64 [M]
 * (fused only; may be NULL).  [P1] */
void oracle_act_quant(const uint16_t* x, int64_t M, int64_t K,
                      const uint16_t* gain, float rms_eps,
                      int8_t* x_q, float* scale, double* rms_out);

/* acc[m][n] = sum_k x_q[m][k] * q[n][k] in int32.  [P3c], [P5] */
void oracle_int_matmul(const int8_t* x_q, int64_t M, int64_t K,
                       const int8_t* q, int64_t N, int32_t* acc);

/* Same sum written the pages' way: inputs where q=+1 added, where q=-1
 * subtracted, zeros skipped.  [P3c], [P5] */
void oracle_addsub_matmul(const int8_t* x_q, int64_t M, int64_t K,
                          const int8_t* q, int64_t N, int32_t* acc);

/* y[m][n] = (float)((double)acc * (double)scale[m] * (double)gamma).  [P1] */
void oracle_epilogue(const int32_t* acc, int64_t M, int64_t N,
                     const float* scale, float gamma, float* y);

/* h = bf16_rne((r*r)*u), r = g > 0 ? g : 0, fp32 arithmetic. */
void oracle_relu2_glu(const float* g, const float* u, int64_t count,
                      uint16_t* h);

/* h = bf16_rne(fp32(silu(g)) * u), silu(g) = g / (1 + exp(-g)) in fp64
 * (SwiGLU, comrad404.com «Метод: как устроен BitNet b1.58»: the b1.58
 * variant keeps the LLaMA stack's SwiGLU). */
void oracle_swiglu(const float* g, const float* u, int64_t count, uint16_t* h);

/* Binary codes q = (W >= 0) ? +1 : -1.  [P3d] */
void oracle_binarize(const float* W, int64_t N, int64_t K, int8_t* q);
/* 1-bit packing of codes in {-1, +1}; rows of row_words words.  [P3d] */
void oracle_pack_binary(const int8_t* q, int64_t N, int64_t K, int64_t row_words,
                        uint32_t* packed);
void oracle_unpack_binary(const uint32_t* packed, int64_t N, int64_t K, int64_t row_words,
                          int8_t* q);
/* Base-3 packing, five ternary codes per byte; rows of row_bytes bytes. [P3b] */
void oracle_pack_base3(const int8_t* q, int64_t N, int64_t K, int64_t row_bytes,
                       uint8_t* packed);
void oracle_unpack_base3(const uint8_t* packed, int64_t N, int64_t K, int64_t row_bytes,
                         int8_t* q);

/* Transposed 2-bit codes for the backward pass, four n per byte.  [P5b] */
void oracle_pack_ste_t(const int8_t* q, int64_t N, int64_t K, int64_t row_bytes,
                       uint8_t* qT);
/* dx = gamma * dy . q, dy bf16 [M][N], q [N][K], fp64 sum, one rounding. [P5b] */
void oracle_ste_dx(const uint16_t* dy, int64_t M, int64_t N, const int8_t* q, int64_t K,
                   float gamma, float* dx);
/* dW[n][k] = sum_m dy[m][n] * x_q[m][k] * x_scale[m]: the straight-through
 * gradient of the latent weights, dy bf16 [M][N], x_q int8 [M][K], x_scale
 * fp32 [M], dW fp32 [N][K]; exact fp64 products, fp64 sum over m, one
 * rounding. [P5b] */
void oracle_ste_dw(const uint16_t* dy, int64_t M, int64_t N, const int8_t* x_q,
                   const float* x_scale, int64_t K, float* dW);

#ifdef __cplusplus
}
#endif
#endif
