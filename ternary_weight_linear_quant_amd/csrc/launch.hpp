// Host-side launch entry points of the kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, uint32_t* packed,
                                   float* gamma, double* rowsums, hipStream_t stream);

hipError_t launch_quantize_acts(const uint16_t* x, int64_t M, int64_t K, const uint16_t* gain,
                                float rms_eps, int8_t* xq, float* scale, hipStream_t stream);

// Decode GEMV (M <= 16, x held in LDS). Returns hipErrorInvalidValue if the
// shape does not fit the kernel.
bool gemv_supported(int64_t M, int64_t K);
hipError_t launch_gemv(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                       const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream);

// Decode for one token: each wave streams whole rows as 1 KB contiguous
// pieces (K up to 65536). Returns hipErrorInvalidValue otherwise.
bool gemv1_supported(int64_t M, int64_t K);
bool gemv1_preferred(int64_t M, int64_t K);
hipError_t launch_gemv1(const int8_t* xq, const float* xs, int K, const uint32_t* Wp,
                        const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream);
// One token quantised in the GEMV's own launch (gain: RMSNorm gain or null):
// the codes and scale go to xq_out / xs_out as well.
bool gemv1_quant_supported(int64_t M, int64_t K, bool norm);
hipError_t launch_gemv1_quant(const uint16_t* x, const uint16_t* gain, float rms_eps, int K,
                              const uint32_t* Wp, const float* gamma, int N, float* y,
                              int8_t* xq_out, float* xs_out, hipStream_t stream);

// Split K: int32 zeros into y, and y[m][n] = acc * (x_scale[m] * gamma) in
// place afterwards (acc, if not null, receives the sums).
hipError_t launch_splitk_zero(int32_t* y, size_t total, hipStream_t stream);
hipError_t launch_splitk_finalize(float* y, const float* xs, const float* gamma, int32_t* acc,
                                  int N, size_t total, hipStream_t stream);

// Decode for 17..64 tokens: 128 weight rows per workgroup, the activations
// staged in 512-wide K blocks.
bool gemv_wide_supported(int64_t M, int64_t K);
bool gemv_wide_preferred(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_wide(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                            const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream);

// Prefill GEMM (any M).
hipError_t launch_gemm(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                       const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream);

// Gating of a gated FFN (kind kGluRelu2 or kGluSwiglu): h = bf16(act(g) * u).
hipError_t launch_glu(const float* g, const float* u, int64_t count, int kind, uint16_t* h,
                      hipStream_t stream);

// The gating fused with the per-token quantisation of its output. gain (bf16 [K]) may be null; otherwise the sub-layer RMSNorm precedes the
// quantisation.
hipError_t launch_glu_quant(const float* gate, const float* up, int64_t M, int64_t K, int kind,
                            const uint16_t* gain, float rms_eps, int8_t* hq, float* scale,
                            hipStream_t stream);

// Two decode GEMVs sharing one quantised input, in one launch.
hipError_t launch_gemv_pair(const int8_t* xq, const float* xs, int M, int K, const uint32_t* W1,
                            const float* g1, int N1, float* y1, const uint32_t* W2,
                            const float* g2, int N2, float* y2, hipStream_t stream);

// Two-launch decode FFN (act quant + gate/up + squared-ReLU gating, then act
// quant + down), bit-identical to the unfused sequence.
bool ffn_fused_supported(int64_t M, int64_t K, int64_t N_ff, bool subln);
hipError_t launch_ffn_fused(const uint16_t* x, int M, int K, const uint32_t* Wg,
                            const float* gg, const uint32_t* Wu, const float* gu, int N_ff,
                            const uint32_t* Wd, const float* gd, uint16_t* h, float* y,
                            int kind, const uint16_t* subln_gain, float subln_eps,
                            hipStream_t stream);

// Launch A of the above alone: act quant + gate/up + gating into h (bf16).
bool ffn_gate_up_supported(int64_t M, int64_t K, int64_t N_ff);
hipError_t launch_ffn_gate_up(const uint16_t* x, int M, int K, const uint32_t* Wg,
                              const float* gg, const uint32_t* Wu, const float* gu, int N_ff,
                              uint16_t* h, int kind, hipStream_t stream);

// Other weight formats (decode GEMV only): 1 bit per {-1, +1} weight and
// five ternary weights per byte.
int64_t packed_row_bytes_binary(int64_t K);
int64_t packed_row_bytes_base3(int64_t K);
bool gemv_binary_supported(int64_t M, int64_t K);
bool gemv_base3_supported(int64_t M, int64_t K);
hipError_t launch_quantize_weights_binary(const float* W, int64_t N, int64_t K, uint32_t* packed,
                                          int64_t row_words, float* gamma, double* rowsums,
                                          hipStream_t stream);
hipError_t launch_pack_base3(const uint32_t* packed2, int64_t N, int64_t K, uint8_t* out,
                             int64_t row_bytes, hipStream_t stream);
hipError_t launch_gemv_binary(const int8_t* xq, const float* xs, int M, int K,
                              const uint32_t* Wb, const float* gamma, int N, float* y,
                              int32_t* acc, hipStream_t stream);
hipError_t launch_gemv_base3(const int8_t* xq, const float* xs, int M, int K, const uint8_t* W3,
                             const float* gamma, int N, float* y, int32_t* acc,
                             hipStream_t stream);

// Straight-through backward with respect to the input: transposed codes and
// dx = gamma * dy . q (bf16 matrix cores).
int64_t ste_t_row_bytes(int64_t N);
hipError_t launch_pack_ste_t(const uint32_t* packed2, int64_t N, int64_t K, uint8_t* qT,
                             hipStream_t stream);
hipError_t launch_ste_dx(const uint16_t* dy, int M, int N, const uint8_t* qT, const float* gamma,
                         int K, float* dx, hipStream_t stream);

// Straight-through backward with respect to the latent weights: dW = dy^T .
// (x_q * x_scale), bf16 matrix cores on split operands; workspace for the
// transposed operands.
int64_t ste_dw_padded_tokens(int64_t M);
size_t ste_dw_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_ste_dw(const uint16_t* dy, int M, int N, const int8_t* xq, const float* xs,
                         int K, float* dW, void* workspace, hipStream_t stream);

// Calibration kernels (measured ceilings; not part of the method).
constexpr int kCalibMfmaBlocks = 512;        // 256-thread blocks of the MFMA loop
hipError_t launch_calib_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_calib_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_calib_mfma(int iters, int32_t* sink, hipStream_t stream);
int64_t calib_mfma_ops(int64_t iters);

}  // namespace bl
