/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear library.
 *
 * The library computes the BitLinear forward pass: latent weights are
 * quantised once to ternary codes {-1, 0, +1} with one scale per matrix and
 * stored at 2 bits per weight; activations are quantised per token to int8;
 * their product is accumulated exactly in int32 and rescaled to fp32.
 *
 * Sources (prose only; the pages print no formula or listing):
 *   comrad404.com, "BitNet b1.58: что показала работа Microsoft об «эре
 *     1-битных LLM»", section «Метод: как устроен BitNet b1.58» -- ternary
 *     weights via absmean quantisation, 8-bit activations, RMSNorm, no biases,
 *     and the forward order: normalise, quantise activations, ternary
 *     weights, low-bit matmul, rescale.
 *   inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów" -- section
 *     "„Trenowany od zera” — i czemu to nie jest zwykła kwantyzacja" (the whole
 *     matrix is scaled by its mean absolute value, entries go to the nearest
 *     of {-1, 0, +1}); section "Skąd te 1,58 bita" (two bits per stored
 *     ternary value); section "Mnożenie? Jakie mnożenie" (+1 adds, -1
 *     subtracts, 0 is skipped).
 *   juhe.plus (Habr repost), section «Когда - три лучше двух» -- y = W x as
 *     a sum over +1 weights minus a sum over -1 weights.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers (hipMalloc'd or equivalent) on
 *     the current HIP device; the caller owns all memory. The library never
 *     allocates, on the hot path or elsewhere, and keeps no state beyond a
 *     cached device count and, per device, which kernels have had their
 *     LDS limit raised (set on a kernel's first launch on that device).
 *     Calls may come from several host threads; bl_last_hip_error() is per
 *     thread.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on `stream` and never synchronises, so it
 *     may be captured into a HIP graph. Calls on different streams may run
 *     concurrently when their output buffers do not overlap.
 *   - Arguments are validated on the host before anything is enqueued. On any
 *     violation the call returns BL_ERR_INVALID_ARG and enqueues nothing.
 *     If no HIP device is visible the call returns BL_ERR_NO_DEVICE. A failed
 *     launch returns BL_ERR_HIP (bl_last_hip_error() gives the hipError_t).
 *     Before enqueuing, a call clears HIP's pending error of the calling
 *     thread (hipGetLastError), so BL_ERR_HIP always names this call's own
 *     failed launch; check your own launches before calling in. A call that
 *     returns BL_ERR_HIP leaves no pending HIP error behind.
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Shapes: M tokens, K input features, N output features; 1 <= M, N,
 *     64 <= K, K % 64 == 0, and M*K, N*K below 2^31. Base pointers of x,
 *     x_q, W and W_packed must be 16-byte aligned.
 *   - Inputs must be finite; non-finite values are outside the contract.
 *   - Every result is deterministic: the same inputs give the same bits.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    BL_OK = 0,
    BL_ERR_INVALID_ARG = 1,
    BL_ERR_HIP = 2,
    BL_ERR_NO_DEVICE = 3
};

/* Human-readable name of a status code (static string, never NULL). */
const char* bl_status_string(int status);

/* hipError_t of the most recent BL_ERR_HIP returned on this thread (0 if none). */
int bl_last_hip_error(void);

/* Library version string (static). */
const char* bl_version(void);

/* SHA-256 (hex) of the sources and compile flags this library was built from
 * (static string; "unknown" when built without it). The Python binding
 * refuses a library whose digest differs from its source tree's. */
const char* bl_source_sha256(void);

/* Bytes of the packed weight buffer: N*K/4 (2 bits per weight); 0 if the shape
 * is invalid. Host-only, no device needed. */
size_t bl_packed_bytes(int64_t N, int64_t K);

/* Bytes of the workspace bl_quantize_weights needs: 8*N (fp64 row sums);
 * 0 if the shape is invalid. Host-only. */
size_t bl_quantize_weights_workspace_bytes(int64_t N, int64_t K);

/* Absmean ternary weight quantisation and 2-bit packing (offline, once per
 * matrix). Source: inferownia.pl "BitNet b1.58: era 1-bitowych LLM-ów",
 * section "„Trenowany od zera”" (absmean, nearest of {-1,0,+1}) and section
 * "Skąd te 1,58 bita" (two bits per weight).
 *
 *   W          in   fp32 [N][K] row-major (out_features x in_features), latent
 *                   weights.
 *   W_packed   out  uint32 [N][K/16] (bl_packed_bytes(N,K) bytes). Code
 *                   c = q + 1 in {0,1,2}; weight k of row n lives in word k/16
 *                   at bits 8*(i%4) + 2*(i/4), i = k % 16, so
 *                   (word >> 2p) & 0x03030303 holds the codes of weights
 *                   16j+4p .. 16j+4p+3 in bytes 0..3.
 *   gamma      out  one fp32 (device): gamma = (float)(S / (N*K)) where S sums,
 *                   in fp64, the per-row sums R_n = sum_k |W[n][k]| (each in
 *                   fp64, k increasing) in increasing n.
 *   workspace  tmp  >= bl_quantize_weights_workspace_bytes(N,K) bytes, 8-byte
 *                   aligned; contents undefined afterwards.
 * Codes: q = clamp(rne(W / (gamma + 1e-5f)), -1, 1), fp32 correctly rounded
 * division, ties to even. */
int bl_quantize_weights(const float* W, int64_t N, int64_t K,
                        uint32_t* W_packed, float* gamma,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Per-token absmax int8 activation quantisation, optionally fused with the
 * RMSNorm that precedes BitLinear. Source: comrad404.com page above, section
 * «Метод: как устроен BitNet b1.58» (8-bit activations; normalise, then
 * quantise).
 *
 *   x          in   bf16 [M][K] row-major, raw uint16 bits.
 *   rms_gain   in   NULL for plain quantisation, else bf16 [K] RMSNorm gain.
 *   rms_eps    in   RMSNorm epsilon (> 0 when rms_gain != NULL; else ignored).
 *   x_q        out  int8 [M][K].
 *   x_scale    out  fp32 [M], dequantisation multiplier (x ~ x_q * x_scale).
 * Per token m, with z_k = x_k (plain) or z_k = x_k * g_k (fused; exact in
 * fp32): a = max(max_k |z_k|, 1e-5f); x_q = clamp(rne(z_k * (127.0f / a)),
 * -127, 127) with fp32 correctly rounded quotient and product, ties to even.
 * Plain: x_scale = a / 127.0f. Fused: x_scale = (float)(a / (127 * rms)) with
 * rms = sqrt(sum_k x_k^2 / K + rms_eps) in fp64 (within 1e-6 relative of the
 * sequential-sum value; codes are exact). */
int bl_quantize_acts(const uint16_t* x, int64_t M, int64_t K,
                     const uint16_t* rms_gain, float rms_eps,
                     int8_t* x_q, float* x_scale, void* stream);

/* BitLinear product: y = (x_q . q^T) * x_scale * gamma, no bias.
 * Source: inferownia.pl page above, section "Mnożenie? Jakie mnożenie", and
 * juhe.plus section «Когда - три лучше двух» (ternary weights turn the product
 * into additions and subtractions); comrad404.com «Метод…» (rescale after the
 * low-bit matmul).
 *
 *   x_q, x_scale  in  int8 [M][K] and fp32 [M] from bl_quantize_acts.
 *   W_packed, gamma in packed weights [N][K/16] and fp32 gamma (device) from
 *                 bl_quantize_weights.
 *   y          out  fp32 [M][N] row-major: y[m][n] = (float)acc[m][n] *
 *                   (x_scale[m] * gamma) in fp32 (within 2.5e-7 relative of
 *                   the fp64-evaluated product).
 *   acc        out  optional int32 [M][N]: acc[m][n] = sum_k q[n][k]*x_q[m][k],
 *                   exact (|acc| <= 127*K). NULL to skip.
 * Small M runs a weight-streaming GEMV, large M an int8 MFMA GEMM; all give
 * identical bits. When the grid is small (few tokens or few output
 * features) the K dimension is split across workgroups: the call then
 * enqueues three kernels and y's memory holds int32 partial sums until the
 * last one has rescaled them, so y must not alias any input. */
int bl_bitlinear(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                 const uint32_t* W_packed, const float* gamma, int64_t N,
                 float* y, int32_t* acc, void* stream);

/* As bl_bitlinear with an explicit kernel choice, for testing and tuning:
 * path 0 = automatic, 1 = GEMV (requires M <= 16 and M*K <= 128 KiB),
 * 2 = GEMM, 3 = wide GEMV for up to 64 tokens (128 weight rows per
 * workgroup, activations staged in K blocks; requires M <= 64), 4 = one-token
 * GEMV (each wave streams whole rows as 1 KB contiguous pieces; requires
 * M == 1 and K <= 65536). All give the same bits. Automatic: the one-token
 * GEMV at one token when K <= 8192 or K is a multiple of 4096, else the GEMV
 * when it applies, else the wide GEMV up to 64
 * tokens when each of its workgroups streams at least four K blocks of 512
 * and the matrix is not one where the GEMM measured faster (from 48 tokens
 * on matrices of at least 16 Mi weights, from 33 tokens on wide ones, N > K,
 * of at least 24 Mi), else the GEMM. Any other value, or an unsupported
 * choice, is BL_ERR_INVALID_ARG. */
int bl_bitlinear_path(const int8_t* x_q, const float* x_scale, int64_t M,
                      int64_t K, const uint32_t* W_packed, const float* gamma,
                      int64_t N, float* y, int32_t* acc, int path, void* stream);

/* The kernel bl_bitlinear_path(..., path, ...) runs for an M x K by N x K
 * product: 1..4 as above (path 0 resolved by the automatic rule), or -1 when
 * the shape or the choice is invalid. Host only, no device needed. */
int bl_bitlinear_choice(int64_t M, int64_t K, int64_t N, int path);

/* Activation quantisation (optionally fused with the preceding RMSNorm) and
 * the BitLinear product in one call: exactly bl_quantize_acts(x, M, K,
 * rms_gain, rms_eps, x_q, x_scale) followed by bl_bitlinear(x_q, x_scale, M,
 * K, W_packed, gamma, N, y, NULL). Source: comrad404.com page above, section
 * «Метод: как устроен BitNet b1.58»: normalise, quantise the activations to
 * 8 bits, multiply by the ternary weights, rescale.
 *
 *   x, rms_gain, rms_eps   in   as bl_quantize_acts.
 *   W_packed, gamma, N     in   as bl_bitlinear.
 *   y          out  fp32 [M][N], the same bits as the two calls give.
 *   x_q        out  int8 [M][K], x_scale out fp32 [M]: the quantised input,
 *                   the same bits as bl_quantize_acts gives (the caller
 *                   provides both; they are written whichever way the call
 *                   runs).
 * At one token (M == 1) a single launch does both when K <= 4096, or when K
 * is 8192, 12288, ..., 32768 (a multiple of 4096 up to eight times it) and
 * rms_gain is NULL: every workgroup of the one-token GEMV quantises the token
 * itself (its weight loads already in flight) and workgroup 0 writes x_q and
 * x_scale. Other shapes enqueue the two calls (rows with a partial second
 * piece: every workgroup's copy of the token costs more than the second
 * launch; longer rows with a gain: the fp64 sum of squares would be taken in
 * another order than bl_quantize_acts takes it). Pointers 16-byte aligned; y,
 * x_q and x_scale must not overlap each other or any input. */
int bl_quant_bitlinear(const uint16_t* x, int64_t M, int64_t K, const uint16_t* rms_gain,
                       float rms_eps, const uint32_t* W_packed, const float* gamma, int64_t N,
                       float* y, int8_t* x_q, float* x_scale, void* stream);

/* Squared-ReLU gating between the gate/up and down projections of a 2B4T-style
 * FFN: h[i] = bf16_rne((r*r) * up[i]) with r = gate[i] > 0 ? gate[i] : 0, all
 * fp32. Source: inferownia.pl page above, section "Zrób to sam — Microsoft
 * wypuścił konkretny model", and kripta.biz (2B4T article): the 2B4T FFN uses
 * squared ReLU. gate, up: fp32 [count]; h: bf16 bits [count]. count >= 1;
 * pointers 16-byte aligned. */
int bl_relu2_glu(const float* gate, const float* up, int64_t count,
                 uint16_t* h, void* stream);

/* Gating kinds of a gated FFN, h = bf16_rne(act(gate) * up) in fp32:
 *   BL_GLU_RELU2   act(g) = relu(g)^2 (the 2B4T FFN, as bl_relu2_glu);
 *   BL_GLU_SWIGLU  act(g) = SiLU(g) = g / (1 + exp(-g)) evaluated in fp64
 *                  (exp from the device math library, fp64 division) and
 *                  rounded once to fp32: the correctly rounded SiLU except
 *                  where the fp64 value lies within about 1e-16 relative of an
 *                  fp32 rounding boundary; a gate below about -709 gives -0.
 *                  Source: comrad404.com page above, section «Метод: как
 *                  устроен BitNet b1.58»: the b1.58 variant keeps the LLaMA
 *                  stack's SwiGLU. */
enum { BL_GLU_RELU2 = 0, BL_GLU_SWIGLU = 1 };

/* h[i] = bf16_rne(act(gate[i]) * up[i]) for glu_kind (above); arguments as
 * bl_relu2_glu; any other kind is BL_ERR_INVALID_ARG. */
int bl_glu(const float* gate, const float* up, int64_t count, int glu_kind, uint16_t* h,
           void* stream);

/* Two BitLinear products that share one quantised input -- the gate and up
 * projections of an FFN -- in a single launch: y1 = BitLinear(x_q, W1) and
 * y2 = BitLinear(x_q, W2), each exactly as bl_bitlinear computes it (same
 * bits). Same contract as bl_bitlinear per product (no acc output); N1 and N2
 * may differ. Source: comrad404.com page above, section «Метод: как устроен
 * BitNet b1.58» (the LLaMA-style block whose FFN projections are BitLinear),
 * and inferownia.pl page above, section "Mnożenie? Jakie mnożenie". */
int bl_bitlinear_pair(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                      const uint32_t* W1, const float* gamma1, int64_t N1, float* y1,
                      const uint32_t* W2, const float* gamma2, int64_t N2, float* y2,
                      void* stream);

/* Squared-ReLU gating fused with the per-token int8 quantisation of its
 * result: h = bf16_rne((relu(gate)^2) * up) as in bl_relu2_glu, then h_q /
 * h_scale exactly as bl_quantize_acts(h, rms_gain = NULL) computes them (same
 * bits), without writing h. gate, up: fp32 [M][K]; h_q: int8 [M][K]; h_scale:
 * fp32 [M]. Shape rules of bl_quantize_acts; pointers 16-byte aligned. Source:
 * inferownia.pl page above, section "Zrób to sam — Microsoft wypuścił
 * konkretny model" (squared ReLU) and comrad404.com «Метод…» (8-bit
 * activations). */
int bl_relu2_glu_quant(const float* gate, const float* up, int64_t M, int64_t K, int8_t* h_q,
                       float* h_scale, void* stream);

/* As bl_relu2_glu_quant with the sub-layer RMSNorm (subln) between the
 * gating and the quantisation: h_q / h_scale are exactly what
 * bl_quantize_acts(h, gain, rms_eps) computes from h = bf16_rne(relu(gate)^2
 * * up): the codes of z = h * gain (bit-exact), and h_scale = a / (127 *
 * rms) with rms = sqrt(sum h^2 / K + rms_eps), sum h^2 in fp64 in an order
 * of the kernel's choosing (h_scale within 1e-6 relative of any order).
 * gain: bf16 [K] (raw bits), 16-byte aligned, not null; rms_eps > 0.
 * Source: inferownia.pl page above, section "Zrób to sam — Microsoft
 * wypuścił konkretny model": the 2B4T model normalises with subln; the
 * norm's place (on the FFN's gated hidden state, before its quantisation for
 * the down projection) is this library's reading. */
int bl_relu2_glu_subln_quant(const float* gate, const float* up, int64_t M, int64_t K,
                             const uint16_t* gain, float rms_eps, int8_t* h_q, float* h_scale,
                             void* stream);

/* The gating of glu_kind fused with the per-token quantisation of its
 * result: h_q / h_scale exactly as bl_quantize_acts(bl_glu(gate, up, kind),
 * gain, rms_eps) computes them. gain may be null (no norm: every bit as the
 * two calls) or bf16 [K] (the sub-layer RMSNorm, rules of
 * bl_relu2_glu_subln_quant). Other arguments as bl_relu2_glu_quant. */
int bl_glu_quant(const float* gate, const float* up, int64_t M, int64_t K, int glu_kind,
                 const uint16_t* gain, float rms_eps, int8_t* h_q, float* h_scale, void* stream);

/* Bytes of the workspace bl_ffn_relu2 needs for these shapes (0 if the
 * shapes are invalid). Host-only. */
size_t bl_ffn_relu2_workspace_bytes(int64_t M, int64_t K, int64_t N_ff);

/* One FFN step of a 2B4T-style block (no residual, no norm):
 *   x_q, x_scale = quantize_acts(x)                 (plain, per token)
 *   h = bf16_rne(relu(BitLinear(x, W_gate))^2 * BitLinear(x, W_up))
 *   y = BitLinear(quantize_acts(h), W_down)
 * with every step exactly as the single calls compute it, so y has the bits
 * of bl_quantize_acts -> bl_bitlinear (gate, up) -> bl_relu2_glu ->
 * bl_quantize_acts -> bl_bitlinear (down). Source: inferownia.pl page above,
 * section "Zrób to sam — Microsoft wypuścił konkretny model" (2B4T, squared
 * ReLU) and section "Mnożenie? Jakie mnożenie"; comrad404.com «Метод…»
 * (8-bit activations before each low-bit product).
 *
 *   x          in   bf16 [M][K] (raw bits).
 *   W_gate, W_up    packed [N_ff][K/16] with their gammas (device).
 *   W_down     in   packed [K][N_ff/16] with its gamma (device).
 *   y          out  fp32 [M][K].
 *   workspace  tmp  >= bl_ffn_relu2_workspace_bytes(M, K, N_ff) bytes,
 *                   256-byte aligned; contents undefined afterwards.
 * Shapes follow the rules above for (M, K), (M, N_ff) and both weight
 * matrices. For M in {1, 2, 4, 8} with M*K and M*N_ff up to 128 KiB the
 * step runs in two launches, with each workgroup quantising its activations
 * itself; for M = 16 (same limits) in three: the gate/up launch, one act
 * quant of h, and the GEMV on its codes; otherwise in four. */
int bl_ffn_relu2(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
                 const float* gamma_gate, const uint32_t* W_up, const float* gamma_up,
                 int64_t N_ff, const uint32_t* W_down, const float* gamma_down, float* y,
                 void* workspace, size_t workspace_bytes, void* stream);

/* bl_ffn_relu2 with the sub-layer RMSNorm (subln) on h before its
 * quantisation for the down projection:
 *   y = BitLinear(quantize_acts(h, subln_gain, subln_eps), W_down)
 * with h_q bit-exact and h_scale within 1e-6 relative of
 * bl_relu2_glu_subln_quant's (the fp64 sum of squares is taken in another
 * order when the step runs in two or three launches). subln_gain: bf16 [N_ff] (raw
 * bits), 16-byte aligned, not null; subln_eps > 0. Workspace, shapes and
 * launches as bl_ffn_relu2. Source: as bl_relu2_glu_subln_quant. */
int bl_ffn_relu2_subln(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
                       const float* gamma_gate, const uint32_t* W_up, const float* gamma_up,
                       int64_t N_ff, const uint32_t* W_down, const float* gamma_down,
                       const uint16_t* subln_gain, float subln_eps, float* y, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The gated FFN step for either gating kind, with or without the sub-layer
 * norm: bl_ffn_relu2 (glu_kind BL_GLU_RELU2, subln_gain null),
 * bl_ffn_relu2_subln (BL_GLU_RELU2, gain), or the same steps with SwiGLU
 * gating (BL_GLU_SWIGLU). Every step is the single call's (bl_glu of the
 * kind, bl_quantize_acts of h with or without the gain). Workspace, shapes
 * and launches as bl_ffn_relu2; subln_gain rules of bl_ffn_relu2_subln. */
int bl_ffn_step(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
                const float* gamma_gate, const uint32_t* W_up, const float* gamma_up,
                int64_t N_ff, const uint32_t* W_down, const float* gamma_down, int glu_kind,
                const uint16_t* subln_gain, float subln_eps, float* y, void* workspace,
                size_t workspace_bytes, void* stream);

/* bl_ffn_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, the same launches and the same bits.
 * Its workspace is a fixed 8 MiB array in device memory that the library
 * holds on every device it runs on until the process ends; the call
 * allocates nothing. Shapes whose bl_ffn_relu2_workspace_bytes exceed 8 MiB
 * are BL_ERR_INVALID_ARG (the 8192 -> 28672 -> 8192 FFN fits up to 25
 * tokens, the 2560 -> 6912 one up to 106). All calls on one device share the
 * array: calls that overlap in time on the same device (on different
 * streams, or from different host threads without ordering) race on it and
 * give undefined results; calls ordered on one stream are safe. The first
 * call on a device resolves the array's address there (hipGetSymbolAddress);
 * a failure there is BL_ERR_HIP. */
int bl_ffn_step_noalloc(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
                        const float* gamma_gate, const uint32_t* W_up, const float* gamma_up,
                        int64_t N_ff, const uint32_t* W_down, const float* gamma_down,
                        int glu_kind, const uint16_t* subln_gain, float subln_eps, float* y,
                        void* stream);

/* ---- Other weight formats (decode) ----------------------------------------
 * Two storage formats besides the 2-bit one, each with its own decode
 * product for M <= 16 tokens (the weight-streaming GEMV; the prefill GEMM
 * takes the 2-bit format). Same conventions and shape rules as above; the
 * product additionally needs M * k_extent(K) <= 128 KiB of activations
 * (k_extent: K rounded up to the format's row). */

/* Bytes of a matrix of 1-bit weights: N * 16*ceil(K/128); of base-3 weights:
 * N * 16*ceil(ceil(K/5)/16). 0 if the shape is invalid. Host-only. */
size_t bl_packed_bytes_binary(int64_t N, int64_t K);
size_t bl_packed_bytes_base3(int64_t N, int64_t K);

/* Binary weights, the original BitNet's {-1, +1}. Source: inferownia.pl
 * page above, section "Dlaczego akurat ternarne, a nie czyste zero-jeden"
 * (the earlier BitNet used only -1 and +1 weights).
 *
 *   W          in   fp32 [N][K] latent weights (as bl_quantize_weights).
 *   W_bits     out  uint32 rows of 4*ceil(K/128) words (bl_packed_bytes_binary
 *                   bytes). q = +1 where W >= 0 (either zero), else -1; bit 1
 *                   for +1 in word k/32 at bit 8*(i%4) + i/4, i = k % 32, so
 *                   (word >> p) & 0x01010101 holds the bits of weights
 *                   32j+4p .. 32j+4p+3. Bits past K are 0.
 *   gamma      out  one fp32 (device): the same absmean gamma as
 *                   bl_quantize_weights (mean |W| over the whole matrix).
 *   workspace  tmp  >= bl_quantize_weights_workspace_bytes(N,K) bytes, 8-byte
 *                   aligned. */
int bl_quantize_weights_binary(const float* W, int64_t N, int64_t K, uint32_t* W_bits,
                               float* gamma, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Five ternary weights per byte (1.6 bits per weight), repacked from the
 * 2-bit format so both hold the same codes. Source: inferownia.pl page
 * above, section "Skąd te 1,58 bita" (log2(3) = 1.58 bits carry a ternary
 * weight).
 *
 *   W_packed   in   2-bit weights [N][K/16] from bl_quantize_weights.
 *   W3         out  uint8 rows of 16*ceil(ceil(K/5)/16) bytes: byte j is
 *                   sum_{i<5} c_i 3^i with c_i = q[5j+i] + 1 (least
 *                   significant digit first); positions past K count as
 *                   weight 0, so padding bytes are 121. 16-byte aligned. */
int bl_pack_base3(const uint32_t* W_packed, int64_t N, int64_t K, uint8_t* W3, void* stream);

/* y = (x_q . q^T) * x_scale * gamma for 1-bit (bl_bitlinear_binary) or
 * base-3 (bl_bitlinear_base3) weights, M <= 16: same outputs, bits and
 * arguments as bl_bitlinear for the same codes. Sources as bl_bitlinear,
 * plus the format's passage above. */
int bl_bitlinear_binary(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                        const uint32_t* W_bits, const float* gamma, int64_t N, float* y,
                        int32_t* acc, void* stream);
int bl_bitlinear_base3(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                       const uint8_t* W3, const float* gamma, int64_t N, float* y,
                       int32_t* acc, void* stream);

/* ---- Straight-through backward (training) -------------------------------
 * The gradient of the loss with respect to the BitLinear input when the
 * forward's rounding is treated as the identity (straight-through
 * estimator). Source: juhe.plus (Habr repost), the section on training that
 * follows BinaryConnect (the forward rounds, the backward passes the gradient
 * through as if there were no rounding); comrad404.com «Метод…» (gradients
 * stay in high precision). Both gradients are here: the input's dx and the
 * latent weights' dW. */

/* Bytes of the transposed codes bl_pack_ste_t writes:
 * K * 16*ceil(ceil(N/4)/16); 0 if the shape is invalid. Host-only. */
size_t bl_ste_t_bytes(int64_t N, int64_t K);

/* Transposes the 2-bit weights for the backward pass (offline, once per
 * matrix): row k of qT holds q[n][k] for all n, code c = q + 1 of n = 4j + i
 * at bits 2i of byte j; n >= N is code 1 (weight 0).
 *   W_packed  in   2-bit weights [N][K/16] from bl_quantize_weights.
 *   qT        out  uint8 [K][16*ceil(ceil(N/4)/16)], 16-byte aligned. */
int bl_pack_ste_t(const uint32_t* W_packed, int64_t N, int64_t K, uint8_t* qT, void* stream);

/* dx[m][k] = gamma * sum_n dy[m][n] * q[n][k].
 *   dy     in   bf16 [M][N] (raw bits), gradient of the BitLinear output;
 *               N % 8 == 0, 16-byte aligned.
 *   qT     in   transposed codes from bl_pack_ste_t; gamma from
 *               bl_quantize_weights (device).
 *   dx     out  fp32 [M][K]; must not alias an input.
 * Products of bf16 by {-1, 0, +1} are exact; they are summed in fp32 (within
 * N * 2^-24 * gamma * sum_n |dy[m][n] q[n][k]| of the exact value) and then
 * multiplied by gamma in fp32. Shapes: M >= 1, N >= 8, K >= 64, K % 64 == 0,
 * M*N, M*K, N*K < 2^31. */
int bl_ste_backward_dx(const uint16_t* dy, int64_t M, int64_t N, const uint8_t* qT,
                       const float* gamma, int64_t K, float* dx, void* stream);

/* Bytes of the workspace bl_ste_backward_dw needs: 4*N*Mp + 2*K*Mp with Mp
 * = M rounded up to 64 (bf16 operands with the token index contiguous),
 * plus S*R*K*4 where the call splits the contraction of its last output
 * rows over S workgroups (R = those rows rounded up to 128, at most half a
 * round of 128 x 256 tiles; S >= 2 from 512 tokens on, fp32 partial
 * results); 0 if the shape is invalid (rules of bl_ste_backward_dw).
 * Host-only. */
size_t bl_ste_dw_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Gradient of the latent weights under the straight-through estimator: the
 * forward multiplies the dequantised activations x~ = x_q * x_scale by the
 * weights, and the backward treats the weights' rounding as the identity, so
 *     dW[n][k] = sum_m dy[m][n] * x_q[m][k] * x_scale[m].
 *   dy        in   bf16 [M][N] (raw bits), gradient of the BitLinear output;
 *                  N % 8 == 0, 16-byte aligned.
 *   x_q, x_scale in the forward's quantised input, int8 [M][K] and fp32 [M]
 *                  (bl_quantize_acts); x_q 16-byte aligned.
 *   dW        out  fp32 [N][K] (the latent weights' layout), 16-byte aligned;
 *                  must not alias an input or the workspace.
 *   workspace tmp  >= bl_ste_dw_workspace_bytes(M, N, K) bytes, 256-byte
 *                  aligned; contents undefined afterwards.
 * Each dy * x_scale is rounded to fp32 and split into two bf16 parts whose
 * sum is within 2^-16 of it; products with x_q are exact and accumulate in
 * fp32, so |dW - exact| <= (2^-16 + 2^-24 + 2*Mp*2^-24) * sum_m |dy x_q
 * x_scale| elementwise. Shapes: M >= 1, N >= 8, K >= 64, K % 64 == 0,
 * M*N, M*K, N*K, 2*Mp*N < 2^31. Source: as the section above; juhe.plus
 * (latent full-precision weights receive the gradient). */
int bl_ste_backward_dw(const uint16_t* dy, int64_t M, int64_t N, const int8_t* x_q,
                       const float* x_scale, int64_t K, float* dW, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---- Calibration kernels ------------------------------------------------
 * Measured ceilings for the roofline of the kernels above; they compute
 * nothing of the method. Same conventions as above. */

/* Reads `bytes` bytes at `src` once with 16-byte loads and discards them (a
 * read-only HBM stream). bytes >= 16, bytes % 16 == 0, src 16-byte aligned;
 * sink: >= 4 bytes of device memory, written only for one data pattern. */
int bl_calib_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Copies `bytes` bytes from src to dst with 16-byte loads and stores. Same
 * size and alignment rules as bl_calib_read for both pointers; the ranges
 * must not overlap. */
int bl_calib_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Number of int8 operations (2 per multiply-add) one bl_calib_mfma_i8 call
 * performs for `iters` (0 if iters is out of range), and the int32 elements
 * of the sink it writes. Host-only. */
int64_t bl_calib_mfma_i8_ops(int64_t iters);
size_t bl_calib_mfma_i8_sink_elems(void);

/* Runs a fixed grid of waves, each issuing `iters` rounds of 8 independent
 * 32x32x32 int8 matrix-core instructions on register operands, and writes
 * one int32 per lane to sink. 1 <= iters <= 2^24. */
int bl_calib_mfma_i8(int64_t iters, int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
