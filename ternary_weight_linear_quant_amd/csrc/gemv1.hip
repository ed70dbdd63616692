// Decode BitLinear for one token: the packed weights streamed as 1 KB pieces.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
// "Mnożenie? Jakie mnożenie", and juhe.plus (Habr repost), section «Когда - три
// лучше двух»: with weights in {-1, 0, +1} the product is the sum of the inputs
// whose weight is +1 minus the sum of those whose weight is -1; zero weights
// add nothing. At one token the call reads every packed weight once and does
// little arithmetic per byte: its roofline is HBM bandwidth. What holds it
// below a plain read of the same bytes is each wave's chain (issue the loads,
// stage the token, barrier, consume, reduce, retire) and its VALU work at the
// eight waves per SIMD the hardware keeps, so the variants below amortise the
// per-wave work over as many weights as they can.
//
// Each wave owns RW whole rows (output features) and streams them in order:
// one load instruction per 1 KB piece of a row (16 bytes per lane, 64 lanes
// over contiguous memory; the last piece of a row may be partial). A 16-byte
// load that spreads over 16 rows x 64 bytes, the MFMA operand shape of the
// multi-token GEMV, measured 7-8% slower than contiguous loads of the same
// bytes here.
//
// Arithmetic: the stored codes are c = q + 1 in {0, 1, 2}, four consecutive
// weights per byte position (bit pair p of byte b holds weight 4p + b of its
// 16-weight word). Masking a word in place, without shifting the fields down,
// gives four dwords of byte operands:
//   w & 0x03030303          =      c of weights 0..3
//   w & 0x0C0C0C0C          =  4 * c of weights 4..7
//   w & 0x30303030          = 16 * c of weights 8..11
//   (w >> 2) & 0x30303030   = 16 * c of weights 12..15
// (every byte below 128, so signed bytes read them correctly). v_dot4 of each
// with the four matching activation bytes accumulates 1x, 4x and 16x sums; the
// latter two are exact multiples of 4 and 16, so shifting them right is exact
// division. Their total is sum_k c_k x_k = sum_k q_k x_k + sum_k x_k, and the
// activation sum is subtracted once per row. Five VALU operations expand 16
// weights (the sign-select permute of the multi-token kernels takes nine).
//
// Activations: one token of K int8 values, staged in LDS so that lane l's 64
// bytes for piece j lie at (4j + s) * 1024 + 16 l, s = 0..3 (conflict-free
// 16-byte reads; zeros past K). Three variants:
//   k_gemv1_cached  K <= 4096 * S (S = 1 or 2 pieces per row, the second
//                   partial): the block is loaded by direct global-to-LDS
//                   transfers and each lane keeps its 64 * S bytes in
//                   registers; every wave sums its own lanes' bytes (no
//                   extra barrier);
//   k_gemv1_rows    two to four whole pieces, several rows per wave: staged
//                   through registers and summed per workgroup before one
//                   barrier, then kept in registers while the wave streams
//                   its rows through one ring;
//   k_gemv1_stream  other rows longer than one piece (one row per wave): the
//                   block goes through registers, summed on the way, one
//                   barrier; each piece reads its activations from LDS.
// Waves are independent after the staging barrier (no barrier at the end).
//
// Quantising variants (QX): the input is the bf16 token itself, and every
// workgroup quantises it on the way into LDS with the stand-alone quantiser's
// arithmetic (the helpers in act_quant.hpp); workgroup 0 also writes the codes
// and the scale to global memory. The token's loads are issued before the
// weight loads, which then stay in flight across the reductions and barriers.
// One launch does what the quantiser and the GEMV do in two, at the price of
// 2K bytes of input per workgroup (from L2) instead of K.
//   k_gemv1_cached, QX = 1 or 2 (rows of one piece, optional RMSNorm gain):
//                   256 threads in k_act_quant's assignment and reduction
//                   order, so that the fp64 sum of squares matches too;
//   k_gemv1_rows / k_gemv1_stream, QX (whole pieces, no gain): each thread
//                   quantises its own activation slots after an exact
//                   workgroup max|x| (an integer max of the magnitude bits).
//
// Roofline: HBM. Algorithmic bytes per call = N * K/4 (packed weights) + K
// (activations) + 4 (scale) + 4 (gamma) + 4 * N (y).
#include "act_quant.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace bl {

namespace {

constexpr int kPiece = 1024;                        // packed bytes per piece
constexpr int kPieceK = 4 * kPiece;                 // weights per piece
constexpr int kStreamMaxK = 16 * kPieceK;           // 64 KiB of staged activations
constexpr uint32_t kZeroCodes = 0x55555555u;        // sixteen weights of 0

// Sum over one 16-byte piece of (masked codes) x (activations), exact.
__device__ __forceinline__ int piece_dot(const uint4 wv, const uint4 (&a)[4]) {
    const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
    int v0 = 0, v1 = 0, v2 = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        v0 = __builtin_amdgcn_sdot4((int)(w[s] & 0x03030303u), (int)a[s].x, v0, false);
        v1 = __builtin_amdgcn_sdot4((int)(w[s] & 0x0C0C0C0Cu), (int)a[s].y, v1, false);
        v2 = __builtin_amdgcn_sdot4((int)(w[s] & 0x30303030u), (int)a[s].z, v2, false);
        v2 = __builtin_amdgcn_sdot4((int)((w[s] >> 2) & 0x30303030u), (int)a[s].w, v2, false);
    }
    return v0 + (v1 >> 2) + (v2 >> 4);
}

__device__ __forceinline__ int bytes_sum(const uint4 a, int s) {
    s = __builtin_amdgcn_sdot4((int)a.x, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)a.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)a.z, 0x01010101, s, false);
    return __builtin_amdgcn_sdot4((int)a.w, 0x01010101, s, false);
}

__device__ __forceinline__ void store_row(float* y, int32_t* acc_out, int n, int a, float sc) {
    y[n] = (float)a * sc;
    if (acc_out) acc_out[n] = a;
}

}  // namespace

// Kernel arguments. QX == 0: xq / xs are the token's codes and scale. QX > 0:
// x is the bf16 token (gain: the RMSNorm gain when QX == 2), and xq_out /
// xs_out receive its codes and scale from workgroup 0.
struct Gemv1Args {
    const int8_t* xq;
    const float* xs;
    const uint16_t* x;
    const uint16_t* gain;
    float rms_eps;
    int8_t* xq_out;
    float* xs_out;
    int K;
    const uint8_t* W;
    const float* gamma;
    int N;
    float* y;
    int32_t* acc_out;
};

// Byte offset in the staging layout of activation k.
__device__ __forceinline__ int stage_offset(int k) {
    return (4 * (k / kPieceK) + (k / 16) % 4) * kPiece + 16 * ((k / 64) % 64) + k % 16;
}

// Quantises the token held by threads 0..255 as 16-byte bf16 vectors v =
// tid + 256 j (j < VPT, loaded by load_token), the assignment and reduction
// order of k_act_quant. Writes the codes of every vector below
// NV8 (vectors past K get zero codes) at their staging offsets and returns
// the scale. Workgroup 0 also stores the codes and the scale. Contains two
// barriers: every thread of the workgroup calls it.
template <bool NORM, int VPT>
__device__ __forceinline__ float quantise_token(const uint4 (&cx)[VPT], const uint4 (&cg)[VPT],
                                                int K, int NV8, float rms_eps, uint8_t* smem,
                                                int8_t* xq_out, float* xs_out) {
    __shared__ float s_max[kActThreads / kWave];
    __shared__ double s_ss[kActThreads / kWave];
    const int tid = threadIdx.x;
    const int nvec = K / 8;
    float amax = 0.0f;
    double ss = 0.0;
    act_u16x2 m2 = {0, 0};  // plain: max|x| on the raw bits
    if (tid < kActThreads) {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            if (tid + kActThreads * j < nvec) {
                if constexpr (NORM) act_scan8<true>(cx[j], cg[j], amax, ss);
                else act_scan8_bits(cx[j], m2);
            }
        }
    }
    if constexpr (!NORM) amax = act_bits_max(m2);
    amax = act_reduce<float, true>(amax, s_max);
    double ss_tot = 0.0;
    if (NORM) ss_tot = act_reduce<double, false>(ss, s_ss);
    const float a = act_clamped_max(amax);
    const float inv = 127.0f / a;  // correctly rounded
    const bool first = blockIdx.x == 0;
    if (tid < kActThreads) {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = tid + kActThreads * j;
            if (v < NV8) {
                const uint2 c = v < nvec ? act_quant8<NORM>(cx[j], cg[j], inv) : make_uint2(0u, 0u);
                *reinterpret_cast<uint2*>(smem + stage_offset(8 * v)) = c;
                if (first && v < nvec) reinterpret_cast<uint2*>(xq_out)[v] = c;
            }
        }
    }
    const float scale = act_scale<NORM>(a, ss_tot, K, rms_eps);
    if (first && tid == 0) xs_out[0] = scale;
    return scale;
}

// Loads this thread's bf16 vectors of the token (threads 0..255 only).
template <bool NORM, int VPT>
__device__ __forceinline__ void load_token(const Gemv1Args& p, uint4 (&cx)[VPT], uint4 (&cg)[VPT]) {
    const int tid = threadIdx.x;
    const int nvec = p.K / 8;
    if (tid >= kActThreads) return;
    const uint4* xr = reinterpret_cast<const uint4*>(p.x);
    const uint4* gr = reinterpret_cast<const uint4*>(p.gain);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int v = tid + kActThreads * j;
        if (v < nvec) {
            cx[j] = xr[v];
            cg[j] = NORM ? gr[v] : cx[j];
        }
    }
}

// Plain quantisation of the token in the slot layout of k_gemv1_rows and
// k_gemv1_stream: slot t holds activations 16t .. 16t+15, here as two bf16
// vectors xb[i][0], xb[i][1] for this thread's slots ts[i] (slots at or past
// XP hold zeros and get no codes). max|x| is exact (an integer max of the
// magnitude bits, then over the workgroup's NW waves), and each slot's codes
// come from the stand-alone quantiser's arithmetic, so codes and scale are the
// same bits as k_act_quant's. Workgroup 0 also stores them. Contains a
// barrier: every thread of the workgroup calls it.
template <int XPT, int NW>
__device__ __forceinline__ float quantise_slots(const uint4 (&xb)[XPT][2], const int (&ts)[XPT],
                                                int XP, uint4 (&codes)[XPT], int8_t* xq_out,
                                                float* xs_out) {
    __shared__ float s_max[NW];
    act_u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        act_scan8_bits(xb[i][0], m2);
        act_scan8_bits(xb[i][1], m2);
    }
    const float amax = act_reduce<float, true, NW>(act_bits_max(m2), s_max);
    const float a = act_clamped_max(amax);
    const float inv = 127.0f / a;  // correctly rounded
    const bool first = blockIdx.x == 0;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const uint2 lo = act_quant8<false>(xb[i][0], xb[i][0], inv);
        const uint2 hi = act_quant8<false>(xb[i][1], xb[i][1], inv);
        codes[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        if (first && ts[i] < XP) reinterpret_cast<uint4*>(xq_out)[ts[i]] = codes[i];
    }
    const float scale = act_scale<false>(a, 0.0, 0, 0.0f);
    if (first && threadIdx.x == 0) xs_out[0] = scale;
    return scale;
}

// S pieces per row (K <= 4096 S), RW rows per wave, R loads in flight per lane,
// WPB waves per workgroup, QX as for Gemv1Args. Requires N >= RW.
template <int S, int RW, int R, int WPB, int QX>
__global__ __launch_bounds__(64 * WPB) void k_gemv1_cached(const Gemv1Args p) {
    constexpr int L = S * RW;  // pieces per wave
    constexpr bool NORM = QX == 2;
    constexpr int VPT = QX ? S * kPieceK / 8 / kActThreads : 1;  // bf16 vectors per thread
    static_assert(QX == 0 || 64 * WPB == kActThreads, "the token is quantised by 256 threads");
    __shared__ __align__(16) uint8_t smem[S * kPieceK];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int K = p.K, N = p.N;
    const int RB = K / 4;

    // 1. QX == 0: the codes straight into LDS: transfer q = 4j + s moves, for
    //    each lane l, x[4096 j + 64 l + 16 s, +16) to q * 1024 + 16 l; lanes
    //    past K store zeros instead. QX > 0: the bf16 token into registers.
    uint4 cx[VPT], cg[VPT];
    if constexpr (QX == 0) {
        const uint32_t xbase = lds_offset(smem);
        for (int q = wave; q < 4 * S; q += WPB) {
            const int k0 = kPieceK * (q / 4) + 64 * lane;
            if (k0 < K)
                lds_dma16(p.xq + k0 + 16 * (q % 4), xbase + q * kPiece);
            else
                *reinterpret_cast<uint4*>(smem + q * kPiece + 16 * lane) = make_uint4(0, 0, 0, 0);
        }
    } else {
        load_token<NORM, VPT>(p, cx, cg);
    }
    asm volatile("" ::: "memory");

    // 2. The wave's rows nb .. nb+RW-1 (the last wave of the grid shifts back
    //    to stay inside N and stores only rows from n0 on).
    const int n0 = (blockIdx.x * WPB + wave) * RW;
    const int nb = min(n0, N - RW);
    const uint8_t* wrow = p.W + (size_t)nb * RB + 16 * lane;
    auto load = [&](int i) -> uint4 {
        const int r = i / S, j = i % S;
        return kPiece * j + 16 * lane < RB
                   ? load_stream16(wrow + (size_t)r * RB + kPiece * j)
                   : make_uint4(kZeroCodes, kZeroCodes, kZeroCodes, kZeroCodes);
    };
    uint4 wb[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
        if (u < L) wb[u] = load(u);
    asm volatile("" ::: "memory");

    // 3. QX == 0: this wave's transfers landed (the weight loads, issued after
    //    them, may still be in flight); then every wave's are visible. QX > 0:
    //    quantise the token into LDS, then the codes are visible.
    float scale = 0.0f;
    if constexpr (QX == 0) {
        wait_vmcnt_le8(L < R ? L : R);
    } else {
        scale = quantise_token<NORM, VPT>(cx, cg, K, S * kPieceK / 8, p.rms_eps, smem, p.xq_out,
                                          p.xs_out);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();

    uint4 act[S][4];
    int sx = 0;
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            act[j][s] = *reinterpret_cast<const uint4*>(smem + (4 * j + s) * kPiece + 16 * lane);
            sx = bytes_sum(act[j][s], sx);
        }

    int acc[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r] = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int u = i % R;
        acc[i / S] += piece_dot(wb[u], act[i % S]);
        if (i + R < L) wb[u] = load(i + R);
    }

    if constexpr (QX == 0) scale = p.xs[0];
    const float sc = scale * (*p.gamma);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        // Each lane subtracts its own share of sum x, so one reduction gives
        // sum q x.
        const int a = wave_sum_i32(acc[r] - sx);
        const int n = nb + r;
        if (lane == r && n >= n0) store_row(p.y, p.acc_out, n, a, sc);
    }
}

// One row per wave, R loads in flight per lane. SP > 0: exactly SP whole
// pieces per row (K = 4096 SP), every bound known at compile time; SP = 0:
// any K up to kStreamMaxK, the last piece possibly partial.
template <int SP, int R, int WPB, bool QX = false>
__global__ __launch_bounds__(64 * WPB) void k_gemv1_stream(const Gemv1Args p) {
    static_assert(!QX || SP > 0, "the quantising variant takes whole pieces");
    constexpr int NT = 64 * WPB;
    constexpr int XPT = SP > 0 ? (SP * (kPieceK / 16) + NT - 1) / NT : 4;  // slots per thread
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int wsum[WPB];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int K = SP > 0 ? SP * kPieceK : p.K;
    const int N = p.N;
    const int RB = K / 4;
    const int NP = SP > 0 ? SP : (RB + kPiece - 1) / kPiece;  // pieces per row
    const int XP = NP * (kPieceK / 16);  // 16-byte activation slots, zero past K

    // 1. This thread's activation slots: x[16 t, +16) lands at (4j + s) * 1024
    //    + 16 l with t = 256 j + 4 l + s. Within each run of 64 slots, lane
    //    16 g + i takes slot 4 i + g, so that each quarter-wave writes one
    //    s-block's 16 consecutive slots (256 bytes, every bank once); the
    //    wave's loads still cover its 1 KB of x.
    //    QX: the bf16 values of the same slots, quantised in step 3.
    auto slot_of = [](int u) { return (u & ~63) + 4 * (u % 16) + (u % 64) / 16; };
    uint4 xv[XPT];
    uint4 xb[QX ? XPT : 1][2];
    int ts[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int t = slot_of(tid + NT * i);
        ts[i] = t;
        if constexpr (QX) {
            const uint4* x16 = reinterpret_cast<const uint4*>(p.x);
            xb[i][0] = t < XP ? x16[2 * t] : make_uint4(0, 0, 0, 0);
            xb[i][1] = t < XP ? x16[2 * t + 1] : make_uint4(0, 0, 0, 0);
        } else {
            xv[i] = 16 * t < K ? *reinterpret_cast<const uint4*>(p.xq + 16 * t)
                               : make_uint4(0, 0, 0, 0);
        }
    }
    asm volatile("" ::: "memory");

    // 2. The wave's row (the grid's last waves repeat row N-1 and store nothing).
    const int n0 = blockIdx.x * WPB + wave;
    const int n = min(n0, N - 1);
    const uint8_t* wrow = p.W + (size_t)n * RB + 16 * lane;
    auto load = [&](int j) -> uint4 {
        if (SP > 0) return load_stream16(wrow + kPiece * j);
        return kPiece * j + 16 * lane < RB
                   ? load_stream16(wrow + kPiece * j)
                   : make_uint4(kZeroCodes, kZeroCodes, kZeroCodes, kZeroCodes);
    };
    uint4 wb[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
        if (u < NP) wb[u] = load(u);
    asm volatile("" ::: "memory");

    // 3. Only the weight loads may remain in flight; (QX: quantise the token,)
    //    store the slots and sum them.
    wait_vmcnt_le8(NP < R ? NP : R);
    float scale = 0.0f;
    if constexpr (QX) scale = quantise_slots<XPT, WPB>(xb, ts, XP, xv, p.xq_out, p.xs_out);
    auto slot = [&](int t) { return smem + (4 * (t / 256) + t % 4) * kPiece + 16 * ((t / 4) % 64); };
    int s = 0;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int t = ts[i];
        if (t < XP) {
            *reinterpret_cast<uint4*>(slot(t)) = xv[i];
            s = bytes_sum(xv[i], s);
        }
    }
    for (int u = tid + NT * XPT; SP == 0 && u < XP; u += NT) {  // more slots than XPT per thread
        const int t = slot_of(u);
        const uint4 v =
            16 * t < K ? *reinterpret_cast<const uint4*>(p.xq + 16 * t) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(slot(t)) = v;
        s = bytes_sum(v, s);
    }
    s = wave_sum_i32(s);
    if (lane == 0) wsum[wave] = s;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    int sx = 0;
#pragma unroll
    for (int w = 0; w < WPB; ++w) sx += wsum[w];

    // 4. Ring of R pieces: consume piece j, then refill its slot with j + R.
    int acc = 0;
    for (int b0 = 0; b0 < NP; b0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int j = b0 + u;
            if (j < NP) {
                uint4 a[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[q] = *reinterpret_cast<const uint4*>(smem + (4 * j + q) * kPiece + 16 * lane);
                acc += piece_dot(wb[u], a);
                if (j + R < NP) wb[u] = load(j + R);
            }
        }
    }
    if constexpr (!QX) scale = p.xs[0];
    const int a = wave_sum_i32(acc) - sx;
    if (lane == 0 && n == n0) store_row(p.y, p.acc_out, n, a, scale * (*p.gamma));
}

// Rows of SP whole pieces (K = 4096 SP, SP small), RW rows per wave: the
// stream kernel's staging (through registers, sum x reduced per workgroup, one
// barrier), after which each lane keeps its SP x 64 bytes of activations in
// registers and the wave streams its RW rows through one ring of R pieces, so
// the staging, the barrier and the sum-x reduction are paid once per RW rows
// and no LDS is read per piece. Requires N >= RW.
template <int SP, int RW, int R, int WPB, bool QX = false>
__global__ __launch_bounds__(64 * WPB) void k_gemv1_rows(const Gemv1Args p) {
    constexpr int NT = 64 * WPB;
    constexpr int K = SP * kPieceK;
    constexpr int RB = K / 4;
    constexpr int XP = SP * (kPieceK / 16);            // 16-byte activation slots
    constexpr int XPT = (XP + NT - 1) / NT;            // slots per thread
    constexpr int L = SP * RW;                         // pieces per wave
    __shared__ __align__(16) uint8_t smem[SP * kPieceK];
    __shared__ int wsum[WPB];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int N = p.N;

    // 1. Activation slots as in k_gemv1_stream (the same quarter-wave order;
    //    QX: their bf16 values).
    auto slot_of = [](int u) { return (u & ~63) + 4 * (u % 16) + (u % 64) / 16; };
    auto slot = [&](int t) { return smem + (4 * (t / 256) + t % 4) * kPiece + 16 * ((t / 4) % 64); };
    uint4 xv[XPT];
    uint4 xb[QX ? XPT : 1][2];
    int ts[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int t = slot_of(tid + NT * i);
        ts[i] = t;
        if constexpr (QX) {
            const uint4* x16 = reinterpret_cast<const uint4*>(p.x);
            xb[i][0] = t < XP ? x16[2 * t] : make_uint4(0, 0, 0, 0);
            xb[i][1] = t < XP ? x16[2 * t + 1] : make_uint4(0, 0, 0, 0);
        } else {
            xv[i] = t < XP ? *reinterpret_cast<const uint4*>(p.xq + 16 * t) : make_uint4(0, 0, 0, 0);
        }
    }
    asm volatile("" ::: "memory");

    // 2. The wave's rows nb .. nb+RW-1 (the last wave of the grid shifts back
    //    to stay inside N and stores only rows from n0 on); the first R pieces.
    const int n0 = (blockIdx.x * WPB + wave) * RW;
    const int nb = min(n0, N - RW);
    const uint8_t* wrow = p.W + (size_t)nb * RB + 16 * lane;
    auto load = [&](int i) -> uint4 {
        return load_stream16(wrow + (size_t)(i / SP) * RB + kPiece * (i % SP));
    };
    uint4 wb[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
        if (u < L) wb[u] = load(u);
    asm volatile("" ::: "memory");

    // 3. (QX: quantise the token,) stage and sum the activations; one barrier
    //    (two with QX).
    wait_vmcnt_le8(L < R ? L : R);
    float scale = 0.0f;
    if constexpr (QX) scale = quantise_slots<XPT, WPB>(xb, ts, XP, xv, p.xq_out, p.xs_out);
    int s = 0;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int t = ts[i];
        if (t < XP) {
            *reinterpret_cast<uint4*>(slot(t)) = xv[i];
            s = bytes_sum(xv[i], s);
        }
    }
    s = wave_sum_i32(s);
    if (lane == 0) wsum[wave] = s;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    int sx = 0;
#pragma unroll
    for (int w = 0; w < WPB; ++w) sx += wsum[w];
    uint4 act[SP][4];
#pragma unroll
    for (int j = 0; j < SP; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            act[j][q] = *reinterpret_cast<const uint4*>(smem + (4 * j + q) * kPiece + 16 * lane);

    // 4. The wave's L pieces through a ring of R; each row's sum stored when
    //    its last piece is in.
    if constexpr (!QX) scale = p.xs[0];
    const float sc = scale * (*p.gamma);
    int acc = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int u = i % R;
        acc += piece_dot(wb[u], act[i % SP]);
        if (i + R < L) wb[u] = load(i + R);
        if (i % SP == SP - 1) {
            const int a = wave_sum_i32(acc) - sx;
            const int n = nb + i / SP;
            if (lane == 0 && n >= n0) store_row(p.y, p.acc_out, n, a, sc);
            acc = 0;
        }
    }
}

template <int S, int RW, int R, int WPB, int QX>
static hipError_t launch_cached(const Gemv1Args& a, hipStream_t stream) {
    const int waves = (a.N + RW - 1) / RW;
    const int blocks = (waves + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_gemv1_cached<S, RW, R, WPB, QX>), dim3(blocks), dim3(64 * WPB), 0, stream,
                       a);
    return hipGetLastError();
}

template <int SP, int RW, int R, int WPB, bool QX = false>
static hipError_t launch_rows(const Gemv1Args& a, hipStream_t stream) {
    const int waves = (a.N + RW - 1) / RW;
    const int blocks = (waves + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_gemv1_rows<SP, RW, R, WPB, QX>), dim3(blocks), dim3(64 * WPB), 0, stream,
                       a);
    return hipGetLastError();
}

template <int SP, int R, int WPB, bool QX = false>
static hipError_t launch_stream(const Gemv1Args& a, hipStream_t stream) {
    const int NP = (a.K / 4 + kPiece - 1) / kPiece;
    const size_t lds = (size_t)NP * kPieceK;
    const int blocks = (a.N + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_gemv1_stream<SP, R, WPB, QX>), dim3(blocks), dim3(64 * WPB), lds, stream,
                       a);
    return hipGetLastError();
}

bool gemv1_supported(int64_t M, int64_t K) { return M == 1 && K <= kStreamMaxK; }

// The automatic choice at one token: every shape except rows longer than two
// pieces that end in a partial one (8640 -> 3200 and 11008 -> 4096 measured
// level with the multi-token GEMV there).
bool gemv1_preferred(int64_t M, int64_t K) {
    return gemv1_supported(M, K) && (K <= 2 * kPieceK || K % kPieceK == 0);
}

// Launch shapes, measured (probe copies over ten distinct weight buffers) on
// the 70B rows and on 8192-row matrices of 12288, 16384, 11008 and 32768
// columns. Two to four whole pieces: several rows per wave with the token in
// registers (8192 -> 28672: 11.7 us against 13.2 for one row per wave and 13.5
// for the cached kernel; 12288: 6.1 against 6.4; 16384: 7.5 against 7.7).
// Five to seven pieces: one row per wave, 16-wave workgroups, two pieces in
// flight (28672 -> 8192: 10.7 against 12.0 us for all seven in flight in
// 8-wave workgroups; 20480: 9.4 against 9.8 for two in flight in 8-wave
// ones); eight: all in flight. Rows of one piece, and partial second pieces,
// keep the cached kernel.
hipError_t launch_gemv1(const int8_t* xq, const float* xs, int K, const uint32_t* Wp,
                        const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream) {
    if (K > kStreamMaxK) return hipErrorInvalidValue;
    Gemv1Args a{};
    a.xq = xq;
    a.xs = xs;
    a.K = K;
    a.W = reinterpret_cast<const uint8_t*>(Wp);
    a.gamma = gamma;
    a.N = N;
    a.y = y;
    a.acc_out = acc;
    if (K <= kPieceK) {
        if (N >= 4) return launch_cached<1, 4, 4, 4, 0>(a, stream);
        return launch_cached<1, 1, 1, 4, 0>(a, stream);
    }
    if (K < 2 * kPieceK) {
        if (N >= 2) return launch_cached<2, 2, 2, 4, 0>(a, stream);
        return launch_cached<2, 1, 2, 4, 0>(a, stream);
    }
    // Whole pieces: the piece count as a template.
    switch (K % kPieceK == 0 ? K / kPieceK : 0) {
        case 2:
            if (N >= 4) return launch_rows<2, 4, 4, 4>(a, stream);
            return launch_stream<2, 2, 8>(a, stream);
        case 3:
            if (N >= 4) return launch_rows<3, 4, 4, 4>(a, stream);
            return launch_stream<3, 2, 8>(a, stream);
        case 4:
            if (N >= 2) return launch_rows<4, 2, 4, 8>(a, stream);
            return launch_stream<4, 2, 8>(a, stream);
        case 5: return launch_stream<5, 2, 16>(a, stream);
        case 6: return launch_stream<6, 2, 16>(a, stream);
        case 7: return launch_stream<7, 2, 16>(a, stream);
        case 8: return launch_stream<8, 8, 8>(a, stream);
        default: return launch_stream<0, 2, 8>(a, stream);
    }
}

// One launch quantises and multiplies: rows of one piece (any gain) through
// the cached kernel, whose 256 threads take k_act_quant's assignment and
// reduction order; whole pieces up to eight (no gain) through the rows and
// stream kernels, whose max|x| is exact whatever the order. Measured (HIP
// graphs, ten rotated copies per matrix) against act quant + GEMV: 2560 ->
// 2560 3.9 against 5.2 us per projection, 3200 -> 8640 6.1 against 7.2,
// 8192 -> 28672 13.7 against 15.6, 28672 -> 8192 14.2 against 16.1; on
// 8192-row matrices of 12288 / 16384 / 20480 / 24576 / 32768 columns 7.3 /
// 9.4 / 11.6 / 13.0 / 16.4 against 9.8 / 11.4 / 13.4 / 14.9 / 19.4.
// Workgroup sizes differ from the GEMV's where that measured faster: three
// pieces take 8 waves (7.3 against 7.8 us with 4; at two pieces 8 or 16 waves
// were slower, 14.4-16.0 against 13.6), and from five pieces on 16 waves,
// whose threads hold fewer slots of the token (8-wave workgroups took 13.0,
// 14.5 and 20.3 us at five, six and eight pieces). With a gain on longer rows
// the fp64 sum of squares would be taken in another order than the
// stand-alone quantiser's (the scale could differ in its last bit), and rows
// with a partial second piece keep the cached kernel, whose per-workgroup
// token copies cost more than the second launch saves there.
bool gemv1_quant_supported(int64_t M, int64_t K, bool norm) {
    if (M != 1) return false;
    if (K <= kPieceK) return true;
    return !norm && K % kPieceK == 0 && K <= 8 * kPieceK;
}

hipError_t launch_gemv1_quant(const uint16_t* x, const uint16_t* gain, float rms_eps, int K,
                              const uint32_t* Wp, const float* gamma, int N, float* y,
                              int8_t* xq_out, float* xs_out, hipStream_t stream) {
    if (!gemv1_quant_supported(1, K, gain != nullptr)) return hipErrorInvalidValue;
    Gemv1Args a{};
    a.x = x;
    a.gain = gain;
    a.rms_eps = rms_eps;
    a.xq_out = xq_out;
    a.xs_out = xs_out;
    a.K = K;
    a.W = reinterpret_cast<const uint8_t*>(Wp);
    a.gamma = gamma;
    a.N = N;
    a.y = y;
    if (K <= kPieceK) {
        if (gain) {
            if (N >= 4) return launch_cached<1, 4, 4, 4, 2>(a, stream);
            return launch_cached<1, 1, 1, 4, 2>(a, stream);
        }
        if (N >= 4) return launch_cached<1, 4, 4, 4, 1>(a, stream);
        return launch_cached<1, 1, 1, 4, 1>(a, stream);
    }
    switch (K / kPieceK) {
        case 2:
            if (N >= 4) return launch_rows<2, 4, 4, 4, true>(a, stream);
            return launch_stream<2, 2, 8, true>(a, stream);
        case 3:
            if (N >= 4) return launch_rows<3, 4, 4, 8, true>(a, stream);
            return launch_stream<3, 2, 8, true>(a, stream);
        case 4:
            if (N >= 2) return launch_rows<4, 2, 4, 8, true>(a, stream);
            return launch_stream<4, 2, 8, true>(a, stream);
        case 5: return launch_stream<5, 2, 16, true>(a, stream);
        case 6: return launch_stream<6, 2, 16, true>(a, stream);
        case 7: return launch_stream<7, 2, 16, true>(a, stream);
        default: return launch_stream<8, 4, 16, true>(a, stream);
    }
}

}  // namespace bl
