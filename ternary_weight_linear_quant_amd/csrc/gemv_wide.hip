// Decode BitLinear for 17..64 tokens: stream the packed weights once, with
// the activations staged in K blocks.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
// "Mnożenie? Jakie mnożenie", and juhe.plus (Habr repost), section «Когда -
// три лучше двух»: the ternary product is a sum of the inputs with +1 weights
// minus those with -1 weights; zero weights drop out. As in the small-M
// GEMV, the int8 matrix cores do the sign selection on weights expanded to
// {+1, 0, -1} bytes (negated; the exact sums are flipped at the end).
//
// Between the GEMV (M <= 16: 16 weight rows per workgroup, the whole
// activation block in LDS) and the GEMM (tiles staged stage by stage behind
// a barrier each 128 k), this shape needs both: at 64 tokens the activations
// are re-read from L2 once per workgroup (ratio 256 / rows per workgroup to
// the weight bytes), so a workgroup takes 128 weight rows; and they no
// longer fit LDS whole, so they are staged in 512-wide K blocks, double
// buffered through registers, one barrier per block.
//
// v_mfma_i32_32x32x32_i8 with A = activations (32 tokens x 32 k; tokens
// 32..63 in a second accumulator) and B = weights (32 rows x 32 k): a lane
// (r = l % 32, g = l / 32) of a wave loads, for chunk c (0..3) of a K block,
// 16 bytes of weight row r covering k = 128c + 64g .. +64 within the block,
// i.e. four packed words, word s feeding sub-step s with k = 128c + 64g +
// 16s .. +16; the activation lane
// (t, g) reads the same 16 k of token t. The C layout (rows = tokens,
// columns = weight rows) makes the output stores run along a token's row.
// When 128-row workgroups would leave CUs idle, K is split across
// workgroups whose int32 partial sums are added into y (zeroed first) and
// rescaled by a final kernel; integer sums are exact in any order.
//
// Roofline: HBM (weights) and int8 MFMA (2*M*N*K ops) together: at 64
// tokens the shape sits at the ridge.
#include "common.hpp"
#include "launch.hpp"

namespace bl {

constexpr int kWideThreads = 256;  // 4 waves of 32 weight rows
constexpr int kWideRows = 128;
constexpr int kWideKB = 512;       // K block
constexpr int kWideMaxM = 64;
constexpr int kWideSlots = (kWideKB / 16) * kWideMaxM;  // 16-byte activation slots per block
constexpr int kWideXLoads = kWideSlots / kWideThreads;  // per thread per block

__global__ __launch_bounds__(kWideThreads, 2) void k_gemv_wide(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, int K,
    const uint32_t* __restrict__ Wp, const float* __restrict__ gamma_p, int N,
    float* __restrict__ y, int32_t* __restrict__ acc_out, int kb_per_split, int split) {
    // Two activation buffers: slot (j, t) = 16 bytes of token t at k = 16j
    // of the block, at (j * 64 + (t ^ j)) * 16. The XOR keeps both the
    // staging stores (32 consecutive j of one token per half-wave) and the
    // fragment reads (consecutive tokens of one j) on distinct banks.
    __shared__ __align__(16) uint8_t xbuf[2][kWideSlots * 16];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int nRB = (N + kWideRows - 1) / kWideRows;
    const int rb = (int)blockIdx.x % nRB, sp = (int)blockIdx.x / nRB;
    const int KBt = (K + kWideKB - 1) / kWideKB;
    const int kb0 = split ? sp * kb_per_split : 0;
    const int nkb = split ? min(kb_per_split, KBt - kb0) : KBt;  // >= 1

    const int r = lane % 32, g = lane / 32;
    const int wrow = rb * kWideRows + wave * 32 + r;
    const uint8_t* wbase = reinterpret_cast<const uint8_t*>(Wp) +
                           (size_t)min(wrow, N - 1) * (K / 4) + 16 * g;

    // Loads of K block kb into registers: activations (kWideXLoads slots per
    // thread; tokens >= M and k >= K read as zeros) and this lane's weights
    // (4 chunks of 16 bytes; k >= K, always whole 64-weight ranges since
    // K % 64 == 0, are left zero and masked at the MFMA).
    uint4 xr[kWideXLoads];
    uint4 wb[4], wn[4];
    // Staging: thread p reads chunk j = p % 32 of token t = p / 32, so 32
    // lanes read one token's 512 contiguous bytes.
    auto load_x = [&](int kb) {
#pragma unroll
        for (int i = 0; i < kWideXLoads; ++i) {
            const int p = tid + kWideThreads * i;
            const int j = p % 32, t = p / 32;
            const int k = kb * kWideKB + 16 * j;
            xr[i] = (t < M && k < K) ? *reinterpret_cast<const uint4*>(xq + (size_t)t * K + k)
                                     : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kWideXLoads; ++i) {
            const int p = tid + kWideThreads * i;
            const int j = p % 32, t = p / 32;
            *reinterpret_cast<uint4*>(&xbuf[buf][16 * (j * kWideMaxM + (t ^ j))]) = xr[i];
        }
    };
    auto load_w = [&](uint4* w, int kb) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int k0 = kb * kWideKB + 128 * c + 64 * g;
            w[c] = k0 < K ? *reinterpret_cast<const uint4*>(wbase + (size_t)kb * (kWideKB / 4) +
                                                          32 * c)
                          : make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
        }
    };

    v16i acc[2];
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[tg][v] = 0;

    auto process = [&](const uint4* w, int buf) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w4[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const v4i b = expand_word_neg(w4[s]);
                const int j = 8 * c + 4 * g + s;
#pragma unroll
                for (int tg = 0; tg < 2; ++tg) {
                    if (tg == 1 && M <= 32) break;  // wave-uniform: no tokens 32..63
                    const v4i a = *reinterpret_cast<const v4i*>(
                        &xbuf[buf][16 * (j * kWideMaxM + ((32 * tg + r) ^ j))]);
                    acc[tg] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[tg], 0, 0, 0);
                }
            }
        }
    };

    // Prologue: block kb0 staged, its weights in registers.
    load_x(kb0);
    load_w(wb, kb0);
    store_x(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    for (int i = 0; i < nkb; ++i) {
        const int buf = i & 1;
        const bool more = i + 1 < nkb;
        if (more) {
            load_x(kb0 + i + 1);
            load_w(wn, kb0 + i + 1);
        }
        process(wb, buf);
        if (more) {
            store_x(buf ^ 1);
#pragma unroll
            for (int c = 0; c < 4; ++c) wb[c] = wn[c];
        }
        // Every wave is done with buffer `buf` and has stored buffer buf^1.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }

    // C layout: lane l, register v holds token 8*(v/4) + 4*(l/32) + v%4 (+32
    // for the second accumulator) and weight row l % 32 of this wave.
    if (wrow >= N) return;
    // Two straight loops, one per mode, so the compiler's wait placement
    // sees no joins between the atomics or the stores.
    if (split) {
        int32_t* yi = reinterpret_cast<int32_t*>(y);
#pragma unroll
        for (int tg = 0; tg < 2; ++tg)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = 32 * tg + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
                if (t < M)
                    __hip_atomic_fetch_add(yi + (size_t)t * N + wrow, -acc[tg][v],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        return;
    }
    // Token scales before the first store, then one wait: a load issued among
    // the stores would wait for them too (one counter, issue order).
    const float gm = *gamma_p;
    float xsr[2][16];
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = 32 * tg + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
            xsr[tg][v] = t < M ? xs[t] : 0.0f;
        }
    BL_WAIT_VMCNT(0);
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = 32 * tg + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
            if (t < M) {
                const int32_t a = -acc[tg][v];
                const size_t o = (size_t)t * N + wrow;
                y[o] = (float)a * (xsr[tg][v] * gm);
                if (acc_out) acc_out[o] = a;
            }
        }
}

bool gemv_wide_supported(int64_t M, int64_t K) { return M >= 1 && M <= kWideMaxM && K >= 64; }

namespace {

struct WidePlan {
    int nRB, KBt, splits, per;
};

// Two workgroups fit a CU (64 KB of LDS each). The split count minimises
// the makespan: rounds of 2 * 256 resident workgroups times the K blocks of
// one split, plus one block's worth for its prologue and partial-sum
// atomics.
WidePlan wide_plan(int N, int K) {
    constexpr long kSlots = 2 * 256;
    WidePlan p{(N + kWideRows - 1) / kWideRows, (K + kWideKB - 1) / kWideKB, 1, 0};
    long best = -1;
    for (int s = 1; s <= p.KBt; ++s) {
        const int per = (p.KBt + s - 1) / s;
        const int used = (p.KBt + per - 1) / per;
        const long cost = (((long)p.nRB * used + kSlots - 1) / kSlots) * (per + 1);
        if (best < 0 || cost < best) best = cost, p.splits = used, p.per = per;
    }
    return p;
}

}  // namespace

// Only worth it when a workgroup streams at least four K blocks: with
// fewer, the prologue (first block's loads, nothing to overlap them with)
// dominates and the GEMM's deeper staging wins. Beyond that, against the GEMM (measured with HIP graphs at 17..64 tokens on the 2B4T,
// 3B and 70B projection shapes): the wide kernel's time grows with the token
// count, the GEMM's hardly (its 64-row tiles are padded either way). The
// wide kernel stays ahead up to 24 tokens and on matrices under 16 Mi
// weights; the GEMM is ahead from 48 tokens on larger matrices, and from 33
// tokens on wide ones (N > K) of at least 24 Mi weights.
bool gemv_wide_preferred(int64_t M, int64_t N, int64_t K) {
    if (!gemv_wide_supported(M, K) || wide_plan((int)N, (int)K).per < 4) return false;
    const int64_t w = N * K;
    if (M >= 48) return w < (16ll << 20);
    if (M > 24) return !(N > K && w >= (24ll << 20));
    return true;
}

hipError_t launch_gemv_wide(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                            const float* gamma, int N, float* y, int32_t* acc,
                            hipStream_t stream) {
    if (!gemv_wide_supported(M, K)) return hipErrorInvalidValue;
    const WidePlan pl = wide_plan(N, K);
    const int nRB = pl.nRB, KBt = pl.KBt, splits = pl.splits;
    if (splits <= 1) {
        hipLaunchKernelGGL(k_gemv_wide, dim3(nRB), dim3(kWideThreads), 0, stream, xq, xs, M, K,
                           Wp, gamma, N, y, acc, KBt, 0);
        return hipGetLastError();
    }
    const int per = pl.per, used = splits;
    const size_t total = (size_t)M * N;
    hipError_t e = launch_splitk_zero(reinterpret_cast<int32_t*>(y), total, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gemv_wide, dim3(nRB * used), dim3(kWideThreads), 0, stream, xq, xs, M,
                       K, Wp, gamma, N, y, acc, per, 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_splitk_finalize(y, xs, gamma, acc, N, total, stream);
}

}  // namespace bl
