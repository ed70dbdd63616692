// Per-token absmax int8 activation quantisation, optionally fused with the
// RMSNorm that precedes BitLinear, and the same quantisation fused with the
// squared-ReLU gating of a 2B4T-style FFN.
//
// Source: comrad404.com, "BitNet b1.58: что показала работа Microsoft об
// «эре 1-битных LLM»", section «Метод: как устроен BitNet b1.58»: activations
// are carried as 8-bit integers, and the input is normalised (RMSNorm) before
// it is quantised. inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów",
// section "Zrób to sam — Microsoft wypuścił konkretny model", and kripta.biz
// (2B4T article): the 2B4T FFN uses squared ReLU.
//
// One workgroup per token, one pass over memory: each thread loads its
// 16-byte vectors of the token once and keeps them in registers while the
// workgroup reduces max|z| (exact, order-free) and, when fused, sum x^2 in
// fp64; then it writes the codes. Codes: rne(z * (127/a)) clamped to
// [-127, 127] in fp32; since a positive per-token factor cancels in absmax
// quantisation, the codes of RMSNorm(x) are those of z = x*g (exact in fp32)
// and 1/rms goes into the scale. Tokens longer than the register cache take a
// second pass that re-reads them (L2-resident). Roofline: HBM, 2 B read +
// 1 B written per element (8 B read for the gated variant).
#include <type_traits>

#include "act_quant.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace bl {

constexpr int kActCache = 14;  // 16-byte vectors cached per thread, at most (K <= 28672)

// CACHE: 16-byte vectors cached per thread, the smallest instantiation that
// holds the token (a larger cache holds registers the token does not use and
// lowers the workgroups a CU keeps in flight); tokens longer than
// kActCache vectors per thread take the uncached two-pass loop. NT: threads
// per token (256, or 1024 for a few long tokens, where one workgroup per
// token leaves most CUs idle and the per-thread chain of loads, scan and
// codes is the call's latency).
template <bool FUSED, int CACHE, int NT>
__global__ __launch_bounds__(NT) void k_act_quant(
    const uint16_t* __restrict__ x, int64_t K, const uint16_t* __restrict__ gain,
    float rms_eps, int8_t* __restrict__ xq, float* __restrict__ scale) {
    constexpr int NW = NT / kWave;
    __shared__ float s_max[NW];
    __shared__ double s_ss[NW];
    const int64_t m = blockIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(x + m * K);
    const uint4* grow = reinterpret_cast<const uint4*>(gain);
    const int tid = threadIdx.x;
    const int nvec = (int)(K / 8);  // 8 bf16 per 16 bytes
    const bool cached = nvec <= CACHE * NT;

    uint4 cx[CACHE];
    uint4 cg[FUSED ? CACHE : 1];
    if (cached) {
#pragma unroll
        for (int j = 0; j < CACHE; ++j) {
            const int v = tid + NT * j;
            if (v < nvec) {
                cx[j] = row[v];
                if (FUSED) cg[j] = grow[v];
            }
        }
    }
    float amax = 0.0f;
    double ss = 0.0;
    act_u16x2 m2 = {0, 0};  // plain: max|x| on the raw bits
    auto scan = [&](const uint4 d, const uint4 gv) {
        if constexpr (FUSED) act_scan8<true>(d, gv, amax, ss);
        else act_scan8_bits(d, m2);
    };
    if (cached) {
#pragma unroll
        for (int j = 0; j < CACHE; ++j)
            if (tid + NT * j < nvec) scan(cx[j], FUSED ? cg[j] : cx[j]);
    } else {
        for (int v = tid; v < nvec; v += NT) scan(row[v], FUSED ? grow[v] : row[v]);
    }
    if constexpr (!FUSED) amax = act_bits_max(m2);
    amax = act_reduce<float, true, NW>(amax, s_max);
    double ss_tot = 0.0;
    if (FUSED) ss_tot = act_reduce<double, false, NW>(ss, s_ss);
    const float a = act_clamped_max(amax);
    const float inv = 127.0f / a;  // correctly rounded

    uint2* out = reinterpret_cast<uint2*>(xq + m * K);
    auto emit = [&](int v, const uint4 d, const uint4 gv) { out[v] = act_quant8<FUSED>(d, gv, inv); };
    if (cached) {
#pragma unroll
        for (int j = 0; j < CACHE; ++j) {
            const int v = tid + NT * j;
            if (v < nvec) emit(v, cx[j], FUSED ? cg[j] : cx[j]);
        }
    } else {
        for (int v = tid; v < nvec; v += NT) emit(v, row[v], FUSED ? grow[v] : row[v]);
    }
    if (tid == 0) scale[m] = act_scale<FUSED>(a, ss_tot, K, rms_eps);
}

// h = bf16_rne(act(g) * u) for one 4-wide fp32 vector, as two dwords of bf16
// bits.
template <int KIND>
__device__ __forceinline__ uint2 glu4(const float4 g, const float4 u) {
    return make_uint2(glu_bits<KIND>(g.x, u.x) | (glu_bits<KIND>(g.y, u.y) << 16),
                      glu_bits<KIND>(g.z, u.z) | (glu_bits<KIND>(g.w, u.w) << 16));
}

// Gating (squared ReLU or SwiGLU) fused with per-token absmax quantisation of
// its bf16 result: identical to the gating call followed by bl_quantize_acts
// (plain).
// SUBLN: the sub-layer RMSNorm with gain g between the gating and the
// quantisation, as bl_quantize_acts(h, g) computes it: codes of z = h*g,
// scale a / (127 * rms(h)) with sum h^2 in fp64.
constexpr int kGluCache = 12;  // 4-element vectors cached per thread, at most (K <= 12288)

// CACHE: as for k_act_quant, the smallest instantiated cache (in 4-element
// vectors per thread) that holds the row.
template <int KIND, bool SUBLN, int CACHE>
__global__ __launch_bounds__(kActThreads) void k_glu_quant(
    const float* __restrict__ gate, const float* __restrict__ up, int64_t K,
    const uint16_t* __restrict__ gain, float rms_eps, int8_t* __restrict__ hq,
    float* __restrict__ scale) {
    __shared__ float s_max[kActThreads / kWave];
    __shared__ double s_ss[kActThreads / kWave];
    const int64_t m = blockIdx.x;
    const float4* grow = reinterpret_cast<const float4*>(gate + m * K);
    const float4* urow = reinterpret_cast<const float4*>(up + m * K);
    const uint2* gnv = reinterpret_cast<const uint2*>(gain);  // 4 bf16 per vector
    const int tid = threadIdx.x;
    const int nvec = (int)(K / 4);
    const bool cached = nvec <= CACHE * kActThreads;

    // With a gain, the cached path keeps the gain vectors beside the gated
    // values: a gain load issued among the code stores would wait for them
    // (vector loads and stores retire through one counter in issue order).
    uint2 ch[CACHE];
    uint2 cgn[SUBLN ? CACHE : 1];
    float amax = 0.0f;
    double ss = 0.0;
    auto scan = [&](const uint2 h, const uint2 gv) {
        const uint32_t hw[2] = {h.x, h.y};
        const uint32_t gw[2] = {gv.x, gv.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float hf = bf16_to_f32((hw[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
            float z = hf;
            if (SUBLN) {
                z = hf * bf16_to_f32((gw[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
                ss += (double)hf * (double)hf;
            }
            amax = fmaxf(amax, fabsf(z));
        }
    };
    if (cached) {
        float4 cg[CACHE], cu[CACHE];
#pragma unroll
        for (int j = 0; j < CACHE; ++j) {
            const int v = tid + kActThreads * j;
            if (v < nvec) {
                cg[j] = grow[v];
                cu[j] = urow[v];
                if (SUBLN) cgn[j] = gnv[v];
            }
        }
#pragma unroll
        for (int j = 0; j < CACHE; ++j) {
            const int v = tid + kActThreads * j;
            if (v < nvec) {
                ch[j] = glu4<KIND>(cg[j], cu[j]);
                scan(ch[j], SUBLN ? cgn[j] : ch[j]);
            }
        }
    } else {
        for (int v = tid; v < nvec; v += kActThreads)
            scan(glu4<KIND>(grow[v], urow[v]), SUBLN ? gnv[v] : make_uint2(0u, 0u));
    }
    amax = act_reduce<float, true>(amax, s_max);
    double ss_tot = 0.0;
    if (SUBLN) ss_tot = act_reduce<double, false>(ss, s_ss);
    const float a = act_clamped_max(amax);
    const float inv = 127.0f / a;

    uint32_t* out = reinterpret_cast<uint32_t*>(hq + m * K);
    auto emit = [&](int v, const uint2 h, const uint2 gv) {
        const uint32_t hw[2] = {h.x, h.y};
        const uint32_t gw[2] = {gv.x, gv.y};
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float z = bf16_to_f32((hw[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
            if (SUBLN) z = z * bf16_to_f32((gw[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
            float t = __builtin_rintf(z * inv);
            t = fminf(fmaxf(t, -127.0f), 127.0f);
            packed |= ((uint32_t)((int)t) & 0xFFu) << (8 * e);
        }
        out[v] = packed;
    };
    if (cached) {
#pragma unroll
        for (int j = 0; j < CACHE; ++j) {
            const int v = tid + kActThreads * j;
            if (v < nvec) emit(v, ch[j], SUBLN ? cgn[j] : ch[j]);
        }
    } else {
        for (int v = tid; v < nvec; v += kActThreads)
            emit(v, glu4<KIND>(grow[v], urow[v]), SUBLN ? gnv[v] : make_uint2(0u, 0u));
    }
    if (tid == 0) scale[m] = act_scale<SUBLN>(a, ss_tot, K, rms_eps);
}

hipError_t launch_quantize_acts(const uint16_t* x, int64_t M, int64_t K, const uint16_t* gain,
                                float rms_eps, int8_t* xq, float* scale, hipStream_t stream) {
    // 1024 threads per token for fewer than 128 tokens of more than 4096
    // values; rows of up to 4096 keep 256 (the one-token GEMV's own quantiser
    // shares that assignment and order, so both give the same scale bits).
    const bool wide = M < 128 && K > 4096;
    const int nt = wide ? 1024 : kActThreads;
    const int64_t per = (K / 8 + nt - 1) / nt;  // vectors per thread
    auto go = [&](auto fused, auto cache, auto threads) {
        hipLaunchKernelGGL((k_act_quant<decltype(fused)::value, decltype(cache)::value,
                                        decltype(threads)::value>),
                           dim3((unsigned)M), dim3(decltype(threads)::value), 0, stream, x, K,
                           gain, rms_eps, xq, scale);
    };
    // At 1024 threads a cache of 8 vectors is the largest that fits without
    // spilling (longer tokens take the two-pass loop).
    auto pick = [&](auto fused, auto threads) {
        constexpr int kMax = decltype(threads)::value == kActThreads ? kActCache : 8;
        if (per <= 2) go(fused, std::integral_constant<int, 2>(), threads);
        else if (per <= 4) go(fused, std::integral_constant<int, 4>(), threads);
        else if (per <= 8 || kMax == 8) go(fused, std::integral_constant<int, 8>(), threads);
        else go(fused, std::integral_constant<int, kMax>(), threads);
    };
    auto by_threads = [&](auto fused) {
        if (wide) pick(fused, std::integral_constant<int, 1024>());
        else pick(fused, std::integral_constant<int, kActThreads>());
    };
    if (gain) by_threads(std::true_type());
    else by_threads(std::false_type());
    return hipGetLastError();
}

namespace {
template <int KIND>
void launch_glu_quant_kind(const float* gate, const float* up, int64_t M, int64_t K,
                           const uint16_t* gain, float rms_eps, int8_t* hq, float* scale,
                           hipStream_t stream) {
    const int64_t per = (K / 4 + kActThreads - 1) / kActThreads;  // vectors per thread
    auto go = [&](auto subln, auto cache) {
        hipLaunchKernelGGL((k_glu_quant<KIND, decltype(subln)::value, decltype(cache)::value>),
                           dim3((unsigned)M), dim3(kActThreads), 0, stream, gate, up, K, gain,
                           rms_eps, hq, scale);
    };
    auto pick = [&](auto subln) {
        if (per <= 2) go(subln, std::integral_constant<int, 2>());
        else if (per <= 4) go(subln, std::integral_constant<int, 4>());
        else if (per <= 8) go(subln, std::integral_constant<int, 8>());
        else go(subln, std::integral_constant<int, kGluCache>());
    };
    if (gain) pick(std::true_type());
    else pick(std::false_type());
}
}  // namespace

hipError_t launch_glu_quant(const float* gate, const float* up, int64_t M, int64_t K, int kind,
                            const uint16_t* gain, float rms_eps, int8_t* hq, float* scale,
                            hipStream_t stream) {
    if (kind == kGluSwiglu)
        launch_glu_quant_kind<kGluSwiglu>(gate, up, M, K, gain, rms_eps, hq, scale, stream);
    else
        launch_glu_quant_kind<kGluRelu2>(gate, up, M, K, gain, rms_eps, hq, scale, stream);
    return hipGetLastError();
}

}  // namespace bl
