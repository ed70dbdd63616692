// Shared device helpers for the gfx950 BitLinear kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace bl {

// Raises a kernel's dynamic LDS limit to `max_lds` (when above HIP's 64 KiB
// default) once per device: the attribute belongs to the kernel on the current
// device. `done` keeps a bit per device (devices 0..63; others set it on every
// call). Two threads racing on a first call both set the same value, which is
// harmless. `max_lds` must cover every launch of the kernel that follows.
inline hipError_t allow_dynamic_lds(const void* kern, size_t max_lds,
                                    std::atomic<uint64_t>& done) {
    if (max_lds <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_lds);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Four int8 codes rne(t) packed little-endian, for fp32 t with |t| < 2^22.
// Adding 1.5 * 2^23 rounds t to an integer (ties to even, the default
// rounding of the add) and leaves it, in two's complement, in the low
// mantissa byte; the result is that of rintf on each t. Callers pass
// t = z * (127 / a) with a = max |z| of the token, so |t| <= 127 (1 + 2^-24)^2
// and the [-127, 127] clamp of the codes can never act; z * inv must be
// rounded before the add (the library is built with fp contraction off).
__device__ __forceinline__ uint32_t pack_codes4(float t0, float t1, float t2, float t3) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const uint32_t a = __float_as_uint(t0 + kMagic), b = __float_as_uint(t1 + kMagic);
    const uint32_t c = __float_as_uint(t2 + kMagic), d = __float_as_uint(t3 + kMagic);
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a.b0, b.b0, 0, 0
    const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000c0cu);  // 0, 0, c.b0, d.b0
    return lo | hi;
}

// Gating of a gated FFN: h = bf16_rne(act(gate) * up), the product in fp32.
// kGluRelu2: act(g) = relu(g)^2 in fp32 (the 2B4T FFN). kGluSwiglu: act(g) =
// SiLU(g) = g / (1 + exp(-g)) (the LLaMA-style SwiGLU) evaluated in fp64 and
// rounded once to fp32, so it is the correctly rounded SiLU unless the fp64
// value lies within about 1e-16 of an fp32 rounding boundary; a gate below
// about -709 gives exp(-g) = inf and SiLU = -0.
constexpr int kGluRelu2 = 0, kGluSwiglu = 1;

template <int KIND>
__device__ __forceinline__ uint32_t glu_bits(float g, float u) {
    if constexpr (KIND == kGluRelu2) {
        const float r = g > 0.0f ? g : 0.0f;
        return f32_to_bf16_rne((r * r) * u);
    } else {
        const double gd = (double)g;
        const float s = (float)(gd / (1.0 + exp(-gd)));
        return f32_to_bf16_rne(s * u);
    }
}

// One packed word holds 16 two-bit codes c = q + 1; (w >> 2p) & 0x03030303
// gives the codes of weights 4p..4p+3 of the word in bytes 0..3. A byte
// permute with the table {0xFF, 0x00, 0x01} turns each code into the signed
// int8 weight, so the result is the 16 weights in k order as MFMA operand
// bytes.
__device__ __forceinline__ v4i expand_word(uint32_t w) {
    const uint32_t m = 0x03030303u;
    const uint32_t lut = 0x000100FFu;  // byte 0 -> -1, 1 -> 0, 2 -> +1
    v4i r;
    r[0] = (int)__builtin_amdgcn_perm(0u, lut, w & m);
    r[1] = (int)__builtin_amdgcn_perm(0u, lut, (w >> 2) & m);
    r[2] = (int)__builtin_amdgcn_perm(0u, lut, (w >> 4) & m);
    r[3] = (int)__builtin_amdgcn_perm(0u, lut, (w >> 6) & m);
    return r;
}

// Same 16 weights NEGATED (-q), in 9 instructions instead of 11. The
// fields of bit-pairs 1 and 3 are masked in place, giving selectors
// {0, 4, 8}: 0 and 4 pick byte 0 of the second and first permute source,
// and 8 replicates bit 15 of the second source (set) into 0xFF. A product
// accumulated with these bytes is the exact negative of the true sum.
__device__ __forceinline__ v4i expand_word_neg(uint32_t w) {
    const uint32_t m0 = 0x03030303u, m1 = 0x0C0C0C0Cu;
    const uint32_t lut0 = 0x00FF0001u;  // sel 0 -> +1, 1 -> 0, 2 -> -1
    const uint32_t lut1 = 0x00008001u;  // sel 0 -> +1, 4 -> 0 (src0), 8 -> -1
    const uint32_t t = w >> 4;
    v4i r;
    r[0] = (int)__builtin_amdgcn_perm(0u, lut0, w & m0);
    r[1] = (int)__builtin_amdgcn_perm(0u, lut1, w & m1);
    r[2] = (int)__builtin_amdgcn_perm(0u, lut0, t & m0);
    r[3] = (int)__builtin_amdgcn_perm(0u, lut1, t & m1);
    return r;
}

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// LDS byte offset of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(size_t)(const lds_u8_t*)p;
}

// 16 bytes of a weight stream that the call reads exactly once, in loads
// whose lines the wave consumes whole at once (the one-token GEMV's 1 KB
// pieces, the fused FFN kernel's chunks): a non-temporal load, so the stream
// does not displace the lines that are reused (the staged activations, the
// token every workgroup reads) from the caches. On the 70B rows at one token
// this took the GEMV from 12.0 to 11.1 us per launch and a plain read of the
// same bytes from 10.6 to 9.9; the fused FFN step at 16 tokens 16.7 -> 16.0
// us per layer. The GEMM's weight tiles (32 bytes of a line per K step) and
// the multi-token GEMV's chunks keep normal loads: with the hint the rest of
// a line is gone before it is read (64 x 8192 -> 28672: 25.0 -> 30.7 us;
// the GEMV at 4 tokens 17.3 -> 18.2, base-3 rows 15.2 -> 16.9).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
    const v4u_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes per lane from global memory straight into LDS at
// lds_base + 16 * lane (global_load_lds_dwordx4). lds_base must be wave-
// uniform. Issued through asm so that the compiler adds no conservative
// waits before later LDS reads; completion is tracked with explicit vmcnt
// waits (vector memory operations complete in issue order). The LDS address
// is an input operand bound to M0, so the compiler sets M0 itself (folding
// the address arithmetic into that move) and knows what M0 holds afterwards:
// one scalar instruction per transfer instead of a save, a set and a restore.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
    asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(gptr), "{m0}"(lds_base) : "memory");
}

// The same transfer from a wave-uniform 64-bit base (SGPRs) plus a per-lane
// 32-bit byte offset: a loop that advances the base moves no per-lane address.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("global_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_base)
                 : "memory");
}

// s_waitcnt with vmcnt = n (other counters unconstrained), n < 64.
#define BL_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | ((((n) >> 4) & 3) << 14))

// Wait until at most n (0..8, wave-uniform) vector memory operations are
// outstanding.
__device__ __forceinline__ void wait_vmcnt_le8(int n) {
    switch (n) {
        case 0: BL_WAIT_VMCNT(0); break;
        case 1: BL_WAIT_VMCNT(1); break;
        case 2: BL_WAIT_VMCNT(2); break;
        case 3: BL_WAIT_VMCNT(3); break;
        case 4: BL_WAIT_VMCNT(4); break;
        case 5: BL_WAIT_VMCNT(5); break;
        case 6: BL_WAIT_VMCNT(6); break;
        case 7: BL_WAIT_VMCNT(7); break;
        default: BL_WAIT_VMCNT(8); break;
    }
}

// Physical 16-byte chunk of logical chunk c in LDS row r: c ^ swz(r). Both
// depend only on r % 32, so fragment addresses of different 32-row tiles
// differ by constants. Any 8 (A: 128-byte rows) or 16 aligned consecutive
// rows map their reads of one logical chunk to distinct banks, for 32 or 64
// LDS banks alike.
__device__ __forceinline__ int swz_a(int r) { return (r ^ ((r >> 3) & 3)) & 7; }
__device__ __forceinline__ int swz_b(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

// Wait until at most `stages` (wave-uniform, 0..S) pipeline stages of LOADS
// vector memory instructions each are still outstanding (they complete in
// issue order).
template <int LOADS, int S>
__device__ __forceinline__ void wait_stages(int stages) {
    static_assert(LOADS * S < 64, "vmcnt range");
    if constexpr (S == 0) {
        BL_WAIT_VMCNT(0);
    } else {
        if (stages >= S) {
            BL_WAIT_VMCNT(S * LOADS);
        } else {
            wait_stages<LOADS, S - 1>(stages);
        }
    }
}

// Sum of an int32 over the 64 lanes of a wave (all lanes active), returned in
// every lane: each 16-lane row forms inclusive prefix sums with DPP row shifts
// (lanes shifted in from outside the row read 0), then the four row totals
// are read from lanes 15, 31, 47 and 63. VALU only, no LDS round trips.
__device__ __forceinline__ int wave_sum_i32(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
    return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) +
           __builtin_amdgcn_readlane(v, 47) + __builtin_amdgcn_readlane(v, 63);
}

// Maximum of a uint32 over the 64 lanes of a wave (all lanes active), in every
// lane, the same way: DPP row shifts (lanes shifted in read 0, neutral for an
// unsigned max), then the four row results.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 15),
                   (uint32_t)__builtin_amdgcn_readlane((int)v, 31)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v, 47),
                   (uint32_t)__builtin_amdgcn_readlane((int)v, 63)));
}

}  // namespace bl
