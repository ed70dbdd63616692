// Prefill BitLinear (many tokens): int8 MFMA GEMM over 2-bit ternary weights.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
// "Mnożenie? Jakie mnożenie", and juhe.plus (Habr repost), section «Когда - три
// лучше двух»: a ternary weight turns each multiply into an add, a subtract or
// nothing. At prefill the work is compute-bound (2*M*N*K int8 operations over
// 2 bits of weight and M*K bytes of activations), so the add/subtract is run
// on the int8 matrix cores with the weights expanded to {-1, 0, +1} bytes:
// every product and every int32 sum is exact.
//
// y = x_q . q^T with v_mfma_i32_32x32x32_i8: A = activation tile (rows =
// tokens), B = weight tile (rows = output features), both k-contiguous.
// Workgroup: WGM x WGN waves over a BM x BN tile, each wave a (BM/WGM) x
// (BN/WGN) block of 32 x 32 MFMA tiles; K step 128. A STAGES-deep LDS ring
// is filled with global_load_lds_dwordx4 (each lane's 16 bytes land directly
// in LDS, no register staging; a wave-uniform base in SGPRs plus a fixed
// per-lane offset, so a stage's addresses cost no vector arithmetic): per
// stage the activation tile (BM x 128 B) and the PACKED weight tile (BN x 32
// B, 2 bits per weight). Loads for stage kt+STAGES-1 are issued before
// computing stage kt, and an explicit vmcnt wait keeps STAGES-1 stages in
// flight.
//
// Fragment reads: lane (r, g) of a B fragment reads 16 B = 4 packed words of
// its weight row; word s feeds k-substep s after expansion to 16 signed bytes
// with byte permutes (v_perm), so the weights cross LDS at 2 bits. The A lane
// (r, g) reads, for substep s, the 16 activation bytes of the same k positions
// (chunk 4g + s of its row). 16-byte chunks are XOR-swizzled by row so that
// these reads are free of bank conflicts.
//
// Roofline: MFMA (int8). Algorithmic work per call = 2*M*N*K operations.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace bl {

constexpr int kBK = 128;            // k per stage
constexpr int kARow = kBK;          // activation bytes per row per stage
constexpr int kBRow = kBK / 4;      // packed weight bytes per row per stage

// WPE: waves per SIMD the register allocation must allow (2 lets two
// workgroups share a CU so that one's barrier gaps are filled by the other).
// SPLIT: the K steps are divided among gridDim.y workgroups per tile (kt_split
// steps each); each adds its exact int32 partial sums into y, which holds
// int32 zeros beforehand, and k_splitk_finalize rescales them afterwards.
// KS: the workgroup holds KS groups of WGM x WGN waves over the same tile;
// group g takes K steps g, g+KS, g+2KS, ... into its own part of each ring
// slot, and the groups' int32 partial sums are added through LDS at the end.
// A tile with few MFMAs per wave then still has KS waves per SIMD to hide
// each other's LDS and VALU latencies, without atomics or extra launches.
template <int BM, int BN, int WGM, int WGN, int STAGES, int WPE, bool SPLIT, int KS>
__global__ __launch_bounds__(64 * WGM * WGN * KS, WPE) void k_gemm(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, int K,
    const uint32_t* __restrict__ Wp, const float* __restrict__ gamma_p, int N,
    float* __restrict__ y, int32_t* __restrict__ acc_out, int kt_split) {
    constexpr int NW = WGM * WGN;               // waves per K group
    static_assert(KS >= 1, "K groups");
    constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int A_STAGE = BM * kARow;
    constexpr int B_STAGE = BN * kBRow;
    constexpr int STAGE = A_STAGE + B_STAGE;
    // Activation rows: BM / 8 load instructions of 8 rows x 128 B. When the
    // waves divide them evenly, wave w takes a block of A_INSTR consecutive
    // ones; otherwise they are dealt round-robin (instruction w + NW*i) and
    // the first A_TOTAL % NW waves take one more.
    constexpr int A_TOTAL = BM / 8;
    constexpr int A_INSTR = (A_TOTAL + NW - 1) / NW;  // most per wave
    constexpr bool A_EVEN = A_TOTAL % NW == 0;
    // Weight rows: 32 rows of 32 B per instruction, spread over the first
    // B_WAVES waves.
    constexpr int B_WAVES = BN / 32 < NW ? BN / 32 : NW;
    constexpr int B_INSTR = BN / 32 / B_WAVES;
    constexpr int B_ROWS = 32 * B_INSTR;         // weight rows loaded per loading wave
    static_assert(TM >= 1 && TN >= 1 && B_INSTR >= 1, "tile shape");
    static_assert(BM % 8 == 0 && NW <= A_TOTAL && B_WAVES * B_ROWS == BN, "tile shape");
    static_assert((A_INSTR + B_INSTR) * (STAGES - 1) < 64, "vmcnt range");

    extern __shared__ __align__(16) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int kg = wave_all / NW;    // K group
    const int wave = wave_all % NW;  // wave within its group
    const int wm0 = (wave % WGM) * WM, wn0 = (wave / WGM) * WN;

    // Tile order: each XCD (workgroups are dealt round-robin to the 8 XCDs)
    // gets a contiguous range of tile ids, walked in groups of 8 row tiles so
    // neighbouring workgroups share activation and weight tiles in its L2.
    const int nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
    const int total = nM * nN;
    const int b = blockIdx.x;
    const int xcd = b % 8, idx = b / 8;
    const int t = xcd * (total / 8) + min(xcd, total % 8) + idx;
    constexpr int G = 8;
    const int group = t / (G * nN);
    const int first_m = group * G;
    const int gsize = min(nM - first_m, G);
    const int bm = first_m + (t % (G * nN)) % gsize;
    const int bn = (t % (G * nN)) / gsize;
    const int m0 = bm * BM, n0 = bn * BN;

    // Thread t < BM fetches the scale of row m0 + t now; the load's latency
    // is hidden behind the main loop, and the epilogue shares it.
    static_assert(BM <= 64 * NW, "one row scale per thread");
    float xs_row = 0.0f;
    if (!SPLIT && tid < BM && m0 + tid < M) xs_row = xs[m0 + tid];

    const int KT = (K + kBK - 1) / kBK;
    const bool k_tail = (K % kBK) != 0;  // last stage holds 64 valid k
    // This workgroup's K steps are global steps kt0 .. kt0 + nk - 1 (nk >= 1).
    // Local step kt covers kt*KS .. kt*KS + KS-1 of them, one per K group; a
    // group whose step lies past the workgroup's range loads its last step
    // again and expands its weights as zeros.
    const int kt0 = SPLIT ? (int)blockIdx.y * kt_split : 0;
    const int nk = SPLIT ? min(kt_split, KT - kt0) : KT;
    const int NK = (nk + KS - 1) / KS;
    auto lstep = [&](int kt) { return kt * KS + kg; };
    constexpr int SLOT = KS * STAGE;  // one ring slot: a stage per K group

    // Stage loads: a wave-uniform base (the tile's first row at this stage's
    // k, in SGPRs) plus a fixed per-lane byte offset, so advancing a stage
    // costs no per-lane arithmetic. Offsets stay below 2^31: at most 127
    // activation rows of K bytes (fewer than M * K) and 511 weight rows of K/4.
    // A instruction i of this wave covers rows 8q .. 8q+7 (q as above); the
    // lane takes row 8q + lane/8, whose LDS slot is physical chunk lane%8.
    const int a_cnt = A_EVEN ? A_INSTR : (A_TOTAL - 1 - wave) / NW + 1;  // wave-uniform
    auto a_q = [&](int i) { return A_EVEN ? wave * A_INSTR + i : wave + NW * i; };
    const int8_t* a_base = xq + (size_t)m0 * K;
    uint32_t a_off[A_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int r = 8 * min(a_q(i), A_TOTAL - 1) + lane / 8;
        const int c = (lane % 8) ^ swz_a(r);
        a_off[i] = (uint32_t)(min(m0 + r, M - 1) - m0) * (uint32_t)K + 16u * c;
    }
    const bool b_loader = B_WAVES == NW || wave < B_WAVES;  // wave-uniform
    const uint8_t* b_base = reinterpret_cast<const uint8_t*>(Wp) + (size_t)n0 * (K / 4);
    uint32_t b_off[B_INSTR];
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
        const int r = min(wave, B_WAVES - 1) * B_ROWS + 32 * i + lane / 2;
        const int c = (lane % 2) ^ swz_b(r);
        b_off[i] = (uint32_t)(min(n0 + r, N - 1) - n0) * (uint32_t)(K / 4) + 16u * c;
    }

    const uint32_t smem_base = (uint32_t)(size_t)(lds_u8_t*)smem;

    // CLEAN (chosen once per workgroup, below): K is a whole number of steps
    // and every K group has the same number of them, so no step is ragged or
    // past the workgroup's range; the masks are then constants and the
    // ragged-step branch is not compiled, which takes most of the scalar
    // control out of the loop (it otherwise rivals the MFMA count when a
    // wave has only two MFMAs per sub-step). Both forms do the same loads,
    // expansions and MFMAs in the same order on such shapes.
    //
    // Ring slots are byte offsets (slot * SLOT) advanced step by step.
    auto next_slot = [](int off) { return off + SLOT == STAGES * SLOT ? 0 : off + SLOT; };

    auto issue = [&](auto clean_c, int kt, int slot) {
        constexpr bool CLEAN = decltype(clean_c)::value;
        const uint32_t st = smem_base + (uint32_t)(slot + kg * STAGE);
        const int ks = CLEAN ? kt0 + lstep(kt) : kt0 + min(lstep(kt), nk - 1);
        const int k0 = ks * kBK;
        const int8_t* ab = a_base + k0;
        const uint8_t* bb = b_base + k0 / 4;
        if (!CLEAN && k_tail && ks == KT - 1) {
            // Last stage of a ragged K (64 valid k): activation chunks 4..7
            // and the second weight chunk would lie past K; they read chunk
            // c - 4 and chunk 0 instead (any valid address: the weights
            // there are expanded as zeros).
#pragma unroll
            for (int i = 0; i < A_INSTR; ++i) {
                if (!A_EVEN && i >= a_cnt) break;
                const int r = 8 * min(a_q(i), A_TOTAL - 1) + lane / 8;
                const bool hi = ((lane % 8) ^ swz_a(r)) >= 4;
                lds_dma16_s(ab, hi ? a_off[i] - 64u : a_off[i], st + 8 * a_q(i) * kARow);
            }
            if (b_loader) {
#pragma unroll
                for (int i = 0; i < B_INSTR; ++i) {
                    const int r = min(wave, B_WAVES - 1) * B_ROWS + 32 * i + lane / 2;
                    const uint32_t c = (uint32_t)((lane % 2) ^ swz_b(r));
                    lds_dma16_s(bb, b_off[i] - 16u * c,
                                st + A_STAGE + (wave * B_ROWS + 32 * i) * kBRow);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < A_INSTR; ++i) {
            if (!A_EVEN && i >= a_cnt) break;
            lds_dma16_s(ab, a_off[i], st + 8 * a_q(i) * kARow);
        }
        if (b_loader) {
#pragma unroll
            for (int i = 0; i < B_INSTR; ++i)
                lds_dma16_s(bb, b_off[i], st + A_STAGE + (wave * B_ROWS + 32 * i) * kBRow);
        }
    };

    // Accumulators hold the NEGATED sums (the weights are expanded as -q).
    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

    const int fr = lane % 32, fg = lane / 32;

    // Fragment reads from the LDS ring slot at byte offset `slot`.
    auto read_b = [&](uint4* bp, int slot) {
        const uint8_t* Bs = smem + slot + kg * STAGE + A_STAGE;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int r = wn0 + 32 * j + fr;
            bp[j] = *reinterpret_cast<const uint4*>(Bs + r * kBRow + 16 * (fg ^ swz_b(r)));
        }
    };
    // Last stage of a K that is not a multiple of 128: the upper 64 k (lane
    // group 1) lie past K, so that group's codes are replaced by code 1
    // (weight 0) when they are expanded. Applied at expansion, not at the
    // LDS read, so the read need not complete right after the barrier.
    auto keep_mask = [&](auto clean_c, int kt) -> uint32_t {
        if constexpr (decltype(clean_c)::value) return 0xFFFFFFFFu;
        if (KS > 1 && lstep(kt) >= nk) return 0u;
        return (k_tail && kt0 + lstep(kt) == KT - 1 && fg) ? 0u : 0xFFFFFFFFu;
    };
    auto read_a = [&](v4i* af, int slot, int s) {
        const uint8_t* As = smem + slot + kg * STAGE;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm0 + 32 * i + fr;
            af[i] = *reinterpret_cast<const v4i*>(As + r * kARow + 16 * ((4 * fg + s) ^ swz_a(r)));
        }
    };
    auto expand = [&](v4i* bf, const uint4* bp, int s, uint32_t keep) {
        const uint32_t fill = 0x55555555u & ~keep;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint32_t w = s == 0 ? bp[j].x : s == 1 ? bp[j].y : s == 2 ? bp[j].z : bp[j].w;
            bf[j] = expand_word_neg((w & keep) | fill);
        }
    };

    // Pipeline. Stage kt+STAGES-1 is issued in the middle of step kt, right
    // after a barrier that (a) follows this wave's wait for stage kt+1, so
    // stage kt+1 is visible to every wave, and (b) proves every wave is done
    // with step kt-1, whose buffer is the one being refilled. Step kt+1's
    // first fragments are then read during the second half of step kt, so
    // the matrix cores never wait on LDS at a step boundary.
    // Loads per stage: this wave's activation instructions (A_INSTR, or one
    // fewer for the later waves of an uneven deal), plus B_INSTR for the
    // weight-loading waves.
    auto wait_for = [&](auto s_const, int after) {
        constexpr int S = decltype(s_const)::value;
        const bool full = A_EVEN || a_cnt == A_INSTR;
        if (b_loader) {
            if (full) wait_stages<A_INSTR + B_INSTR, S>(after);
            else wait_stages<A_INSTR - 1 + B_INSTR, S>(after);
        } else {
            if (full) wait_stages<A_INSTR, S>(after);
            else wait_stages<(A_INSTR > 1 ? A_INSTR - 1 : 0), S>(after);
        }
    };
    static_assert(STAGES >= 3, "pipeline depth");
    auto run = [&](auto clean_c) {
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            if (st < NK) issue(clean_c, st, st * SLOT);
        // Stage 0 landed: STAGES-2 later stages may still be in flight.
        {
            const int after = min(STAGES - 2, NK - 1);
            wait_for(std::integral_constant<int, STAGES - 2>(), after);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        // Operand registers alternate instead of being copied: sub-step s uses
        // the fragment pair of parity s % 2 while the next sub-step's is read into
        // the other (four sub-steps, so each K step starts on pair 0), and the
        // packed weights of step kt and kt + 1 alternate between two buffers as
        // the K loop runs two steps per trip.
        uint4 bpA[TN], bpB[TN];
        v4i a0[TM], a1[TM], b0[TN], b1[TN];
        // Slots of steps kt, kt + 1 and kt + STAGES - 1 (= kt - 1).
        int slot0 = 0, slot1 = SLOT, slot_w = (STAGES - 1) * SLOT;
        read_b(bpA, slot0);
        read_a(a0, slot0, 0);
        expand(b0, bpA, 0, keep_mask(clean_c, 0));

        auto substep = [&](auto s_const, auto steady_c, int kt, bool more_rt,
                           const uint4 (&bp)[TN], uint4 (&bpn)[TN], const v4i (&ac)[TM],
                           const v4i (&bc)[TN], v4i (&an)[TM], v4i (&bn)[TN]) {
            constexpr int s = decltype(s_const)::value;
            constexpr bool STEADY = decltype(steady_c)::value;
            const bool more = STEADY || more_rt;
            // Next fragments: same step for s < 3, else the first of kt+1.
            if (s < 3) {
                read_a(an, slot0, s + 1);
                expand(bn, bp, s + 1, keep_mask(clean_c, kt));
            } else if (more) {
                read_a(an, slot1, 0);
                expand(bn, bpn, 0, keep_mask(clean_c, kt + 1));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] =
                        __builtin_amdgcn_mfma_i32_32x32x32_i8(ac[i], bc[j], acc[i][j], 0, 0, 0);
            // The next sub-step's LDS fragment reads go first, so they have a
            // whole sub-step of MFMAs to land; the expansion arithmetic is
            // interleaved with the MFMAs.
            __builtin_amdgcn_sched_group_barrier(0x100, TM, 0);
#pragma unroll
            for (int q = 0; q < TM * TN; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            if (s == 1 && more) {
                // Stage kt+1 landed once the stages issued after it are the
                // only loads outstanding.
                const int after = STEADY ? STAGES - 3 : min(STAGES - 3, NK - 2 - kt);
                wait_for(std::integral_constant<int, STAGES - 3>(), after);
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (STEADY || kt + STAGES - 1 < NK) issue(clean_c, kt + STAGES - 1, slot_w);
                read_b(bpn, slot1);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        auto kstep = [&](auto steady_c, int kt, const uint4 (&bp)[TN], uint4 (&bpn)[TN]) {
            const bool more = kt + 1 < NK;
            using S0 = std::integral_constant<int, 0>;
            using S1 = std::integral_constant<int, 1>;
            using S2 = std::integral_constant<int, 2>;
            using S3 = std::integral_constant<int, 3>;
            substep(S0(), steady_c, kt, more, bp, bpn, a0, b0, a1, b1);
            substep(S1(), steady_c, kt, more, bp, bpn, a1, b1, a0, b0);
            substep(S2(), steady_c, kt, more, bp, bpn, a0, b0, a1, b1);
            substep(S3(), steady_c, kt, more, bp, bpn, a1, b1, a0, b0);
            slot_w = slot0;
            slot0 = slot1;
            slot1 = next_slot(slot1);
        };
        // Steady state: while the STAGES - 1 steps after kt exist, every bound
        // in the loop body is a constant (a next step exists, stage kt +
        // STAGES - 1 is issued, STAGES - 3 stages stay in flight at the wait),
        // so the body carries no scalar compare-and-branch chains; the last
        // steps take the general body. Both do the same loads, waits and
        // MFMAs in the same order.
        int kt = 0;
        for (; kt + 1 < NK - (STAGES - 1); kt += 2) {
            kstep(std::true_type(), kt, bpA, bpB);
            kstep(std::true_type(), kt + 1, bpB, bpA);
        }
        for (; kt < NK; kt += 2) {
            kstep(std::false_type(), kt, bpA, bpB);
            if (kt + 1 < NK) kstep(std::false_type(), kt + 1, bpB, bpA);
        }
    };
    if (!k_tail && nk % KS == 0)
        run(std::true_type());
    else
        run(std::false_type());

    // Epilogue. C layout of the 32x32 MFMA: lane l, register v holds row
    // 8*(v/4) + 4*(l/32) + v%4 (token) and column l%32 (output feature).
    //
    // The tile's row scales reach every lane through LDS (a region past the
    // ring): a global load issued among the output stores would wait for
    // those stores as well (vector loads and stores retire through one
    // counter in issue order), one round trip per row. Split K has no scales
    // here (k_splitk_finalize applies them) and no such region.
    float* xs_lds = reinterpret_cast<float*>(smem + STAGES * SLOT);
    if constexpr (KS > 1) {
        // Groups 1..KS-1 hand their partial sums to group 0 through the ring
        // (free once every wave has passed this barrier), one int32 per lane
        // per accumulator register: consecutive lanes, consecutive words.
        constexpr int PER_WAVE = TM * TN * 16 * kWave;
        static_assert((KS - 1) * NW * PER_WAVE * 4 <= STAGES * SLOT, "reduction space");
        int32_t* red = reinterpret_cast<int32_t*>(smem);
        __syncthreads();
        if (kg > 0) {
            int32_t* dst = red + ((kg - 1) * NW + wave) * PER_WAVE + lane;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) dst[((i * TN + j) * 16 + v) * kWave] = acc[i][j][v];
        }
        if (!SPLIT && tid < BM) xs_lds[tid] = xs_row;
        __syncthreads();
        if (kg > 0) return;
#pragma unroll 1
        for (int g = 1; g < KS; ++g) {
            const int32_t* src = red + ((g - 1) * NW + wave) * PER_WAVE + lane;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] += src[((i * TN + j) * 16 + v) * kWave];
        }
    } else if constexpr (!SPLIT) {
        if (tid < BM) xs_lds[tid] = xs_row;
        __syncthreads();
    }
    if constexpr (SPLIT) {
        int32_t* yi = reinterpret_cast<int32_t*>(y);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm0 + 32 * i + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
                if (m < M) {
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int n = n0 + wn0 + 32 * j + (lane % 32);
                        if (n < N)
                            __hip_atomic_fetch_add(yi + (size_t)m * N + n, -acc[i][j][v],
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }
    const float gm = *gamma_p;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = wm0 + 32 * i + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
            const int m = m0 + r;
            if (m < M) {
                const float sc = xs_lds[r] * gm;
                float* yrow = y + (size_t)m * N;
                int32_t* arow = acc_out ? acc_out + (size_t)m * N : nullptr;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int n = n0 + wn0 + 32 * j + (lane % 32);
                    if (n < N) {
                        const int32_t a = -acc[i][j][v];
                        // The output is not read again here: keep it out of
                        // the L2 that holds the operand tiles (plain stores
                        // measured 0-9% slower on every prefill shape).
                        __builtin_nontemporal_store((float)a * sc, yrow + n);
                        if (arow) arow[n] = a;
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Split-K helpers: int32 zeros into y before the partial sums are added, and
// the fp32 rescale in place afterwards (y[m][n] = acc * (x_scale[m] * gamma),
// the same product and rounding as the direct epilogue).
__global__ __launch_bounds__(256) void k_splitk_zero(int32_t* __restrict__ y, size_t total) {
    const size_t stride = (size_t)gridDim.x * 256;
    const size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x;
    if ((reinterpret_cast<uintptr_t>(y) & 15) == 0) {
        int4* y4 = reinterpret_cast<int4*>(y);
        for (size_t i = i0; i < total / 4; i += stride) y4[i] = make_int4(0, 0, 0, 0);
        for (size_t i = total / 4 * 4 + i0; i < total; i += stride) y[i] = 0;
    } else {
        for (size_t i = i0; i < total; i += stride) y[i] = 0;
    }
}

__global__ __launch_bounds__(256) void k_splitk_finalize(float* __restrict__ y,
                                                         const float* __restrict__ xs,
                                                         const float* __restrict__ gamma_p,
                                                         int32_t* __restrict__ acc_out, int N,
                                                         size_t total) {
    const float gm = *gamma_p;
    const size_t stride = (size_t)gridDim.x * 256;
    const size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x;
    const bool vec = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(acc_out) & 15) == 0;
    if (vec) {
        // Four consecutive elements of one row.
        for (size_t i = i0; i < total / 4; i += stride) {
            const int4 a = reinterpret_cast<const int4*>(y)[i];
            const float sc = xs[(4 * i) / (size_t)N] * gm;
            reinterpret_cast<float4*>(y)[i] =
                make_float4((float)a.x * sc, (float)a.y * sc, (float)a.z * sc, (float)a.w * sc);
            if (acc_out) reinterpret_cast<int4*>(acc_out)[i] = a;
        }
        return;
    }
    for (size_t i = i0; i < total; i += stride) {
        const int32_t a = reinterpret_cast<const int32_t*>(y)[i];
        y[i] = (float)a * (xs[i / (size_t)N] * gm);
        if (acc_out) acc_out[i] = a;
    }
}

template <int BM, int BN, int WGM, int WGN, int STAGES, int WPE, bool SPLIT = false, int KS = 1>
static hipError_t launch_gemm_tile(const int8_t* xq, const float* xs, int M, int K,
                                   const uint32_t* Wp, const float* gamma, int N, float* y,
                                   int32_t* acc, hipStream_t stream, int splits = 1) {
    // The ring (a stage per K group in each slot), then BM row scales for
    // the epilogue.
    constexpr size_t lds =
        (size_t)STAGES * KS * (BM * kARow + BN * kBRow) + (SPLIT ? 0 : BM * 4);
    static_assert(lds <= 160 * 1024, "a workgroup holds at most 160 KiB of LDS");
    auto kern = &k_gemm<BM, BN, WGM, WGN, STAGES, WPE, SPLIT, KS>;
    static std::atomic<uint64_t> lds_set{0};
    {
        hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
        if (e != hipSuccess) return e;
    }
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int KT = (K + kBK - 1) / kBK;
    if (!SPLIT) {
        hipLaunchKernelGGL(kern, dim3(tiles), dim3(64 * WGM * WGN * KS), lds, stream, xq, xs, M,
                           K, Wp, gamma, N, y, acc, KT);
        return hipGetLastError();
    }
    // Even split of the K steps; every split gets at least one step.
    const int per = (KT + splits - 1) / splits;
    const int used = (KT + per - 1) / per;
    const size_t total = (size_t)M * N;
    hipError_t e = launch_splitk_zero(reinterpret_cast<int32_t*>(y), total, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(tiles, used), dim3(64 * WGM * WGN * KS), lds, stream, xq, xs, M,
                       K, Wp, gamma, N, y, acc, per);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_splitk_finalize(y, xs, gamma, acc, N, total, stream);
}

static int splitk_blocks(size_t total) {
    return (int)std::min<size_t>((total / 4 + 255) / 256 + 1, 2048);
}

hipError_t launch_splitk_zero(int32_t* y, size_t total, hipStream_t stream) {
    hipLaunchKernelGGL(k_splitk_zero, dim3(splitk_blocks(total)), dim3(256), 0, stream, y, total);
    return hipGetLastError();
}

hipError_t launch_splitk_finalize(float* y, const float* xs, const float* gamma, int32_t* acc,
                                  int N, size_t total, hipStream_t stream) {
    hipLaunchKernelGGL(k_splitk_finalize, dim3(splitk_blocks(total)), dim3(256), 0, stream, y, xs,
                       gamma, acc, N, total);
    return hipGetLastError();
}

hipError_t launch_gemm(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                       const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream) {
    auto tiles = [&](int bm, int bn) {
        return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    };
    constexpr int kCUs = 256;
    // 128 x 512 tiles: one 8-wave workgroup per CU, each wave all 128 rows by
    // its own 64 columns (no weight column is expanded twice); the fastest
    // per unit of work. 128 x 256 tiles: two 4-wave workgroups per CU (72 KB
    // of LDS each), not tied by barriers, so one's barrier waits and output
    // stores overlap the other's MFMAs. The busiest CU does two 128 x 256
    // units per round of 128 x 512 tiles and one per round of 128 x 256
    // tiles (a CU's pair shares its matrix cores); the larger tile wins ties,
    // as long as it keeps at least half the CUs busy.
    const int64_t t512 = tiles(128, 512), t256 = tiles(128, 256);
    // N a multiple of 320 where 128 x 512 tiles leave CUs idle: 128 x 320
    // tiles of 10 waves, 64 x 64 each. A SIMD then runs at most three such
    // waves against two 128 x 64 waves of the 128 x 512 tile (3/4 of the
    // work), when one round of them covers at least 3/4 of the CUs.
    if (N % 320 == 0) {
        const int64_t t320 = tiles(128, 320);
        if (t512 < t320 && t320 <= kCUs && 4 * t320 >= 3 * kCUs)
            return launch_gemm_tile<128, 320, 2, 5, 3, 3>(xq, xs, M, K, Wp, gamma, N, y, acc,
                                                          stream);
    }
    if (t512 >= kCUs / 2 && 2 * ((t512 + kCUs - 1) / kCUs) <= (t256 + kCUs - 1) / kCUs)
        return launch_gemm_tile<128, 512, 1, 8, 3, 2>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
    if (t256 >= kCUs)
        return launch_gemm_tile<128, 256, 1, 4, 3, 2>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
    // N a multiple of 160 where 128 x 128 tiles spill a few into a second
    // round (at most half a round more): 128 x 160 tiles of two K groups of
    // five 128 x 32 waves, when one round of them covers at least 3/4 of the
    // CUs. The busiest CU then does 128 x 160 outputs instead of two 128 x
    // 128 tiles (512 x 3200 -> 8640: 23.0 against 25.8 us).
    if (N % 160 == 0) {
        const int64_t t128 = tiles(128, 128), t160 = tiles(128, 160);
        if (t128 > kCUs && 2 * t128 <= 3 * kCUs && t160 <= kCUs && 4 * t160 >= 3 * kCUs)
            return launch_gemm_tile<128, 160, 1, 5, 3, 3, false, 2>(xq, xs, M, K, Wp, gamma, N, y,
                                                                    acc, stream);
    }
    if (tiles(128, 128) >= kCUs)
        return launch_gemm_tile<128, 128, 2, 2, 3, 2>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
    // Few tiles (few tokens, or few output features): 64 x 128 tiles. A
    // 4-wave workgroup alone on a CU leaves one wave per SIMD, whose LDS and
    // VALU latencies the matrix cores then wait on; so the workgroup gets two
    // K groups of 4 waves that add their partial sums through LDS (a 4-deep
    // ring where there is at most one tile per CU and K has at least 48
    // steps). With fewer than half as many tiles as CUs, or few tiles and
    // very long K, the K steps are instead split across workgroups until the
    // grid covers every CU (each split keeps at least 8 steps), their exact
    // int32 partial sums added with atomics into y. Integer addition makes
    // every variant bit-identical.
    const int64_t t64 = tiles(64, 128);
    const int KT = (K + kBK - 1) / kBK;
    const int splits = (int)std::min<int64_t>((kCUs + t64 - 1) / t64, std::max(1, KT / 8));
    const bool groups = splits == 1 || (t64 >= kCUs / 2 && (t64 >= 3 * kCUs / 4 || KT <= 128));
    // Long K with at most one tile per CU: two groups with a 4-deep ring,
    // measured with the steady-state loop against four groups with three
    // stages (the choice before it) and a 6-deep ring: 64 x 8192 -> 28672,
    // weights streamed from HBM, 21.7 against 25.2 and 23.0 us; 512 x 8640 ->
    // 3200 25.7 against 29.1 us.
    if (groups && t64 <= kCUs && KT >= 48)
        return launch_gemm_tile<64, 128, 1, 4, 4, 2, false, 2>(xq, xs, M, K, Wp, gamma, N, y, acc,
                                                               stream);
    // At most 64 tokens (one row of tiles), where the split would leave fewer
    // than 24 steps per workgroup while 64 x 64 tiles still cover half the
    // CUs: those tiles with four K groups of two 64 x 32 waves and no split
    // (64 x 3200 -> 8640: 15.2 against 18.2 us, weights streamed from HBM).
    if (M <= 64) {
        const int64_t t6464 = tiles(64, 64);
        if (!groups && (KT + splits - 1) / splits < 24 && 2 * t6464 >= kCUs && t6464 <= kCUs)
            return launch_gemm_tile<64, 64, 1, 2, 3, 2, false, 4>(xq, xs, M, K, Wp, gamma, N, y,
                                                                  acc, stream);
    }
    if (groups)
        return launch_gemm_tile<64, 128, 1, 4, 3, 4, false, 2>(xq, xs, M, K, Wp, gamma, N, y, acc,
                                                               stream);
    // Split K: with many steps per split, K groups inside each workgroup as
    // well (four from 40 steps, two from 24); fewer steps leave too little
    // per group to pay for the LDS reduction.
    // At most 64 tokens, two groups with a 4-deep ring instead of four (64 x
    // 28672 -> 8192 in four splits: 29.8 against 31.6 us).
    const int per = (KT + splits - 1) / splits;
    if (per >= 40 && M <= 64)
        return launch_gemm_tile<64, 128, 1, 4, 4, 2, true, 2>(xq, xs, M, K, Wp, gamma, N, y, acc,
                                                              stream, splits);
    if (per >= 40)
        return launch_gemm_tile<64, 128, 1, 4, 3, 4, true, 4>(xq, xs, M, K, Wp, gamma, N, y, acc,
                                                              stream, splits);
    if (per >= 24)
        return launch_gemm_tile<64, 128, 1, 4, 3, 4, true, 2>(xq, xs, M, K, Wp, gamma, N, y, acc,
                                                              stream, splits);
    return launch_gemm_tile<64, 128, 1, 4, 6, 2, true>(xq, xs, M, K, Wp, gamma, N, y, acc, stream,
                                                       splits);
}

}  // namespace bl
