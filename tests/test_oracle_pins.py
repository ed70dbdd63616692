"""Pins of the CPU oracle against closed forms, invariants, hand-derived
fixtures, exact rational arithmetic and library routines -- never against a
retyped copy of its own formulas. CPU only.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from ternary_weight_linear_quant_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(v):
    return np.float32(v)


# ---------------------------------------------------------------- gamma ----

def test_gamma_closed_form_power_of_two():
    # |W| = 2^-6 everywhere, random signs: the mean |W| is exactly 2^-6.
    rng = np.random.default_rng(1)
    W = np.where(rng.random((7, 64)) < 0.5, -1.0, 1.0).astype(np.float32) / 64
    assert oracle.absmean_gamma(W) == np.float32(2.0 ** -6)


def test_gamma_identity_matrix():
    for K in (16, 64, 1024):
        assert oracle.absmean_gamma(np.eye(K, dtype=np.float32)) == np.float32(1.0 / K)


def test_gamma_equals_exact_rational_mean_when_sums_are_exact():
    # Entries that are multiples of 2^-20 below 1: every fp64 partial sum is
    # exact, so gamma must be the exact mean rounded once to fp32.
    rng = np.random.default_rng(2)
    for N, K in [(3, 16), (5, 48), (17, 64), (64, 256)]:
        ints = rng.integers(-2**20 + 1, 2**20, size=(N, K))
        W = (ints.astype(np.float64) / 2**20).astype(np.float32)
        exact = sum(Fraction(abs(int(v)), 2**20) for v in ints.ravel()) / (N * K)
        assert oracle.absmean_gamma(W) == np.float32(float(exact))


def test_gamma_close_to_exact_mean_general():
    rng = np.random.default_rng(3)
    W = (0.02 * rng.standard_normal((33, 160))).astype(np.float32)
    exact = math.fsum(abs(float(v)) for v in W.ravel()) / W.size
    g = float(oracle.absmean_gamma(W))
    assert abs(g - exact) <= 2 ** -23 * exact


def test_gamma_statistic_gaussian():
    # E|w| = sigma*sqrt(2/pi) for w ~ N(0, sigma^2).
    sigma = 0.02
    W = wl.weights(99, 0, 512, 2048, sigma)
    g = float(oracle.absmean_gamma(W))
    expect = sigma * math.sqrt(2 / math.pi)
    se = sigma * math.sqrt(1 - 2 / math.pi) / math.sqrt(W.size)
    assert abs(g - expect) < 5 * se


def test_rowsums_match_fsum():
    rng = np.random.default_rng(4)
    W = rng.standard_normal((9, 512)).astype(np.float32)
    R = oracle.absmean_rowsums(W)
    for n in range(W.shape[0]):
        ref = math.fsum(abs(float(v)) for v in W[n])
        assert abs(R[n] - ref) <= 512 * 2 ** -52 * ref


def test_gamma_all_zero():
    W = np.zeros((4, 64), np.float32)
    g = oracle.absmean_gamma(W)
    assert g == 0.0
    assert (oracle.ternarize(W, g) == 0).all()


# ------------------------------------------------------ ternary codes ----

def _exact_code(w: float, s: float) -> int:
    """Code from exact rationals: the fp32 quotient exceeds 0.5 (so rounds to
    a nonzero integer) iff |w|/s > 1/2 + 2^-25, the midpoint between 0.5 and
    the next fp32 value; at the midpoint ties go to 0.5, whose nearest even
    integer is 0."""
    r = Fraction(abs(w)) / Fraction(s)
    if r > Fraction(1, 2) + Fraction(1, 2 ** 25):
        return 1 if w > 0 else -1
    return 0


def test_codes_match_exact_rational_rule():
    rng = np.random.default_rng(5)
    W = (0.02 * rng.standard_normal((24, 64))).astype(np.float32)
    g = oracle.absmean_gamma(W)
    s = float(np.float32(g) + np.float32(oracle.WEIGHT_EPS))
    # Put many entries right at the rounding threshold, just below and above.
    half = np.float32(s) * np.float32(0.5)
    near = [half, np.nextafter(half, np.float32(1)), np.nextafter(half, np.float32(0)),
            np.float32(1.5) * np.float32(s), np.float32(s)]
    q = oracle.ternarize(W, g)
    for n in range(W.shape[0]):
        for k in range(W.shape[1]):
            assert q[n, k] == _exact_code(float(W[n, k]), s)
    Wn = np.array([near + [-v for v in near]], dtype=np.float32)
    Wn = np.pad(Wn, ((0, 0), (0, 16 - Wn.shape[1])))
    qn = oracle.ternarize(Wn, g)
    for k in range(Wn.shape[1]):
        assert qn[0, k] == _exact_code(float(Wn[0, k]), s)


def _force_tie(W, pos):
    """Set W[pos] so that fl32(W[pos]/(gamma+eps)) == 0.5 exactly, where gamma
    is recomputed from the modified matrix (fixed-point iteration)."""
    W = W.copy()
    for _ in range(50):
        g = oracle.absmean_gamma(W)
        s = np.float32(g) + np.float32(oracle.WEIGHT_EPS)
        t = np.float32(0.5) * s
        if W[pos] == t:
            return W, g, s
        W[pos] = t
    raise AssertionError("tie construction did not converge")


def test_forced_tie_rounds_to_zero_and_pins_eps():
    rng = np.random.default_rng(6)
    W = (0.02 * rng.standard_normal((16, 64))).astype(np.float32)
    W, g, s = _force_tie(W, (3, 5))
    assert np.float32(W[3, 5]) / s == np.float32(0.5)
    q = oracle.ternarize(W, g)
    assert q[3, 5] == 0              # ties to even; half-away would give 1
    # With s = gamma (no eps) the quotient exceeds 0.5 and the code is 1, so
    # this also pins that eps is added before the division.
    assert np.float32(W[3, 5]) / np.float32(g) > np.float32(0.5)
    # Negative tie.
    Wm = -W
    assert oracle.ternarize(Wm, oracle.absmean_gamma(Wm))[3, 5] == 0


def test_just_above_tie_rounds_away():
    rng = np.random.default_rng(7)
    W = (0.02 * rng.standard_normal((16, 64))).astype(np.float32)
    W, g, s = _force_tie(W, (0, 0))
    for _ in range(50):
        W2 = W.copy()
        W2[0, 0] = np.nextafter(W[0, 0], np.float32(1))
        g2 = oracle.absmean_gamma(W2)
        s2 = np.float32(g2) + np.float32(oracle.WEIGHT_EPS)
        if W2[0, 0] / s2 > np.float32(0.5):
            assert oracle.ternarize(W2, g2)[0, 0] == 1
            return
        W = W2
    raise AssertionError("could not step above the tie")


def test_identity_gives_identity_codes():
    K = 64
    W = np.eye(K, dtype=np.float32)
    p, g, q = oracle.quantize_weights(W)
    assert (q == np.eye(K, dtype=np.int8)).all()


def test_code_invariants_random():
    W = wl.weights(98, 0, 256, 1024)
    g = oracle.absmean_gamma(W)
    q = oracle.ternarize(W, g)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    nz = q != 0
    assert (np.sign(W[nz]) == q[nz]).all()
    # Monotone in |W|: every nonzero code has |W| above every zero code's |W|.
    assert np.abs(W[nz]).min() > np.abs(W[~nz]).max()
    # Odd symmetry with the same gamma (|-W| = |W|).
    assert oracle.absmean_gamma(-W) == g
    assert (oracle.ternarize(-W, g) == -q).all()
    # Clipping: huge entries still map to +-1.
    W2 = W.copy()
    W2[0, :4] = [1e3, -1e3, 50.0, -50.0]
    q2 = oracle.ternarize(W2, oracle.absmean_gamma(W2))
    assert q2[0, :4].tolist() == [1, -1, 1, -1]


def test_zero_fraction_gaussian():
    # For Gaussian W, |w| <= gamma/2 with gamma = sigma*sqrt(2/pi) has
    # probability erf(1/(2*sqrt(pi))) = 0.31006.
    W = wl.weights(97, 0, 512, 2048)
    q = oracle.ternarize(W, oracle.absmean_gamma(W))
    p = math.erf(1 / (2 * math.sqrt(math.pi)))
    frac = float((q == 0).mean())
    sd = math.sqrt(p * (1 - p) / q.size)
    assert abs(frac - p) < 5 * sd + 2e-4   # + gamma sampling error


# ------------------------------------------------------------ packing ----

def test_pack_layout_property():
    # Layout reading: (word >> 2p) & 0x03030303 holds, in byte b, the code+1
    # of weight 16j + 4p + b.
    rng = np.random.default_rng(8)
    q = rng.integers(-1, 2, size=(5, 64)).astype(np.int8)
    P = oracle.pack(q)
    assert P.shape == (5, 4) and P.dtype == np.uint32
    for n in range(5):
        for j in range(4):
            w = int(P[n, j])
            for p in range(4):
                d = (w >> (2 * p)) & 0x03030303
                for b in range(4):
                    assert (d >> (8 * b)) & 0xFF == int(q[n, 16 * j + 4 * p + b]) + 1


def test_pack_special_words():
    assert (oracle.pack(np.zeros((1, 16), np.int8)) == 0x55555555).all()
    assert (oracle.pack(np.ones((1, 16), np.int8)) == 0xAAAAAAAA).all()
    assert (oracle.pack(-np.ones((1, 16), np.int8)) == 0x00000000).all()


def test_pack_roundtrip_and_no_code_three():
    rng = np.random.default_rng(9)
    for N, K in [(1, 16), (3, 64), (37, 2560)]:
        q = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        P = oracle.pack(q)
        assert P.nbytes == N * K // 4
        assert (oracle.unpack(P, K) == q).all()
        pairs = np.stack([(P >> (2 * i)) & 3 for i in range(16)])
        assert not (pairs == 3).any()


def test_pack_exhaustive_single_word():
    # All 3^8 patterns on the first 8 positions x 2 fill patterns for the rest.
    import itertools
    pats = np.array(list(itertools.product((-1, 0, 1), repeat=8)), np.int8)
    for fill in (-1, 1):
        q = np.concatenate([pats, np.full((pats.shape[0], 8), fill, np.int8)], 1)
        assert (oracle.unpack(oracle.pack(q), 16) == q).all()
        q2 = q[:, ::-1].copy()
        assert (oracle.unpack(oracle.pack(q2), 16) == q2).all()


def test_packed_sizes_of_workloads():
    # 2 bits per weight: 8192 x 28672 -> 58.72 MB.
    assert 28672 * 8192 // 4 == 58_720_256
    for _, projs, _ in wl.WORKLOADS.values():
        for _, K, N in projs:
            assert K % 64 == 0


# ---------------------------------------------------- activation quant ----

def _read_act_cases():
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, "act_quant_ties.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            if key == "case":
                cur = {"name": val.strip()}
                cases.append(cur)
            elif key == "x":
                cur["x"] = [float(v) for v in val.split()]
            elif key == "codes":
                cur["codes"] = [int(v) for v in val.split()]
            elif key == "scale":
                cur["scale"] = float(val)
    return cases


@pytest.mark.parametrize("case", _read_act_cases(), ids=lambda c: c["name"])
def test_act_quant_golden_ties(case):
    x = wl.f32_to_bf16_bits(np.array([case["x"]], np.float32))
    assert (wl.bf16_bits_to_f32(x)[0] == np.float32(case["x"])).all()
    xq, sc = oracle.act_quant(x)
    assert xq[0].tolist() == case["codes"]
    assert sc[0] == np.float32(case["scale"])


def test_act_quant_invariants():
    x = wl.activations(96, 0, 8, 2560)
    xq, sc = oracle.act_quant(x)
    xf = wl.bf16_bits_to_f32(x)
    for m in range(8):
        # The absmax element maps to +-127; codes stay in [-127, 127].
        k = int(np.argmax(np.abs(xf[m])))
        assert abs(int(xq[m, k])) == 127 and np.sign(xq[m, k]) == np.sign(xf[m, k])
        assert np.abs(xq[m].astype(int)).max() == 127
        # Dequantised values are within half a step of the input.
        err = np.abs(xq[m].astype(np.float64) * sc[m] - xf[m])
        assert err.max() <= 0.5 * float(sc[m]) * (1 + 1e-6)
    # Per-token: scaling one token leaves the others unchanged.
    x2 = x.copy()
    x2[0] = wl.f32_to_bf16_bits(xf[0] * 4)
    xq2, sc2 = oracle.act_quant(x2)
    assert (xq2[1:] == xq[1:]).all() and (sc2[1:] == sc[1:]).all()
    # Power-of-two scaling keeps the codes and scales the scale.
    for e in (-3, 5):
        xs = wl.f32_to_bf16_bits(xf * np.float32(2.0 ** e))
        xqs, scs = oracle.act_quant(xs)
        assert (xqs == xq).all()
        assert (scs == sc * np.float32(2.0 ** e)).all()
    # Negation flips codes.
    xqn, scn = oracle.act_quant(wl.f32_to_bf16_bits(-xf))
    assert (xqn == -xq).all() and (scn == sc).all()


def test_act_quant_matches_exact_nearest_integer():
    # Codes are the nearest integer to 127*z/absmax except within a hair of a
    # half-integer, where fp32 rounding of the product decides.
    x = wl.activations(95, 0, 4, 512)
    xq, _ = oracle.act_quant(x)
    xf = wl.bf16_bits_to_f32(x)
    for m in range(4):
        a = Fraction(float(np.abs(xf[m]).max()))
        for k in range(512):
            t = Fraction(127) * Fraction(float(xf[m, k])) / a
            fl = math.floor(t)
            frac = t - fl
            if abs(frac - Fraction(1, 2)) < Fraction(1, 10 ** 5):
                assert int(xq[m, k]) in (fl, fl + 1)
            else:
                assert int(xq[m, k]) == (fl + 1 if frac > Fraction(1, 2) else fl)


def test_act_quant_zero_token():
    x = np.zeros((2, 64), np.uint16)
    x[1, 3] = wl.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    xq, sc = oracle.act_quant(x)
    assert (xq[0] == 0).all()
    assert sc[0] == np.float32(1e-5) / np.float32(127)
    assert xq[1, 3] == 127 and sc[1] == np.float32(1) / np.float32(127)


# ------------------------------------------------- fused RMSNorm + quant ----

def test_rmsnorm_gain_one_keeps_codes():
    x = wl.activations(94, 0, 4, 1024)
    ones = wl.f32_to_bf16_bits(np.ones(1024, np.float32))
    xq, sc = oracle.act_quant(x)
    xq2, sc2, rms = oracle.act_quant(x, ones, return_rms=True)
    assert (xq2 == xq).all()
    assert np.allclose(sc2.astype(np.float64) * 1.0, sc / rms, rtol=2e-7)
    twos = wl.f32_to_bf16_bits(np.full(1024, 2.0, np.float32))
    xq3, _ = oracle.act_quant(x, twos)
    assert (xq3 == xq).all()


def test_rmsnorm_constant_token_closed_form():
    for c in (1.0, 2.0 ** -10, 3.0):
        x = wl.f32_to_bf16_bits(np.full((1, 256), c, np.float32))
        ones = wl.f32_to_bf16_bits(np.ones(256, np.float32))
        xq, sc, rms = oracle.act_quant(x, ones, return_rms=True)
        assert (xq == 127).all()
        r = math.sqrt(c * c + float(np.float32(1e-5)))
        assert abs(rms[0] - r) <= 1e-15 * r
        assert sc[0] == np.float32(c / (127 * r))


def test_rmsnorm_dequant_matches_textbook_rmsnorm():
    K = 2560
    x = wl.activations(93, 0, 6, K)
    g = wl.rms_gain(93, 0, K)
    xq, sc, rms = oracle.act_quant(x, g, return_rms=True)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    gf = wl.bf16_bits_to_f32(g).astype(np.float64)
    ref = xf * gf / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + float(np.float32(1e-5)))
    for m in range(6):
        err = np.abs(xq[m] * float(sc[m]) - ref[m])
        assert err.max() <= 0.5 * float(sc[m]) * (1 + 1e-5)
        k = int(np.argmax(np.abs(ref[m])))
        assert abs(int(xq[m, k])) == 127


# ------------------------------------------------------ integer matmul ----

def test_int_matmul_matches_numpy_and_addsub():
    rng = np.random.default_rng(10)
    for M, K, N in [(1, 64, 3), (4, 128, 17), (16, 2560, 40)]:
        xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        q = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        acc = oracle.int_matmul(xq, q)
        ref = xq.astype(np.int64) @ q.astype(np.int64).T
        assert (acc == ref).all()
        assert (oracle.addsub_matmul(xq, q) == acc).all()
        # fp64 matmul of the quantised operands is exact here (< 2^53).
        assert (xq.astype(np.float64) @ q.astype(np.float64).T == acc).all()


def test_int_matmul_brute_force_tiny():
    rng = np.random.default_rng(11)
    xq = rng.integers(-127, 128, size=(3, 16)).astype(np.int8)
    q = rng.integers(-1, 2, size=(4, 16)).astype(np.int8)
    acc = oracle.int_matmul(xq, q)
    for m in range(3):
        for n in range(4):
            plus = sum(int(xq[m, k]) for k in range(16) if q[n, k] == 1)
            minus = sum(int(xq[m, k]) for k in range(16) if q[n, k] == -1)
            assert acc[m, n] == plus - minus


def test_zero_weights_contribute_nothing():
    rng = np.random.default_rng(12)
    xq = rng.integers(-127, 128, size=(4, 256)).astype(np.int8)
    q = rng.integers(-1, 2, size=(8, 256)).astype(np.int8)
    acc = oracle.int_matmul(xq, q)
    zero_cols = np.where((q == 0).all(axis=0))[0]
    q[:, :32] = 0
    acc0 = oracle.int_matmul(xq, q)
    xq2 = xq.copy()
    xq2[:, :32] = rng.integers(-127, 128, size=(4, 32))
    assert (oracle.int_matmul(xq2, q) == acc0).all()
    assert (oracle.int_matmul(xq, np.zeros_like(q)) == 0).all()
    assert (oracle.int_matmul(xq, np.ones_like(q))
            == xq.astype(np.int64).sum(1, keepdims=True)).all()
    del acc, zero_cols


def test_int_matmul_extreme_no_overflow():
    K = 28672
    xq = np.full((1, K), 127, np.int8)
    q = np.ones((2, K), np.int8)
    q[1] = -1
    acc = oracle.int_matmul(xq, q)
    assert acc[0].tolist() == [127 * K, -127 * K]


# ------------------------------------------------------------ epilogue ----

def test_epilogue_against_float64_dequant_matmul():
    W = wl.weights(92, 0, 96, 512)
    x = wl.activations(92, 0, 5, 512)
    _, g, q = oracle.quantize_weights(W)
    xq, sc = oracle.act_quant(x)
    y, acc = oracle.bitlinear(xq, sc, q, g)
    ref = (xq.astype(np.float64) * sc.astype(np.float64)[:, None]) @ \
          (q.astype(np.float64) * float(g)).T
    assert np.all(np.abs(y - ref) <= 1e-6 * np.abs(ref))
    assert ((y == 0) == (acc == 0)).all()


def test_epilogue_one_hot_token():
    W = wl.weights(91, 0, 32, 64)
    _, g, q = oracle.quantize_weights(W)
    x = np.zeros((1, 64), np.float32)
    x[0, 7] = 3.0
    xq, sc = oracle.act_quant(wl.f32_to_bf16_bits(x))
    y, acc = oracle.bitlinear(xq, sc, q, g)
    assert (acc[0] == 127 * q[:, 7]).all()
    assert np.allclose(y[0], 3.0 * q[:, 7] * float(g), rtol=1e-6, atol=0)


# ------------------------------------------------------------ FFN glue ----

def test_relu2_glu_golden():
    rows = []
    with open(os.path.join(GOLDEN, "relu2_glu.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b, h = line.split()
                rows.append((float(a), float(b), int(h, 16)))
    g = np.array([r[0] for r in rows], np.float32)
    u = np.array([r[1] for r in rows], np.float32)
    h = oracle.relu2_glu(g, u)
    assert h.tolist() == [r[2] for r in rows]


def test_relu2_glu_gate_placement():
    # relu(g)^2 * u, not relu(g*u)^2: a negative gate silences the unit.
    g = np.array([-2.0, -2.0], np.float32)
    u = np.array([-3.0, 3.0], np.float32)
    h = wl.bf16_bits_to_f32(oracle.relu2_glu(g, u))
    assert (h == 0).all()


# ------------------------------------------------------------- SwiGLU ----
# SiLU(x) = x * sigmoid(x) = x / (1 + e^-x), times the up projection. Pins:
# values that follow from the definition by hand, not a retyped formula.

def test_swiglu_zero_gate_and_large_gates():
    # SiLU(0) = 0; for x >= 20, 1 - sigmoid(x) < 2.1e-9 is below half an fp32
    # ulp of 1, so SiLU(x) rounds to x and h = bf16(fp32(x * u)).
    g = np.array([0.0, 0.0, 20.0, 24.0, 40.0, 96.0], np.float32)
    u = np.array([1.5, -3.0, 1.0, -0.75, 0.3, 2.0], np.float32)
    h = wl.bf16_bits_to_f32(oracle.swiglu(g, u))
    assert h[0] == 0 and h[1] == 0
    expect = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits((g[2:] * u[2:]).astype(np.float32)))
    assert np.array_equal(h[2:], expect)


def test_swiglu_very_negative_gate_is_nearly_silent():
    # SiLU(-30) = -30 e^-30 / (1 + e^-30) ~ -2.8e-12: the unit is almost off
    # (a swapped sign in the exponent would give about -30).
    h = wl.bf16_bits_to_f32(oracle.swiglu(np.array([-30.0], np.float32),
                                          np.array([1.0], np.float32)))
    assert h[0] < 0 and abs(h[0]) < 1e-11


def test_swiglu_hand_value_at_one():
    # SiLU(1) = 1 / (1 + 1/e) = 0.73105857863...; in [0.5, 1) bf16 steps are
    # 1/256 and 0.73105857863 * 256 = 187.15, so h = 187/256.
    h = wl.bf16_bits_to_f32(oracle.swiglu(np.array([1.0, -1.0], np.float32),
                                          np.array([1.0, 1.0], np.float32)))
    assert h[0] == np.float32(187 / 256)
    # SiLU(-1) = SiLU(1) - 1 = -0.26894142137; bf16 steps of 1/512 in
    # [0.25, 0.5): 0.26894142137 * 512 = 137.70 -> 138/512.
    assert h[1] == np.float32(-138 / 512)


def test_swiglu_minimum_and_monotone_branch():
    # SiLU has one minimum, -0.27846454276 at x = -1.27846454276 (where
    # 1 + x (1 - sigmoid(x)) = 0), and increases to its right.
    x = np.linspace(-6.0, 6.0, 24001, dtype=np.float32)
    h = wl.bf16_bits_to_f32(oracle.swiglu(x, np.ones_like(x))).astype(np.float64)
    i = int(np.argmin(h))
    assert abs(h[i] - (-0.27846454276)) <= 2.0 ** -9
    assert abs(float(x[i]) - (-1.27846454276)) < 0.2   # flat bottom in bf16
    right = h[x > -1.27]
    assert np.all(np.diff(right) >= 0)


# ----------------------------------------------- workload-sized sanity ----

def test_workload_weight_statistics():
    W = wl.weights(2, 0, 6912, 2560)
    p, g, q = oracle.quantize_weights(W)
    assert abs(float(g) - 0.02 * math.sqrt(2 / math.pi)) < 1e-4
    assert abs(float((q == 0).mean()) - 0.31006) < 2e-3
    assert p.nbytes == 6912 * 2560 // 4


def test_outlier_columns_shared_across_tokens():
    x = wl.bf16_bits_to_f32(wl.activations(2, 0, 16, 2560))
    cols = wl.outlier_columns(2, 0, 2560)
    assert len(cols) == 3
    big = np.abs(x).max(axis=0)
    assert set(np.argsort(big)[-3:].tolist()) == set(cols.tolist())


# ------------------------------------------------- binary weights (1 bit) ----
# inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section "Dlaczego
# akurat ternarne, a nie czyste zero-jeden": the original BitNet used binary
# weights, -1 and +1 only. Readings: sign with W >= 0 -> +1, the same absmean
# gamma, one bit per weight.

def test_binarize_sign_rule_and_zeros():
    W = np.array([[-1.5, -1e-30, -0.0, 0.0, 1e-30, 2.0, -np.float32(1e-45), 7.0]], np.float32)
    assert oracle.binarize(W).tolist() == [[-1, -1, 1, 1, 1, 1, -1, 1]]


def test_binary_codes_and_gamma():
    rng = np.random.default_rng(71)
    W = (0.02 * rng.standard_normal((40, 256))).astype(np.float32)
    pk, g, q = oracle.quantize_weights_binary(W)
    assert set(np.unique(q)) <= {-1, 1}
    assert np.array_equal(q == 1, W >= 0)
    assert g == oracle.absmean_gamma(W)


def test_pack_binary_hand_words():
    K = 128
    def word0(q):
        return int(oracle.pack_binary(np.array([q], np.int8))[0, 0])
    alt = [1 if k % 2 == 0 else -1 for k in range(K)]
    assert word0(alt) == 0x00FF00FF          # even k: bytes 0 and 2 (i%4 in {0,2})
    assert word0([1] * K) == 0xFFFFFFFF
    assert word0([-1] * K) == 0
    for k, w in [(0, 0x1), (4, 0x2), (1, 0x100), (3, 0x1000000), (31, 0x80000000)]:
        q = [-1] * K
        q[k] = 1
        assert word0(q) == w, k


def test_pack_binary_layout_property_and_roundtrip():
    rng = np.random.default_rng(72)
    for K in (64, 128, 192, 8640):
        q = np.where(rng.random((5, K)) < 0.5, 1, -1).astype(np.int8)
        pk = oracle.pack_binary(q)
        assert pk.shape == (5, oracle.binary_row_words(K))
        assert pk.shape[1] * 4 % 16 == 0 and pk.shape[1] * 32 >= K
        assert np.array_equal(oracle.unpack_binary(pk, K), q)
        # (w >> p) & 0x01010101 holds the bits of k = 32j+4p .. 32j+4p+3
        for j in range(K // 32):
            w = int(pk[0, j])
            for p in range(8):
                v = (w >> p) & 0x01010101
                for b in range(4):
                    assert ((v >> (8 * b)) & 1) == int(q[0, 32 * j + 4 * p + b] > 0)
        # padding bits (k >= K; every K here is a multiple of 32) are zero
        assert (pk[:, K // 32:] == 0).all()


def test_binary_product_invariant():
    # x = all ones: acc = (#+1) - (#-1) per row.
    rng = np.random.default_rng(73)
    q = np.where(rng.random((7, 192)) < 0.3, 1, -1).astype(np.int8)
    acc = oracle.int_matmul(np.ones((1, 192), np.int8), q)
    assert np.array_equal(acc[0], 2 * (q == 1).sum(1) - 192)


# ------------------------------------------- base-3 storage (1.6 bits) ----
# inferownia.pl, section "Skąd te 1,58 bita": log2(3) bits carry one ternary
# weight; five of them fit one byte (3^5 = 243 <= 256).

def test_base3_hand_bytes():
    def bytes_of(q):
        return oracle.pack_base3(np.array([q], np.int8))[0].tolist()
    assert bytes_of([0] * 5)[:2] == [121, 121]           # 1+3+9+27+81
    assert bytes_of([1] * 5)[0] == 242
    assert bytes_of([-1] * 5)[0] == 0
    assert bytes_of([-1, 0, 1, -1, 0])[0] == 102         # 0 + 3 + 18 + 0 + 81
    assert bytes_of([-1, 0, 1, -1, 0, 1, 1])[:3] == [102, 125, 121]   # tail: 2+6+9+27+81
    assert bytes_of([1, -1, -1, -1, -1])[0] == 2         # least significant digit first


def test_base3_exhaustive_bijection():
    import itertools
    combos = np.array(list(itertools.product([-1, 0, 1], repeat=5)), np.int8)  # 243 rows
    pk = oracle.pack_base3(combos)
    vals = pk[:, 0].astype(int)
    assert sorted(vals.tolist()) == list(range(243))
    assert np.array_equal(oracle.unpack_base3(pk, 5), combos)
    assert (pk[:, 1:] == 121).all()


def test_base3_rows_padding_and_density():
    rng = np.random.default_rng(74)
    for K in (64, 2560, 6912, 8192, 28672, 3200, 8640):
        rb = oracle.base3_row_bytes(K)
        assert rb % 16 == 0 and 5 * rb >= K and rb - (K + 4) // 5 < 16
        assert K < 1000 or 8 * rb / K <= 1.65   # at the workloads' K
        q = rng.integers(-1, 2, size=(3, K), dtype=np.int8)
        pk = oracle.pack_base3(q)
        assert pk.shape == (3, rb) and int(pk.max()) <= 242
        assert np.array_equal(oracle.unpack_base3(pk, K), q)
        assert (pk[:, (K + 4) // 5:] == 121).all()


# ------------------------------------------- straight-through backward ----
# juhe.plus (Habr repost), the section on training after BinaryConnect: the
# forward rounds, the backward passes the gradient straight through. For the
# input that is dx = gamma * dy . q (the forward's rounding treated as the
# identity; the weight scale stays).

def _bf16_bits(a):
    return wl.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_pack_ste_t_bytes_and_layout():
    q = np.zeros((5, 3), np.int8)
    q[:4, 0] = [-1, 0, 1, -1]
    q[:, 1] = 1
    q[:, 2] = 0
    t = oracle.pack_ste_t(q)
    assert t.shape == (3, 16)
    assert t[0, 0] == 0x24                  # codes 0,1,2,0 at bits 0,2,4,6
    assert t[1, 0] == 0xAA and t[1, 1] == 0x56   # n = 4 is +1, n = 5..7 pad (code 1)
    assert (t[2] == 0x55).all()
    assert (t[:, 2:] == 0x55).all()
    rng = np.random.default_rng(81)
    q = rng.integers(-1, 2, size=(37, 11), dtype=np.int8)
    t = oracle.pack_ste_t(q).astype(int)
    for n in range(37):
        for k in range(11):
            assert ((t[k, n // 4] >> (2 * (n % 4))) & 3) == q[n, k] + 1


def test_ste_dx_identity_and_ones():
    rng = np.random.default_rng(82)
    dy = _bf16_bits(rng.standard_normal((3, 40)))
    g = np.float32(0.0173)
    dyf = wl.bf16_bits_to_f32(dy).astype(np.float64)
    eye = np.eye(40, dtype=np.int8)
    assert np.array_equal(oracle.ste_dx(dy, eye, g), (dyf * np.float64(g)).astype(np.float32))
    ones = np.ones((40, 5), np.int8)
    ref = np.array([[math.fsum(row) * float(g)] * 5 for row in dyf], np.float64).astype(np.float32)
    assert np.array_equal(oracle.ste_dx(dy, ones, g), ref)
    assert np.array_equal(oracle.ste_dx(dy, -ones, g), -ref)
    assert (oracle.ste_dx(dy, np.zeros((40, 5), np.int8), g) == 0).all()


def test_ste_dx_brute_force_fractions():
    from fractions import Fraction
    rng = np.random.default_rng(83)
    dy = _bf16_bits(rng.standard_normal((2, 9)) * 3)
    q = rng.integers(-1, 2, size=(9, 4), dtype=np.int8)
    g = np.float32(0.5)          # exact scale: the result is the exact sum, rounded once
    dx = oracle.ste_dx(dy, q, g)
    dyf = wl.bf16_bits_to_f32(dy)
    for m in range(2):
        for k in range(4):
            s = sum(Fraction(float(dyf[m, n])) * int(q[n, k]) for n in range(9)) * Fraction(0.5)
            assert dx[m, k] == np.float32(float(s))


def test_ste_dx_is_the_adjoint_of_the_forward():
    # <dx, x> = gamma * <dy, x . q^T> for any x: pins the transposition.
    rng = np.random.default_rng(84)
    M, N, K = 3, 70, 50
    dy = _bf16_bits(rng.standard_normal((M, N)))
    q = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    x = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    g = np.float32(0.02)
    dx = oracle.ste_dx(dy, q, g).astype(np.float64)
    lhs = float((dx * x).sum())
    yq = oracle.int_matmul(x, q).astype(np.float64)          # x . q^T, [M][N]
    rhs = float(g) * float((wl.bf16_bits_to_f32(dy).astype(np.float64) * yq).sum())
    # each dx element carries one fp32 rounding
    assert abs(lhs - rhs) <= 2.0 ** -23 * float(np.abs(dx * x).sum())
    assert abs(lhs - rhs) <= 1e-3 * abs(rhs)


def test_ste_dx_sum_is_exact_before_rounding():
    # 2^30 + 1 - 2^30: an fp32 running sum loses the 1, the definition keeps it.
    dy = _bf16_bits(np.array([[2.0 ** 30, 1.0, -(2.0 ** 30)]], np.float32))
    q = np.ones((3, 1), np.int8)
    assert oracle.ste_dx(dy, q, np.float32(0.25))[0, 0] == np.float32(0.25)


# The gradient of the latent weights: with the weights' rounding treated as
# the identity, y = x~ . W^T gives dW = dy^T . x~, x~ = x_q * s_x the
# dequantised activations the forward multiplied.

def test_ste_dw_hand_values():
    # dy = [[1], [2]], x_q = [[1, -2], [3, 4]], s_x = [0.5, 0.25]:
    # x~ = [[0.5, -1], [0.75, 1]], dW = 1 * [0.5, -1] + 2 * [0.75, 1] = [2, 1].
    dy = _bf16_bits(np.array([[1.0], [2.0]], np.float32))
    xq = np.array([[1, -2], [3, 4]], np.int8)
    sx = np.array([0.5, 0.25], np.float32)
    assert oracle.ste_dw(dy, xq, sx).tolist() == [[2.0, 1.0]]


def test_ste_dw_one_hot_rows_and_columns():
    rng = np.random.default_rng(85)
    M, N, K = 6, 5, 9
    xq = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    sx = (rng.random(M) * 0.1 + 0.01).astype(np.float32)
    for m0, n0 in [(0, 0), (3, 4), (5, 2)]:
        d = np.zeros((M, N), np.float32)
        d[m0, n0] = 1.0
        dW = oracle.ste_dw(_bf16_bits(d), xq, sx)
        want = (xq[m0].astype(np.float64) * np.float64(sx[m0])).astype(np.float32)
        assert np.array_equal(dW[n0], want)
        assert (np.delete(dW, n0, axis=0) == 0).all()


def test_ste_dw_is_the_adjoint_of_the_forward():
    # <dW, gamma q> = <dy, y> with y the oracle's own forward on ternary
    # weights gamma * q: pins which operand is transposed and where the
    # per-token scale enters, against the integer product and the epilogue.
    rng = np.random.default_rng(86)
    M, N, K = 7, 33, 21
    dy = _bf16_bits(rng.standard_normal((M, N)))
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    sx = (rng.random(M) * 0.05 + 0.001).astype(np.float32)
    q = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    g = np.float32(0.0183)
    dW = oracle.ste_dw(dy, xq, sx).astype(np.float64)
    lhs = float((dW * (np.float64(g) * q)).sum())
    y, _ = oracle.bitlinear(xq, sx, q, g)
    dyf = wl.bf16_bits_to_f32(dy).astype(np.float64)
    rhs = float((dyf * y.astype(np.float64)).sum())
    # each dW and each y element carries one fp32 rounding
    bound = 2.0 ** -23 * (float(np.abs(dW * (np.float64(g) * q)).sum()) +
                          float(np.abs(dyf * y.astype(np.float64)).sum()))
    assert abs(lhs - rhs) <= bound


def test_ste_dw_brute_force_fractions():
    from fractions import Fraction
    rng = np.random.default_rng(87)
    M, N, K = 11, 3, 4
    dy = _bf16_bits(rng.standard_normal((M, N)) * 2)
    xq = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    sx = (rng.random(M) * 0.3).astype(np.float32)
    dW = oracle.ste_dw(dy, xq, sx)
    dyf = wl.bf16_bits_to_f32(dy)
    for n in range(N):
        for k in range(K):
            s = sum(Fraction(float(dyf[m, n])) * Fraction(float(sx[m])) * int(xq[m, k])
                    for m in range(M))
            assert dW[n, k] == np.float32(float(s))


def test_ste_dw_linear_in_dy_and_zero_tokens():
    rng = np.random.default_rng(88)
    M, N, K = 8, 6, 10
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    sx = (rng.random(M) * 0.1).astype(np.float32)
    d = rng.standard_normal((M, N)).astype(np.float32)
    a = oracle.ste_dw(_bf16_bits(d), xq, sx)
    b = oracle.ste_dw(_bf16_bits(-d), xq, sx)
    assert np.array_equal(a, -b)
    two = oracle.ste_dw(_bf16_bits(2 * d), xq, sx)       # powers of two scale exactly
    assert np.array_equal(two, 2 * a)
    xz = xq.copy()
    xz[3] = 0                                            # a token with all-zero codes
    d3 = d.copy()
    d3[3] *= 7
    assert np.array_equal(oracle.ste_dw(_bf16_bits(d3), xz, sx),
                          oracle.ste_dw(_bf16_bits(d), xz, sx))
