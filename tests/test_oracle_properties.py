"""Oracle checks of two more kinds, CPU only.

T0 -- brute force on tiny inputs: the whole BitLinear forward recomputed in
exact rational arithmetic (fractions for the absmean scale and the
quotients, Python integers for the sums) and compared with the C oracle,
for M, N <= 4 and K in {64, 128}. Where the oracle rounds in fp32, the exact
value must round to the oracle's result or lie within the fp32 rounding of
it; integer results must agree exactly.

T1 -- invariants as property tests (hypothesis): for any small finite input,
the codes are ternary and follow the sign of the weight, activation codes fit
[-127, 127] and reach the bound at the absmax, the packings round-trip, the
product equals the add/subtract identity, and the backward is the adjoint of
the forward.

Sources: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", sections
"„Trenowany od zera”" (absmean, nearest of {-1, 0, +1}), "Skąd te 1,58 bita"
(2-bit and base-3 storage), "Mnożenie? Jakie mnożenie" (add / subtract);
comrad404.com «Метод: как устроен BitNet b1.58» (8-bit activations);
juhe.plus (Habr repost), section «Когда - три лучше двух» and the training
section (straight-through gradient).
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

import oracle
from ternary_weight_linear_quant_amd import workloads as wl

F32 = np.float32


def _exact_gamma(W):
    return sum(Fraction(float(abs(w))) for w in W.ravel()) / W.size


def _round_half_even(fr):
    """Nearest integer to a Fraction, ties to even."""
    f = fr.numerator // fr.denominator
    rem = fr - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


# ------------------------------------------------------------------ T0 ----

@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (2, 3, 64), (4, 4, 128), (3, 2, 128)])
def test_brute_force_pipeline_tiny(M, N, K):
    rng = np.random.default_rng(1000 + 100 * M + 10 * N + K)
    W = (0.02 * rng.standard_normal((N, K))).astype(F32)
    x_bits = wl.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(F32))
    x = wl.bf16_bits_to_f32(x_bits)

    pk, g, q = oracle.quantize_weights(W)
    # gamma: the exact mean of |W| rounds (once, to fp32) to the oracle's
    # gamma up to the fp64 sum's own rounding: within one fp32 ulp.
    gx = _exact_gamma(W)
    assert abs(Fraction(float(g)) - gx) <= Fraction(float(abs(np.spacing(F32(g)))))
    # codes: rne(W / s) with s = fl32(gamma + eps), the quotient's exact
    # value rounded to fp32 first (a correctly rounded division).
    s = F32(g) + F32(oracle.WEIGHT_EPS)
    for n in range(N):
        for k in range(K):
            quo = Fraction(float(F32(W[n, k]) / s))   # one IEEE fp32 division
            # correctly rounded: within half an fp32 ulp of the exact quotient
            assert abs(Fraction(float(W[n, k])) / Fraction(float(s)) - quo) <= \
                Fraction(float(abs(np.spacing(F32(quo))))) / 2
            t = max(-1, min(1, _round_half_even(quo)))
            assert q[n, k] == t

    xq, xs = oracle.act_quant(x_bits)
    for m in range(M):
        a = max(float(np.max(np.abs(x[m]))), float(F32(1e-5)))
        inv = F32(127.0) / F32(a)
        for k in range(K):
            z = Fraction(float(F32(x[m, k]) * inv))       # fp32 product, as defined
            assert xq[m, k] == max(-127, min(127, _round_half_even(z)))
        assert xs[m] == F32(a) / F32(127.0)

    # integer sums with Python ints; the epilogue as an exact rational,
    # rounded once to fp32 by the oracle
    y, acc = oracle.bitlinear(xq, xs, q, g)
    for m in range(M):
        for n in range(N):
            exact = sum(int(xq[m, k]) * int(q[n, k]) for k in range(K))
            assert acc[m, n] == exact
            val = Fraction(exact) * Fraction(float(xs[m])) * Fraction(float(g))
            assert abs(Fraction(float(y[m, n])) - val) <= \
                Fraction(float(np.spacing(F32(abs(float(val)) if val else 1e-38))))


# ------------------------------------------------------------------ T1 ----

finite32 = st.floats(min_value=-4.0, max_value=4.0, allow_nan=False, allow_infinity=False,
                     width=32)


@settings(max_examples=60, deadline=None)
@given(hnp.arrays(np.float32, st.tuples(st.integers(1, 6), st.sampled_from([64, 128])),
                  elements=finite32))
def test_weight_codes_properties(W):
    pk, g, q = oracle.quantize_weights(W)
    assert set(np.unique(q)) <= {-1, 0, 1}
    nz = q != 0
    assert np.all(np.sign(W[nz]) == q[nz])                  # sign follows the weight
    # monotone in |W| within the matrix: a larger |w| never gets code 0 when a
    # smaller one is non-zero
    a = np.abs(W.astype(np.float64)).ravel()
    if nz.any() and (~nz).any():
        assert a[nz.ravel()].min() >= a[(~nz).ravel()].max()
    assert np.array_equal(oracle.unpack(pk, W.shape[1]), q)
    assert np.array_equal(oracle.unpack_base3(oracle.pack_base3(q), W.shape[1]), q)
    assert g >= 0


@settings(max_examples=60, deadline=None)
@given(hnp.arrays(np.float32, st.tuples(st.integers(1, 5), st.sampled_from([64, 192])),
                  elements=finite32))
def test_activation_codes_properties(x):
    bits = wl.f32_to_bf16_bits(x)
    xf = wl.bf16_bits_to_f32(bits)
    xq, xs = oracle.act_quant(bits)
    assert np.abs(xq.astype(int)).max() <= 127
    for m in range(x.shape[0]):
        amax = np.abs(xf[m]).max()
        if amax > 1e-5:
            assert np.abs(xq[m].astype(int)).max() == 127     # the absmax maps to +-127
        assert np.all((xq[m] == 0) | (np.sign(xq[m]) == np.sign(xf[m])))
        assert xs[m] > 0
        # scaling a token by 2 leaves its codes unchanged (exact in bf16),
        # as long as the absmax floor of 1e-5 is not what sets the scale
        if amax > 1e-5:
            xq2, _ = oracle.act_quant(wl.f32_to_bf16_bits((2 * xf[m:m + 1]).astype(F32)))
            assert np.array_equal(xq2[0], xq[m])


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 4), st.integers(1, 6), st.sampled_from([64, 128]), st.integers(0, 2**31))
def test_product_and_backward_properties(M, N, K, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    acc = oracle.int_matmul(xq, q)
    plus = np.where(q[None, :, :] == 1, xq[:, None, :].astype(np.int64), 0).sum(-1)
    minus = np.where(q[None, :, :] == -1, xq[:, None, :].astype(np.int64), 0).sum(-1)
    assert np.array_equal(acc, plus - minus)                # add / subtract identity
    assert np.array_equal(oracle.addsub_matmul(xq, q), acc)
    # binary codes round-trip through the 1-bit packing
    qb = np.where(q >= 0, 1, -1).astype(np.int8)
    assert np.array_equal(oracle.unpack_binary(oracle.pack_binary(qb), K), qb)
    # the straight-through dx is the adjoint of the forward product
    dy = wl.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(F32))
    dx = oracle.ste_dx(dy, q, F32(1.0)).astype(np.float64)
    lhs = float((dx * xq).sum())
    rhs = float((wl.bf16_bits_to_f32(dy).astype(np.float64) * acc).sum())
    assert abs(lhs - rhs) <= 2.0 ** -23 * float(np.abs(dx * xq).sum()) + 1e-12
