"""Pins of the oracle's normalised, input-gated fusion (CPU only).

The form is a reading ("Qwen 3.8 Flash-Next Deep Dive…": an undefined
"Projection / Normalization" stage; "Qwen3.8-Flash-Next: …", summary: a
"gating network"): RMS normalisation with a scale gamma, then a sigmoid gate
unit alpha = 1 / (1 + exp(-(sum u e1 + sum v n + b))) scaling W_g, the output
y = residual + e1 + alpha W_g n rounded once to bf16.  The oracle evaluates it
in float64.  The checks use things other than the oracle: the same formulas
in 60-digit decimal arithmetic (Python's ``decimal``, correctly rounded sqrt
and exp), exact rationals for the final rounding, closed forms where the gate
is exactly 1/2 or fully open, unit RMS, power-of-two scale invariance, and a
constructed output whose correct bf16 value differs from the one a rounding
through fp32 gives.
"""
import decimal
from decimal import Decimal as D
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import bf16_bits_to_f32, bf16_midpoint_near, round_to_bf16

U = 2.0 ** -53
CTX = decimal.Context(prec=60)


def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _dec(x):
    return CTX.create_decimal(float(x))


def reference(x, e1v, resv, W, gamma, u, v, b, eps):
    """r, n[d], logit, alpha, y[d] of one token in 60-digit decimal
    arithmetic, from the formulas alone."""
    d = x.size
    S = sum((CTX.multiply(_dec(t), _dec(t)) for t in x), D(0))
    r = CTX.divide(D(1), CTX.sqrt(CTX.add(CTX.divide(S, D(d)), _dec(eps))))
    n = [CTX.multiply(CTX.multiply(_dec(x[j]), r), _dec(gamma[j])) for j in range(d)]
    Z = D(0)
    for j in range(d):
        Z = CTX.add(Z, CTX.add(CTX.multiply(_dec(u[j]), _dec(e1v[j])), CTX.multiply(_dec(v[j]), n[j])))
    logit = CTX.add(Z, _dec(b))
    alpha = CTX.divide(D(1), CTX.add(D(1), CTX.exp(-logit)))
    y = []
    for j in range(d):
        t = CTX.add(_dec(e1v[j]), CTX.multiply(CTX.multiply(alpha, _dec(W[j])), n[j]))
        y.append(CTX.add(_dec(resv[j]), t) if resv is not None else t)
    return r, n, logit, alpha, y


def _inputs(n, d, V=7, seed=0):
    rng = np.random.default_rng(seed)
    e1 = _bf16(rng.standard_normal((V, d)) * 0.02)
    tok = rng.integers(0, V, size=n).astype(np.int32)
    res = _bf16(rng.standard_normal((n, d)))
    return rng, e1, tok, res


# ------------------------------ bf16 rounding --------------------------------

def test_bf16_from_f64_rounds_once_to_nearest_even():
    rng = np.random.default_rng(1)
    x = (rng.choice([-1.0, 1.0], 3000) * rng.random(3000) * np.exp2(rng.integers(-140, 128, 3000))).tolist()
    # exact midpoints between bf16 neighbours, and their float64 neighbours
    for m in (1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.0 * 2 ** -9 * 2 ** -126, (2 - 2 ** -8) * 2.0 ** 127):
        x += [m, np.nextafter(m, 0.0), np.nextafter(m, np.inf), -m]
    x += [0.0, -0.0, 2.0 ** 128, 2.0 ** -134, 2.0 ** -133 * 1.5, 2.0 ** -134 * 1.0000001]
    got = oracle.bf16_rne_f64(np.array(x))
    for xi, g in zip(x, got):
        want = round_to_bf16(Fraction(xi)) if xi != 0 else np.uint16(0x8000 if np.signbit(xi) else 0)
        assert g == want, f"{xi!r}: {g:#06x} != {want:#06x}"
    special = oracle.bf16_rne_f64(np.array([np.inf, -np.inf, np.nan]))
    assert special.tolist() == [0x7F80, 0xFF80, 0x7FC0]


def test_bf16_from_f64_is_not_a_rounding_through_fp32():
    """1 + 2^-8 + 2^-30 lies above the midpoint between 1 and 1 + 2^-7, so it
    rounds up; rounded to fp32 first it would land on the midpoint and tie
    down to 1."""
    x = 1.0 + 2 ** -8 + 2 ** -30
    assert oracle.bf16_rne_f64(np.array([x]))[0] == 0x3F81
    assert oracle.bf16_rne(np.array([x], np.float32))[0] == 0x3F80


# ---------------------------- normalisation factor ---------------------------

@pytest.mark.parametrize("d,eps", [(64, 2.0 ** -4), (520, 2.0 ** -10), (2560, 1e-6), (64, 0.0)])
def test_rms_factor_against_decimal(d, eps):
    rng, e1, tok, _ = _inputs(4, d, seed=d)
    x = rng.integers(-9, 10, size=(4, d)).astype(np.float32)
    z = np.zeros(d, np.float32)
    _, stats, _ = oracle.norm_gate_add(x, tok, e1, z, np.ones(d, np.float32), z, z, 0.0, eps)
    for i in range(4):
        S = int((x[i].astype(np.int64) ** 2).sum())                    # exact
        r = CTX.divide(D(1), CTX.sqrt(CTX.add(CTX.divide(D(S), D(d)), _dec(np.float32(eps)))))
        assert abs(_dec(stats[i, 0]) - r) <= D(4 * U) * r


def test_rms_factor_of_general_values_against_decimal():
    """Values with wide exponents, whose squares' sum rounds in fp32: the
    float64 factor stays within a few float64 ulps of the 60-digit one."""
    d = 2560
    rng, e1, tok, _ = _inputs(3, d, seed=3)
    m = rng.integers(1 << 23, 1 << 24, size=(3, d)).astype(np.float64)
    x = (rng.choice([-1.0, 1.0], (3, d)) * m * np.exp2(rng.integers(-12, 4, (3, d)) - 23)).astype(np.float32)
    z = np.zeros(d, np.float32)
    _, stats, _ = oracle.norm_gate_add(x, tok, e1, z, np.ones(d, np.float32), z, z, 0.0, 1e-6)
    for i in range(3):
        r = reference(x[i], np.zeros(d), None, z, np.ones(d), z, z, 0.0, np.float32(1e-6))[0]
        assert abs(_dec(stats[i, 0]) - r) <= D((d + 8) * U) * r


def _open_gate_y(x, e1, tok, gamma, eps=0.0):
    """y = n exactly: u = v = 0 and b = 200 give alpha = 1 (exp(-200) is
    below half an ulp of 1 in float64), W_g = 1, e1 = 0 and no residual give
    y = 0 + 1 * 1 * n = n."""
    n_tok, d = x.shape
    z = np.zeros(d, np.float32)
    _, stats, y = oracle.norm_gate_add(x, tok, np.zeros_like(e1), np.ones(d, np.float32), gamma, z, z, 200.0, eps)
    return stats, y


def test_normalised_vector_against_decimal_and_unit_rms():
    d = 1040
    rng, e1, tok, _ = _inputs(3, d, seed=11)
    x = (rng.standard_normal((3, d)) * 0.08).astype(np.float32)
    gamma = (0.5 + rng.random(d)).astype(np.float32)
    _, y = _open_gate_y(x, e1, tok, gamma, eps=1e-6)
    for i in range(3):
        _, n, _, _, _ = reference(x[i], np.zeros(d), None, np.ones(d), gamma, np.zeros(d), np.zeros(d), 200.0,
                                  np.float32(1e-6))
        for j in range(0, d, 37):
            assert abs(_dec(y[i, j]) - n[j]) <= D((d + 8) * U) * abs(n[j])
    stats1, y1 = _open_gate_y(x, e1, tok, np.ones(d, np.float32))
    rms = np.sqrt((y1 ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 1e-13)


def test_power_of_two_scaling_leaves_the_output_unchanged():
    """Scaling the sums by 8 scales every float64 partial sum of squares by 64
    exactly, the factor by 1/8 exactly and leaves n, the logit and y
    bit-identical (eps = 0)."""
    d = 1040
    rng, e1, tok, res = _inputs(5, d, seed=12)
    x = (rng.standard_normal((5, d)) * 0.05).astype(np.float32)
    W, gamma, u, v = (rng.random(d).astype(np.float32) for _ in range(4))
    o1, s1, y1 = oracle.norm_gate_add(x, tok, e1, W, gamma, u, v, -0.25, 0.0, res)
    o2, s2, y2 = oracle.norm_gate_add(x * np.float32(8.0), tok, e1, W, gamma, u, v, -0.25, 0.0, res)
    assert np.array_equal(o1, o2) and np.array_equal(y1.view(np.uint64), y2.view(np.uint64))
    assert np.array_equal(s1[:, 1].view(np.uint64), s2[:, 1].view(np.uint64))
    assert np.array_equal((s1[:, 0] / 8.0).view(np.uint64), s2[:, 0].view(np.uint64))


# ---------------------------------- the gate ---------------------------------

@pytest.mark.parametrize("b", [-20.0, -1.5, 0.0, 0.75, 9.0])
def test_sigmoid_of_the_bias_alone(b):
    """u = v = 0: logit = b; W_g = 1, e1 = 0, no residual and the sums x = 1
    with gamma = 1 (so n = 1 exactly, eps = 0) make y = alpha."""
    d = 64
    _, e1, tok, _ = _inputs(2, d, seed=13)
    x = np.ones((2, d), np.float32)
    z = np.zeros(d, np.float32)
    out, stats, y = oracle.norm_gate_add(x, tok, np.zeros_like(e1), np.ones(d, np.float32), np.ones(d, np.float32),
                                         z, z, b, 0.0)
    assert np.all(stats[:, 0] == 1.0) and np.all(stats[:, 1] == b)
    alpha = CTX.divide(D(1), CTX.add(D(1), CTX.exp(-_dec(b))))
    assert np.all(np.abs(y - float(alpha)) <= 4 * U * float(alpha))
    if b == 0.0:
        assert np.all(y == 0.5)


def test_gate_of_one_half_against_decimal():
    """u = v = 0, b = 0: logit = 0 and alpha = 1/2 exactly; every y agrees
    with the 60-digit value and every output is that value rounded once."""
    d = 520
    rng, e1, tok, res = _inputs(4, d, seed=13)
    x = (rng.standard_normal((4, d)) * 0.05).astype(np.float32)
    W = rng.random(d).astype(np.float32)
    gamma = (0.5 + rng.random(d)).astype(np.float32)
    z = np.zeros(d, np.float32)
    out, stats, y = oracle.norm_gate_add(x, tok, e1, W, gamma, z, z, 0.0, 1e-6, res)
    assert np.all(stats[:, 1] == 0)
    e1f, resf = bf16_bits_to_f32(e1[tok]), bf16_bits_to_f32(res)
    for i in range(4):
        _, _, _, alpha, yr = reference(x[i], e1f[i], resf[i], W, gamma, z, z, 0.0, np.float32(1e-6))
        assert alpha == D("0.5")
        for j in range(d):
            mag = abs(float(resf[i, j])) + abs(float(e1f[i, j])) + abs(float(yr[j]) - float(resf[i, j]))
            bound = (d + 16) * U * mag
            assert abs(_dec(y[i, j]) - yr[j]) <= D(bound)
            if not bf16_midpoint_near(float(yr[j]), 2 * bound):
                assert out[i, j] == round_to_bf16(Fraction(yr[j]))


def test_closed_gate_and_zero_gamma_give_e1_plus_residual():
    d = 64
    rng, e1, tok, res = _inputs(8, d, seed=14)
    x = (rng.standard_normal((8, d)) * 0.05).astype(np.float32)
    W, u, v = (rng.random(d).astype(np.float32) for _ in range(3))
    exact = [[Fraction(float(a)) + Fraction(float(c)) for a, c in zip(ra, rc)]
             for ra, rc in zip(bf16_bits_to_f32(e1[tok]), bf16_bits_to_f32(res))]
    want = np.array([[round_to_bf16(q) for q in row] for row in exact], dtype=np.uint16)
    z = np.zeros(d, np.float32)
    out0, _, _ = oracle.norm_gate_add(x, tok, e1, W, np.ones(d, np.float32), z, z, -800.0, 1e-6, res)
    assert np.array_equal(out0, want)                       # alpha = 0 (exp(800) overflows to inf)
    outg, _, _ = oracle.norm_gate_add(x, tok, e1, W, np.zeros(d, np.float32), u, v, 1.5, 1e-6, res)
    assert np.array_equal(outg, want)                       # n = 0


def test_a_nearly_closed_gate_tips_an_exact_midpoint_up():
    """residual = 1 and e1 = 2^-8 put residual + e1 exactly on the midpoint
    between the bf16 values 1 and 1 + 2^-7; the gate alpha = sigmoid(-24)
    adds about 2^-35 (positive W_g and n), which float64 keeps and fp32 would
    lose, so every output is 1 + 2^-7 (0x3F81)."""
    d, V = 256, 3
    rng = np.random.default_rng(15)
    x = (0.5 + 0.5 * rng.random((4, d))).astype(np.float32)
    e1 = np.full((V, d), 0x3B80, np.uint16)                # 2^-8
    res = np.full((4, d), 0x3F80, np.uint16)               # 1.0
    tok = np.array([0, 1, 2, 1], np.int32)
    W = (0.5 + 0.5 * rng.random(d)).astype(np.float32)
    z = np.zeros(d, np.float32)
    out, stats, y = oracle.norm_gate_add(x, tok, e1, W, np.ones(d, np.float32), z, z, -24.0, 0.0, res)
    assert np.all(y > 1.0 + 2 ** -8) and np.all(y - (1.0 + 2 ** -8) < 2 ** -30)
    assert np.all(out == 0x3F81)


def test_gate_logit_and_output_against_decimal():
    d = 2560
    rng, e1, tok, res = _inputs(3, d, seed=16)
    x = (rng.standard_normal((3, d)) * 0.08).astype(np.float32)
    W = rng.random(d).astype(np.float32)
    gamma = (0.5 + rng.random(d)).astype(np.float32)
    u = (rng.standard_normal(d) * 0.3).astype(np.float32)
    v = (rng.standard_normal(d) * 0.02).astype(np.float32)
    b = np.float32(0.75)
    out, stats, y = oracle.norm_gate_add(x, tok, e1, W, gamma, u, v, b, 1e-6, res)
    e1f, resf = bf16_bits_to_f32(e1[tok]), bf16_bits_to_f32(res)
    signs = set()
    for i in range(3):
        r, n, logit, alpha, yr = reference(x[i], e1f[i], resf[i], W, gamma, u, v, b, np.float32(1e-6))
        A = sum(abs(float(u[j]) * float(e1f[i, j])) + abs(float(v[j]) * float(n[j])) for j in range(d))
        assert abs(_dec(stats[i, 0]) - r) <= D((d + 8) * U) * r
        assert abs(_dec(stats[i, 1]) - logit) <= D(4 * d * U * (A + abs(float(b))))
        signs.add(logit > 0)
        for j in range(d):
            mag = abs(float(resf[i, j])) + abs(float(e1f[i, j])) + abs(float(W[j]) * float(n[j]))
            bound = 8 * d * U * mag
            assert abs(_dec(y[i, j]) - yr[j]) <= D(bound)
            if not bf16_midpoint_near(float(yr[j]), 2 * bound):
                assert out[i, j] == round_to_bf16(Fraction(yr[j]))
    assert signs == {True, False}                          # both signs of the logit are exercised


def test_sum_order_is_not_part_of_the_definition():
    """Reversing the columns (and the per-column parameters with them) leaves
    r, the logit and every output within float64 rounding of the original:
    the sums are plain sums."""
    d = 1040
    rng, e1, tok, res = _inputs(3, d, seed=16)
    x = (rng.standard_normal((3, d)) * 0.08).astype(np.float32)
    W, gamma = rng.random(d).astype(np.float32), (0.5 + rng.random(d)).astype(np.float32)
    u, v = (rng.standard_normal(d) * 0.3).astype(np.float32), (rng.standard_normal(d) * 0.02).astype(np.float32)
    o1, s1, y1 = oracle.norm_gate_add(x, tok, e1, W, gamma, u, v, 0.25, 1e-6, res)
    rv = lambda a: np.ascontiguousarray(a[..., ::-1])
    o2, s2, y2 = oracle.norm_gate_add(rv(x), tok, rv(e1), rv(W), rv(gamma), rv(u), rv(v), 0.25, 1e-6, rv(res))
    assert np.allclose(s1, s2, rtol=4 * d * U, atol=0)
    assert np.allclose(y1, rv(y2), rtol=0, atol=1e-13)
