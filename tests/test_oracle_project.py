"""Pins for the oracle's projection (CPU only).

The oracle computes y[i][o] = sum over j of P[o][j] * bf16(x[i][j]) in
float64 (plain loop, ascending j).  The pins below fix it by facts other than
that loop: an identity and a non-involutive permutation (each output is one
rounded input, the rounding checked against a rational rounding routine),
integer data whose sums an exact integer matrix product gives, a rank-one
weight whose result has a closed form, and numpy's float64 product of the
same rounded operands within the float64 error bound of two summation orders.
"""
from fractions import Fraction

import numpy as np

import oracle
from tests.exact import round_to_bf16

ONE = 0x3F80          # bf16 1.0


def bf16_bits(a):
    """bf16 bits of values that bf16 holds exactly (checked)."""
    f = np.asarray(a, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), f), "not bf16 values"
    return b


def bf16_values(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_identity_gives_the_bf16_rounding_of_each_input():
    rng = np.random.default_rng(1)
    d = 48
    x = (rng.standard_normal((5, d)) * np.exp2(rng.integers(-20, 20, size=(5, d)))).astype(np.float32)
    x[0, :6] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -(1.0 + 2.0 ** -8), 2.0 ** -130, 0.0, -0.0]   # ties, subnormal
    P = np.zeros((d, d), np.uint16)
    P[np.arange(d), np.arange(d)] = ONE
    y, a = oracle.project(x, P)
    want = bf16_values([[round_to_bf16(Fraction(float(v))) for v in row] for row in x])
    assert np.array_equal(y, want)
    assert np.array_equal(a, np.abs(want))


def test_permutation_routes_each_output_to_its_input_column():
    rng = np.random.default_rng(2)
    d_in, d_out = 40, 24
    x = rng.standard_normal((4, d_in)).astype(np.float32)
    src = (np.arange(d_out) * 7 + 3) % d_in          # output o reads column src[o]; not an involution
    P = np.zeros((d_out, d_in), np.uint16)
    P[np.arange(d_out), src] = ONE
    y, _ = oracle.project(x, P)
    want = bf16_values([[round_to_bf16(Fraction(float(row[c]))) for c in src] for row in x])
    assert np.array_equal(y, want)


def test_integer_data_gives_the_exact_integer_product():
    rng = np.random.default_rng(3)
    n, d_in, d_out = 6, 200, 33
    xi = rng.integers(-255, 256, size=(n, d_in))
    Pi = rng.integers(-255, 256, size=(d_out, d_in))
    y, a = oracle.project(xi.astype(np.float32), bf16_bits(Pi))
    assert np.array_equal(y, (xi @ Pi.T).astype(np.float64))
    assert np.array_equal(a, (np.abs(xi) @ np.abs(Pi).T).astype(np.float64))


def test_rank_one_weight_has_a_closed_form():
    """P[o][j] = c_o * 2^(j mod 3) and x of powers of two: every term and
    partial sum is exact, y[i][o] = c_o * sum_j 2^(j mod 3) x[i][j]."""
    rng = np.random.default_rng(4)
    n, d_in, d_out = 3, 30, 10
    x = np.exp2(rng.integers(-6, 6, size=(n, d_in))) * rng.choice([-1.0, 1.0], size=(n, d_in))
    c = rng.integers(1, 16, size=d_out).astype(np.float64)
    w = np.exp2(np.arange(d_in) % 3).astype(np.float64)
    P = bf16_bits(np.outer(c, w))
    y, _ = oracle.project(x.astype(np.float32), P)
    s = np.array([sum(Fraction(float(w[j])) * Fraction(float(x[i, j])) for j in range(d_in)) for i in range(n)])
    want = np.array([[float(Fraction(float(co)) * si) for co in c] for si in s])
    assert np.array_equal(y, want)


def test_random_data_matches_numpy_within_the_float64_bound():
    rng = np.random.default_rng(5)
    n, d_in, d_out = 7, 256, 96
    x = (rng.standard_normal((n, d_in)) * 0.05).astype(np.float32)
    P = (rng.standard_normal((d_out, d_in)).astype(np.float32) / 16).view(np.uint32)
    P = (P >> 16).astype(np.uint16)
    y, a = oracle.project(x, P)
    xb = bf16_values([[round_to_bf16(Fraction(float(v))) for v in row] for row in x])
    want = xb @ bf16_values(P).T
    bound = 2.0 * (d_in + 1) * 2.0 ** -53 * a
    assert np.all(np.abs(y - want) <= bound)
    assert np.allclose(a, np.abs(xb) @ np.abs(bf16_values(P)).T, rtol=1e-13, atol=0)
    assert np.all(a >= np.abs(y))


def test_ragged_shapes_and_empty_batch():
    x = np.ones((0, 64), np.float32)
    y, a = oracle.project(x, np.zeros((32, 64), np.uint16))
    assert y.shape == (0, 32) and a.shape == (0, 32)
    x = np.arange(3 * 8, dtype=np.float32).reshape(3, 8)
    P = np.zeros((5, 8), np.uint16)
    P[:, -1] = ONE                                     # every output reads the last column
    y, _ = oracle.project(x, P)
    assert np.array_equal(y, np.repeat(x[:, -1:].astype(np.float64), 5, axis=1))
