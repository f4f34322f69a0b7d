"""The bounded comparisons of tests.tolerance, exercised on the CPU: a
float64 evaluation of the normalised, gated fusion and of the gate gradient
with numpy's pairwise sums (another order than the oracle's) passes them
against the oracle, and a result off by more than its bound fails them."""
import numpy as np
import pytest

import oracle
from tests.exact import bf16_bits_to_f32
from tests.tolerance import (assert_bf16_rounded_once, assert_f32_rounded_once, assert_f64_close, gated_bounds,
                             sum_bound)


def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _gated_inputs(m=6, d=1040, seed=0):
    rng = np.random.default_rng(seed)
    eN = (rng.standard_normal((m, d)) * 0.08).astype(np.float32)
    e1 = _bf16(rng.standard_normal((m, d)) * 0.02)
    res = _bf16(rng.standard_normal((m, d)))
    W, gamma = rng.random(d).astype(np.float32), (0.5 + rng.random(d)).astype(np.float32)
    u, v = (rng.standard_normal(d) * 0.3).astype(np.float32), (rng.standard_normal(d) * 0.02).astype(np.float32)
    return eN, e1, res, W, gamma, u, v


def _numpy_gated(eN, e1v, resv, W, gamma, u, v, b, eps):
    """The same float64 formulas with numpy's pairwise sums."""
    x = eN.astype(np.float64)
    r = 1.0 / np.sqrt((x * x).sum(axis=1) / x.shape[1] + np.float64(np.float32(eps)))
    n = x * r[:, None] * gamma.astype(np.float64)
    logit = (u * e1v + v * n).sum(axis=1) + np.float64(np.float32(b))
    alpha = 1.0 / (1.0 + np.exp(-logit))
    y = resv + (e1v + alpha[:, None] * W.astype(np.float64) * n)
    return r, logit, y


def test_another_float64_order_passes_the_gated_bounds():
    eN, e1, res, W, gamma, u, v = _gated_inputs()
    ids = np.arange(eN.shape[0], dtype=np.int32)
    out, stats, y = oracle.norm_gate_add(eN, ids, e1, W, gamma, u, v, 0.25, 1e-6, res)
    e1v, resv = bf16_bits_to_f32(e1).astype(np.float64), bf16_bits_to_f32(res).astype(np.float64)
    b_r, b_logit, b_y = gated_bounds(eN, e1v, resv, W, gamma, u, v, stats)
    r, logit, y2 = _numpy_gated(eN, e1v, resv, W, gamma, u, v, 0.25, 1e-6)
    assert_f64_close(r, stats[:, 0], b_r, "r")
    assert_f64_close(logit, stats[:, 1], b_logit, "logit")
    got = oracle.bf16_rne_f64(y2)
    assert assert_bf16_rounded_once(got, out, y, b_y, "out") == 0
    assert np.all(b_y < 1e-9 * (np.abs(resv) + 1))             # the bounds are tiny next to a bf16 step
    with pytest.raises(AssertionError):
        assert_f64_close(logit + 1e-9, stats[:, 1], b_logit, "logit")
    bad = got.copy()
    bad[0, 0] ^= 1
    with pytest.raises(AssertionError):
        assert_bf16_rounded_once(bad, out, y, b_y, "out")


def test_a_midpoint_within_the_bound_allows_the_neighbour():
    y = np.array([[1.0 + 2 ** -8 + 2 ** -40]])                 # just above the midpoint of 1 and 1 + 2^-7
    want = oracle.bf16_rne_f64(y)
    assert want[0, 0] == 0x3F81
    assert assert_bf16_rounded_once(np.array([[0x3F80]], np.uint16), want, y, np.array([[2 ** -30]]), "y") == 1
    with pytest.raises(AssertionError):
        assert_bf16_rounded_once(np.array([[0x3F80]], np.uint16), want, y, np.array([[2 ** -50]]), "y")


def test_another_float64_order_passes_the_gate_gradient_bound():
    rng = np.random.default_rng(3)
    n, d = 700, 16
    rows = np.zeros((n, 16), np.int32)
    rows[5] = -1
    g = _bf16(rng.standard_normal((n, d)))
    eN = rng.standard_normal((n, d)).astype(np.float32)
    eN[5] = np.nan
    _, want64 = oracle.grad_gate(rows, g, eN, with_f64=True)
    valid = rows[:, 0] >= 0
    p = bf16_bits_to_f32(g).astype(np.float64)[valid] * eN[valid].astype(np.float64)
    got = p[::-1].sum(axis=0).astype(np.float32)               # pairwise, reversed
    assert_f32_rounded_once(got, want64, sum_bound(int(valid.sum()), np.abs(p).sum(axis=0)), "dW_g")
    with pytest.raises(AssertionError):
        assert_f32_rounded_once(np.nextafter(got, np.float32(np.inf)), want64,
                                sum_bound(int(valid.sum()), np.abs(p).sum(axis=0)), "dW_g")
