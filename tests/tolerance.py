"""Comparisons of GPU results with the oracle's float64 values under error
bounds derived from the arithmetic (test infrastructure).

Two float64 evaluations of the same sum of m terms in different orders each
lie within (m - 1) u sum|terms| of the exact sum (u = 2^-53), so they differ
by at most 2 (m - 1) u sum|terms|.  A result rounded once from such a value
(to fp32, or to bf16) can then differ from the oracle's rounding only where a
rounding midpoint lies within that bound of the oracle's value, and only by
one step to the value on the other side of that midpoint.  The helpers below
accept exactly those differences, and count them.
"""
from fractions import Fraction

import numpy as np

from tests.exact import round_to_bf16, round_to_f32

U = 2.0 ** -53
MARGIN = 4.0          # safety factor on every derived bound


def sum_bound(m, abs_sum):
    """|difference| of two float64 evaluations of a sum of m terms whose
    absolute values add to abs_sum (one product rounding per term included)."""
    return MARGIN * 2.0 * (np.asarray(m, np.float64) + 1.0) * U * np.asarray(abs_sum, np.float64)


def _either_side(x, bound, rounder):
    return {rounder(Fraction(float(x)) - Fraction(float(bound))), rounder(Fraction(float(x)) + Fraction(float(bound)))}


def assert_f32_rounded_once(got, want64, bound, what):
    """got (fp32) equals want64 rounded to fp32, or, where an fp32 midpoint
    lies within ``bound`` of want64, the rounding of a value within the bound.
    Returns the number of elements that needed the allowance."""
    want64 = np.asarray(want64, np.float64)
    bound = np.broadcast_to(np.asarray(bound, np.float64), want64.shape).reshape(-1)
    want64 = want64.reshape(-1)
    got = np.asarray(got, np.float32).reshape(-1)
    want32 = want64.astype(np.float32)
    nan = np.isnan(want64)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN pattern differs"
    diff = np.nonzero((got.view(np.uint32) != want32.view(np.uint32)) & ~nan)[0]
    for k in diff:
        ok = _either_side(want64[k], bound[k], round_to_f32)
        assert len(ok) > 1 and any(o.view(np.uint32) == got[k].view(np.uint32) for o in ok), \
            f"{what}[{k}]: {got[k]!r} vs {want64[k]!r} (bound {bound[k]:.3g})"
    return diff.size


def assert_f64_close(got, want, bound, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN pattern differs"
    err = np.abs(got - want)[~nan]
    b = np.broadcast_to(np.asarray(bound, np.float64), want.shape)[~nan]
    if err.size == 0:
        return
    assert np.all(err <= b), f"{what}: max error {err.max():.3g}, at bound {b[np.argmax(err - b)]:.3g}"


def assert_bf16_rounded_once(got, want_bits, y64, bound, what):
    """got (bf16 bits) equals the oracle's bf16 rounding of y64 (want_bits),
    or, where a bf16 midpoint lies within ``bound`` of y64, the rounding of
    a value within the bound (then the two are neighbours).  Returns the
    number of elements that needed the allowance."""
    y64 = np.asarray(y64, np.float64)
    bound = np.broadcast_to(np.asarray(bound, np.float64), y64.shape).reshape(-1)
    y64 = y64.reshape(-1)
    got = np.asarray(got, np.uint16).reshape(-1)
    want = np.asarray(want_bits, np.uint16).reshape(-1)
    nan = np.isnan(y64)
    gnan = (got & 0x7FFF) > 0x7F80
    assert np.array_equal(gnan, nan), f"{what}: NaN pattern differs"
    diff = np.nonzero((got != want) & ~nan)[0]
    for k in diff:
        ok = _either_side(y64[k], bound[k], round_to_bf16)
        assert len(ok) > 1 and got[k] in ok, \
            f"{what}[{k}]: {got[k]:#06x} vs {want[k]:#06x} from y = {y64[k]!r} (bound {bound[k]:.3g})"
    return diff.size


def gated_bounds(eN, e1v, resv, W, gamma, u, v, stats):
    """Bounds on the difference between two float64 evaluations of the
    normalised, gated fusion of the sums eN [m][d] (e1v, resv [m][d] float
    values or None, stats the oracle's (r, logit)), returned as (r bound [m],
    logit bound [m], y bound [m][d]):
      S = sum eN^2: d same-sign terms, relative 2 (d + 1) u;
      r = (S/d + eps)^(-1/2): half of S's relative error plus 4 roundings;
      n = eN r gamma: r's relative error plus 2 roundings;
      Z = sum u e1 + v n: 2d terms, plus v n's share of n's error;
      alpha = sigmoid(logit): slope at most 1/4, plus exp's and the
        division's roundings;
      y = residual + e1 + alpha W n: W n's share of alpha's and n's errors
        plus 4 roundings on the terms' sizes."""
    x = np.asarray(eN, np.float64)
    m, d = x.shape
    r, logit = stats[:, 0], stats[:, 1]
    rel_r = 0.5 * MARGIN * 2.0 * (d + 1) * U + MARGIN * 8 * U
    rel_n = rel_r + MARGIN * 4 * U
    n = x * r[:, None] * np.asarray(gamma, np.float64)
    e1v = np.zeros_like(x) if e1v is None else np.asarray(e1v, np.float64)
    resv = np.zeros_like(x) if resv is None else np.asarray(resv, np.float64)
    vn = np.abs(np.asarray(v, np.float64) * n)
    A = (np.abs(np.asarray(u, np.float64) * e1v) + vn).sum(axis=1)
    b_logit = sum_bound(2 * d, A) + vn.sum(axis=1) * rel_n + MARGIN * 4 * U * np.abs(logit)
    with np.errstate(over="ignore"):
        alpha = 1.0 / (1.0 + np.exp(-logit))
    b_alpha = b_logit / 4 + MARGIN * 8 * U
    wn = np.abs(np.asarray(W, np.float64) * n)
    b_y = wn * (b_alpha[:, None] + alpha[:, None] * rel_n) + \
        MARGIN * 8 * U * (np.abs(resv) + np.abs(e1v) + alpha[:, None] * wn)
    return r * rel_r, b_logit, b_y


def project_bound(m, abs_sum):
    """|difference| between the exact sum of m exact products and an fp32
    evaluation of it in any order and association: each of the m - 1
    additions and the final rounding errs by at most 2^-23 relative (a
    rounding to nearest errs by half that; the allowance also covers a
    rounding toward zero), so (m + 1) 2^-23 sum|terms|, plus m 2^-126 for
    partial sums below fp32's normal range."""
    m = np.asarray(m, np.float64)
    return MARGIN * ((m + 1.0) * 2.0 ** -23 * np.asarray(abs_sum, np.float64) + m * 2.0 ** -126)


def assert_project_close(got, y64, abs64, m, what):
    """GPU fp32 projection against the oracle's float64 value (whose own
    error, below (m - 1) 2^-53 sum|terms|, the bound absorbs).  Returns the
    largest error as a fraction of the bound."""
    got = np.asarray(got, np.float64)
    bound = project_bound(m, abs64)
    err = np.abs(got - y64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (f"{what}: error {err[worst]:.3g} above bound {bound[worst]:.3g} at {worst} "
                                  f"(got {got[worst]!r}, want {y64[worst]!r})")
    return float(np.max(err / np.maximum(bound, np.finfo(np.float64).tiny)))
