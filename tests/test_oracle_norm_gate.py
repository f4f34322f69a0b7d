"""Pins of the oracle's normalised, input-gated fusion (CPU only).

The form is a reading ("Qwen 3.8 Flash-Next Deep Dive…": an undefined
"Projection / Normalization" stage; "Qwen3.8-Flash-Next: …", summary: a
"gating network"): RMS normalisation with a scale gamma, then a sigmoid gate
unit alpha = 1 / (1 + exp(-(u.e1 + v.n + b))) scaling W_g.  The checks use
things other than the oracle: exact integer sums, exact-rational replays of
the stated blocked order (one rounding per operation, square root rounded
correctly by bracketing), closed forms where the gate is exactly 0, 1/2 or 1,
unit RMS of the normalised vector, power-of-two scale invariance, and float64
predictions of the gate's effect.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import bf16_bits_to_f32, f, round_sqrt_f32, round_to_f32


def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _wide(rng, size, emax=20):
    """fp32 values with random signs, exponents in [-emax, emax) and full
    24-bit significands: sums and products of these round."""
    m = rng.integers(1 << 23, 1 << 24, size=size).astype(np.float64)
    e = rng.integers(-emax, emax, size=size)
    s = rng.choice([-1.0, 1.0], size=size)
    return (s * m * np.exp2(e - 23)).astype(np.float32)


def _replay_blocked(group_terms):
    """Exact-rational replay of the blocked order: group_terms[g] is the list
    of (a, b) products of group g, chained with one rounding per fma."""
    gs = []
    for terms in group_terms:
        s = np.float32(0.0)
        for a, b in terms:
            s = round_to_f32(f(a) * f(b) + f(s))
        gs.append(s)
    total = None
    for c in range(0, len(gs), 64):
        p = [gs[c + l] if c + l < len(gs) else np.float32(0.0) for l in range(64)]
        w = 1
        while w < 64:
            for l in range(0, 64, 2 * w):
                p[l] = round_to_f32(f(p[l]) + f(p[l + w]))
            w *= 2
        total = p[0] if total is None else round_to_f32(f(total) + f(p[0]))
    return np.float32(0.0) if total is None else total


# ------------------------------- blocked sums --------------------------------

@pytest.mark.parametrize("d", [8, 64, 512, 520, 1040, 2560])
def test_sum_of_squares_exact_on_integers(d):
    x = np.random.default_rng(d).integers(-64, 65, size=d)
    assert oracle.blocked_sumsq(x.astype(np.float32)) == np.float32(int((x.astype(np.int64) ** 2).sum()))


@pytest.mark.parametrize("d", [8, 64, 512, 520, 1040, 2560])
def test_dot_exact_on_integers(d):
    rng = np.random.default_rng(d + 1)
    a, b, c, e = (rng.integers(-40, 41, size=d) for _ in range(4))
    want = int((a.astype(np.int64) * b + c.astype(np.int64) * e).sum())
    assert oracle.blocked_dot2(*(z.astype(np.float32) for z in (a, b, c, e))) == np.float32(want)


@pytest.mark.parametrize("d,seed", [(64, 0), (520, 1), (1536, 2), (2560, 3)])
def test_sum_of_squares_follows_the_blocked_order(d, seed):
    x = _wide(np.random.default_rng(seed), d)
    want = _replay_blocked([[(x[j], x[j]) for j in range(8 * g, 8 * g + 8)] for g in range(d // 8)])
    got = oracle.blocked_sumsq(x)
    assert got.view(np.uint32) == want.view(np.uint32)


def test_blocked_order_is_observable():
    """The stated order differs from a sequential fp32 sum on these inputs,
    so a different order cannot pass the replay above by accident."""
    differ = 0
    for seed in range(8):
        x = _wide(np.random.default_rng(100 + seed), 1040)
        seq = np.float32(0.0)
        for v in x:
            seq = np.float32(seq + np.float32(v * v))
        differ += oracle.blocked_sumsq(x) != seq
    assert differ >= 6


@pytest.mark.parametrize("d,seed", [(64, 5), (520, 7), (1040, 5)])
def test_dot_follows_the_blocked_order(d, seed):
    rng = np.random.default_rng(seed)
    a, b, c, e = (_wide(rng, d, emax=3) for _ in range(4))
    groups = [[t for j in range(8 * g, 8 * g + 8) for t in ((a[j], b[j]), (c[j], e[j]))] for g in range(d // 8)]
    want = _replay_blocked(groups)
    assert oracle.blocked_dot2(a, b, c, e).view(np.uint32) == want.view(np.uint32)
    swapped = _replay_blocked([[t for j in range(8 * g, 8 * g + 8) for t in ((c[j], e[j]), (a[j], b[j]))]
                               for g in range(d // 8)])
    assert swapped != want                     # the term order inside a group is observable here


# ---------------------------- normalisation factor ---------------------------

def _inputs(n, d, V=7, seed=0):
    rng = np.random.default_rng(seed)
    e1 = _bf16(rng.standard_normal((V, d)) * 0.02)
    tok = rng.integers(0, V, size=n).astype(np.int32)
    res = _bf16(rng.standard_normal((n, d)))
    return rng, e1, tok, res


@pytest.mark.parametrize("d,eps", [(64, 2.0 ** -4), (520, 2.0 ** -10), (2560, 1e-6), (64, 0.0)])
def test_rms_factor_is_correctly_rounded(d, eps):
    rng, e1, tok, _ = _inputs(4, d, seed=d)
    x = rng.integers(-9, 10, size=(4, d)).astype(np.float32)
    z = np.zeros(d, np.float32)
    _, stats, _ = oracle.norm_gate_add(x, tok, e1, z, np.ones(d, np.float32), z, z, 0.0, eps)
    for i in range(4):
        S = Fraction(int((x[i].astype(np.int64) ** 2).sum()))           # exact
        m = round_to_f32(S / d)
        q = round_to_f32(f(m) + f(np.float32(eps)))
        s = round_sqrt_f32(f(q))
        r = round_to_f32(1 / f(s))
        assert stats[i, 0].view(np.uint32) == r.view(np.uint32)


def _unit_gate_y(x, e1, tok, gamma, eps=0.0):
    """y = n exactly: u = v = 0 and b = 200 give alpha = 1 (exp(-200) is 0 in
    fp32), W_g = 1, e1 = 0 and no residual give h = fmaf(1, n, 0) = n."""
    n_tok, d = x.shape
    z = np.zeros(d, np.float32)
    e1z = np.zeros_like(e1)
    _, stats, y = oracle.norm_gate_add(x, tok, e1z, np.ones(d, np.float32), gamma, z, z, 200.0, eps)
    return stats, y


def test_normalised_vector_is_the_stated_products_and_has_unit_rms():
    d = 2560
    rng, e1, tok, _ = _inputs(6, d, seed=11)
    x = (rng.standard_normal((6, d)) * 0.08).astype(np.float32)
    gamma = (0.5 + rng.random(d)).astype(np.float32)
    stats, y = _unit_gate_y(x, e1, tok, gamma)
    r = stats[:, :1]
    assert np.array_equal(y.view(np.uint32), ((x * r).astype(np.float32) * gamma).astype(np.float32).view(np.uint32))
    stats1, y1 = _unit_gate_y(x, e1, tok, np.ones(d, np.float32))
    rms = np.sqrt((y1.astype(np.float64) ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 1e-5)
    # the factor is 1/sqrt(mean of squares), within fp32 rounding
    want = 1.0 / np.sqrt((x.astype(np.float64) ** 2).mean(axis=1))
    assert np.allclose(stats1[:, 0], want, rtol=2e-6, atol=0)


def test_power_of_two_scaling_leaves_the_output_unchanged():
    d = 1040
    rng, e1, tok, res = _inputs(5, d, seed=12)
    x = (rng.standard_normal((5, d)) * 0.05).astype(np.float32)
    W, gamma, u, v = (rng.random(d).astype(np.float32) for _ in range(4))
    o1, s1, y1 = oracle.norm_gate_add(x, tok, e1, W, gamma, u, v, -0.25, 0.0, res)
    o2, s2, y2 = oracle.norm_gate_add(x * np.float32(8.0), tok, e1, W, gamma, u, v, -0.25, 0.0, res)
    assert np.array_equal(o1, o2) and np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(s1[:, 1].view(np.uint32), s2[:, 1].view(np.uint32))
    assert np.array_equal((s1[:, 0] / np.float32(8.0)).view(np.uint32), s2[:, 0].view(np.uint32))


# ---------------------------------- the gate ---------------------------------

def test_gate_of_one_half_is_exact():
    """u = v = 0, b = 0: logit = 0 and alpha = 1/2 exactly, so
    y = res + fmaf(W/2, n, e1) with n taken from the alpha = 1 case."""
    d = 520
    rng, e1, tok, res = _inputs(4, d, seed=13)
    x = (rng.standard_normal((4, d)) * 0.05).astype(np.float32)
    W = rng.random(d).astype(np.float32)
    gamma = (0.5 + rng.random(d)).astype(np.float32)
    z = np.zeros(d, np.float32)
    out, stats, y = oracle.norm_gate_add(x, tok, e1, W, gamma, z, z, 0.0, 1e-6, res)
    assert np.all(stats[:, 1] == 0)
    _, nvec = _unit_gate_y(x, e1, tok, gamma, eps=1e-6)
    e1f = bf16_bits_to_f32(e1[tok])
    resf = bf16_bits_to_f32(res)
    for i in range(4):
        for j in (0, 7, 300, 519):
            h = round_to_f32(f(np.float32(W[j] * np.float32(0.5))) * f(nvec[i, j]) + f(e1f[i, j]))
            want = round_to_f32(f(resf[i, j]) + f(h))
            assert y[i, j].view(np.uint32) == want.view(np.uint32)


def test_closed_gate_and_zero_gamma_give_e1_plus_residual():
    d = 64
    rng, e1, tok, res = _inputs(8, d, seed=14)
    x = (rng.standard_normal((8, d)) * 0.05).astype(np.float32)
    W, u, v = (rng.random(d).astype(np.float32) for _ in range(3))
    want = oracle.bf16_rne((bf16_bits_to_f32(e1[tok]) + bf16_bits_to_f32(res)).astype(np.float32)).reshape(8, d)
    z = np.zeros(d, np.float32)
    out0, _, _ = oracle.norm_gate_add(x, tok, e1, W, np.ones(d, np.float32), z, z, -200.0, 1e-6, res)
    assert np.array_equal(out0, want)                       # alpha = 0
    outg, _, _ = oracle.norm_gate_add(x, tok, e1, W, np.zeros(d, np.float32), u, v, 1.5, 1e-6, res)
    assert np.array_equal(outg, want)                       # n = 0


def test_gate_logit_and_output_match_float64():
    d = 2560
    rng, e1, tok, res = _inputs(6, d, seed=15)
    x = (rng.standard_normal((6, d)) * 0.08).astype(np.float32)
    W = rng.random(d).astype(np.float32)
    gamma = (0.5 + rng.random(d)).astype(np.float32)
    u = (rng.standard_normal(d) * 0.3).astype(np.float32)
    v = (rng.standard_normal(d) * 0.02).astype(np.float32)
    b = 0.75
    out, stats, y = oracle.norm_gate_add(x, tok, e1, W, gamma, u, v, b, 1e-6, res)
    x64 = x.astype(np.float64)
    r64 = 1.0 / np.sqrt((x64 ** 2).mean(axis=1) + 1e-6)
    n64 = x64 * r64[:, None] * gamma
    e64 = bf16_bits_to_f32(e1[tok]).astype(np.float64)
    logit64 = (u * e64).sum(axis=1) + (v * n64).sum(axis=1) + b
    scale = (np.abs(u * e64).sum(axis=1) + np.abs(v * n64).sum(axis=1) + abs(b))
    assert np.all(np.abs(stats[:, 1] - logit64) <= 1e-5 * scale)
    assert np.all(np.abs(logit64) > 0.05)                   # the sign of the logit is exercised
    alpha64 = 1.0 / (1.0 + np.exp(-logit64))
    y64 = bf16_bits_to_f32(res).astype(np.float64) + e64 + alpha64[:, None] * W * n64
    mag = np.abs(bf16_bits_to_f32(res)) + np.abs(e64) + np.abs(W * n64)
    assert np.all(np.abs(y - y64) <= 1e-5 * mag + 1e-30)
    # out is y rounded once to bf16
    assert np.array_equal(out, oracle.bf16_rne(y).reshape(out.shape))


def test_exact_sqrt_rounding_agrees_with_ieee_sqrt():
    """The bracketing helper above agrees with numpy's float32 sqrt (an IEEE
    correctly rounded operation) on random fp32 inputs."""
    rng = np.random.default_rng(16)
    q = np.abs(_wide(rng, 2000))
    for v in q:
        assert round_sqrt_f32(f(v)).view(np.uint32) == np.sqrt(v).view(np.uint32)
