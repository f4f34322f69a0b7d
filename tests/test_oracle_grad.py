"""Pins of the oracle's gradients (CPU only).

The reference is torch autograd in float64 on the forward written with torch
ops (embedding_bag sum, gate, residual) - a library derivative, independent
of the oracle's C code - exact where every value is a small dyadic number,
and within a rounding bound otherwise; plus exact-rational replays of the
specified fp32 summation order of the table and e1 gradients on sampled
elements, and exact rational sums for the gate gradient (a plain sum, defined
with no order, rounded once to fp32).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.exact import bf16_bits_to_f32, f, round_to_f32

K = 16


def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _case(n=96, R=61, V=37, d=24, seed=0, dyadic=True):
    rng = np.random.default_rng(seed)
    offs = synth.ragged_offsets([n // 3, n - n // 3])
    toks = synth.tokens(seed + 100, n, V, 1.1)
    rows = oracle.hash_rows(toks, offs, R)          # small R: many repeated rows
    if dyadic:
        g = _bf16(rng.integers(-8, 9, size=(n, d)).astype(np.float32) / 4)
        W = (rng.integers(0, 8, size=d) / 8).astype(np.float32)
        T = rng.integers(-4, 5, size=(R, d)).astype(np.float64)
    else:
        g = _bf16(rng.standard_normal((n, d)).astype(np.float32))
        W = rng.random(d).astype(np.float32)
        T = rng.standard_normal((R, d))
    e1 = rng.standard_normal((V, d))
    return toks, rows, g, W, T, e1


def _autograd(toks, rows, g, W, T, e1, valid=None):
    n = toks.size
    Tt = torch.tensor(T, dtype=torch.float64, requires_grad=True)
    e1t = torch.tensor(e1, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W.astype(np.float64), requires_grad=True)
    r = torch.tensor(np.where(rows < 0, 0, rows).astype(np.int64))
    eN = torch.nn.functional.embedding_bag(r, Tt, mode="sum")
    h = Wt * eN + e1t[torch.tensor(toks.astype(np.int64))]
    gt = torch.tensor(bf16_bits_to_f32(g).astype(np.float64))
    if valid is not None:
        gt = gt * torch.tensor(valid.astype(np.float64))[:, None]
    (h * gt).sum().backward()
    return Tt.grad.numpy(), e1t.grad.numpy(), Wt.grad.numpy(), eN.detach().numpy()


def test_table_and_e1_grads_equal_autograd_exactly_on_dyadic_values():
    toks, rows, g, W, T, e1 = _case()
    dT, de1, dW, eN = _autograd(toks, rows, g, W, T, e1)
    q, got = oracle.grad_table(rows, W, g)
    assert np.array_equal(q, np.unique(rows))
    assert np.array_equal(got.astype(np.float64), dT[q])
    assert np.all(np.delete(dT, q, axis=0) == 0)
    qt, got_e1 = oracle.grad_e1(toks, rows, g)
    assert np.array_equal(qt, np.unique(toks))
    assert np.array_equal(got_e1.astype(np.float64), de1[qt])
    got_w = oracle.grad_gate(rows, g, eN.astype(np.float32))
    assert np.array_equal(got_w.astype(np.float64), dW)


def test_grads_within_fp32_rounding_of_autograd_on_general_values():
    toks, rows, g, W, T, e1 = _case(n=300, R=97, V=53, d=40, seed=3, dyadic=False)
    dT, de1, dW, eN = _autograd(toks, rows, g, W, T, e1)
    eN32 = eN.astype(np.float32)
    dW_ref = (bf16_bits_to_f32(g).astype(np.float64) * eN32.astype(np.float64)).sum(axis=0)
    q, got = oracle.grad_table(rows, W, g)
    mags = np.zeros_like(dT)
    np.add.at(mags, rows.ravel(), np.repeat(np.abs(bf16_bits_to_f32(g).astype(np.float64)), K, axis=0) * W)
    cnt = np.bincount(rows.ravel(), minlength=dT.shape[0])[:, None]
    assert np.all(np.abs(got - dT[q]) <= (cnt[q] + 1) * 2.0 ** -23 * mags[q] + 1e-30)
    qt, got_e1 = oracle.grad_e1(toks, rows, g)
    assert np.allclose(got_e1, de1[qt], rtol=0, atol=1e-4)
    got_w, got_w64 = oracle.grad_gate(rows, g, eN32, with_f64=True)
    mag_w = (np.abs(bf16_bits_to_f32(g).astype(np.float64)) * np.abs(eN32.astype(np.float64))).sum(axis=0)
    n = toks.size
    assert np.all(np.abs(got_w64 - dW_ref) <= 2 * n * 2.0 ** -53 * mag_w)    # two float64 sums of the same terms
    assert np.array_equal(got_w, got_w64.astype(np.float32))                   # rounded once to fp32


def test_table_grad_is_the_specified_fp32_fma_chain():
    toks, rows, g, W, T, e1 = _case(n=200, R=31, d=16, seed=5, dyadic=False)
    q, got = oracle.grad_table(rows, W, g)
    gf = bf16_bits_to_f32(g)
    flat = rows.ravel()
    for qi in (0, len(q) // 2, len(q) - 1):
        r = q[qi]
        for j in (0, 7, 15):
            acc = np.float32(0.0)
            for t in np.nonzero(flat == r)[0]:                 # ascending positions
                acc = round_to_f32(f(W[j]) * f(gf[t // K, j]) + f(acc))
            assert acc.view(np.uint32) == got[qi, j].view(np.uint32)


def test_e1_grad_follows_the_specified_order():
    toks, rows, g, W, T, e1 = _case(n=600, R=97, V=11, d=8, seed=6, dyadic=False)
    gf = bf16_bits_to_f32(g)
    qt, got = oracle.grad_e1(toks, rows, g)
    for qi in range(len(qt)):
        for j in (0, 5):
            acc = np.float32(0.0)
            for i in np.nonzero(toks == qt[qi])[0]:
                acc = round_to_f32(f(acc) + f(gf[i, j]))
            assert acc.view(np.uint32) == got[qi, j].view(np.uint32)


def test_gate_grad_is_the_exact_sum_rounded_once():
    """On values whose float64 partial sums are exact (bf16 integers times
    fp32 values with few significant bits), dW_g is the exact rational sum
    rounded once to fp32, whatever order a fp32 chain would have taken."""
    rng = np.random.default_rng(9)
    n, d = 700, 12
    rows = np.zeros((n, K), np.int32)
    g = _bf16(rng.integers(-7, 8, size=(n, d)).astype(np.float32))
    eN = (rng.integers(1, 1 << 10, size=(n, d)) * np.exp2(rng.integers(-18, 10, size=(n, d)))).astype(np.float32)
    eN *= rng.choice([-1.0, 1.0], size=(n, d)).astype(np.float32)
    gf = bf16_bits_to_f32(g)
    got = oracle.grad_gate(rows, g, eN)
    seq_differs = 0
    for j in range(d):
        want = round_to_f32(sum((f(gf[i, j]) * f(eN[i, j]) for i in range(n)), Fraction(0)))
        assert got[j].view(np.uint32) == want.view(np.uint32)
        acc = np.float32(0.0)
        for i in range(n):
            acc = np.float32(acc + np.float32(gf[i, j] * eN[i, j]))
        seq_differs += acc != want
    assert seq_differs >= d // 2          # a sequential fp32 sum would not pass


def test_gate_grad_float64_sum_within_its_bound_of_the_exact_sum():
    """General values: the float64 sum lies within (n - 1) 2^-53 sum |g eN|
    of the exact rational sum, and the fp32 result is it rounded once."""
    rng = np.random.default_rng(10)
    n, d = 513, 6
    rows = np.zeros((n, K), np.int32)
    g = _bf16(rng.standard_normal((n, d)).astype(np.float32))
    eN = rng.standard_normal((n, d)).astype(np.float32)
    gf = bf16_bits_to_f32(g)
    got, got64 = oracle.grad_gate(rows, g, eN, with_f64=True)
    for j in range(d):
        exact = sum((f(gf[i, j]) * f(eN[i, j]) for i in range(n)), Fraction(0))
        mag = float(sum(abs(f(gf[i, j]) * f(eN[i, j])) for i in range(n)))
        assert abs(f(got64[j]) - exact) <= Fraction((n - 1) * 2.0 ** -53 * mag)
        assert got[j] == np.float32(got64[j])


def test_invalid_tokens_contribute_nothing():
    toks, rows, g, W, T, e1 = _case(seed=8)
    rows = rows.copy()
    bad = [3, 50]
    rows[bad] = -1
    valid = np.ones(toks.size, bool)
    valid[bad] = False
    dT, de1, dW, eN = _autograd(toks, np.where(rows < 0, 0, rows), g, W, T, e1, valid=valid)
    q, got = oracle.grad_table(rows, W, g)
    assert -1 not in q
    assert np.array_equal(got.astype(np.float64), dT[q])
    qt, got_e1 = oracle.grad_e1(toks, rows, g)
    assert np.array_equal(got_e1.astype(np.float64), de1[qt])
    eN32 = eN.astype(np.float32)
    eN32[bad] = np.nan                                        # never read for invalid tokens
    assert np.array_equal(oracle.grad_gate(rows, g, eN32).astype(np.float64), dW)


def test_a_row_used_twice_by_one_token_counts_twice():
    d = 8
    rows = np.array([[5] * 8 + [9] * 8], dtype=np.int32)
    g = _bf16(np.arange(1, d + 1, dtype=np.float32))
    W = np.full(d, 0.5, np.float32)
    q, got = oracle.grad_table(rows, W, g.reshape(1, d))
    assert q.tolist() == [5, 9]
    assert np.array_equal(got, np.stack([8 * 0.5 * np.arange(1, d + 1)] * 2).astype(np.float32))
    q0, got0 = oracle.grad_table(rows, np.zeros(d, np.float32), g.reshape(1, d))
    assert np.all(got0 == 0) and not np.any(np.signbit(got0))


@pytest.mark.parametrize("n", [1, 255, 256, 257, 513])
def test_gate_grad_any_batch_size(n):
    rng = np.random.default_rng(n)
    rows = np.zeros((n, K), np.int32)
    g = _bf16(rng.integers(-3, 4, size=(n, 4)).astype(np.float32))
    eN = rng.integers(-5, 6, size=(n, 4)).astype(np.float32)
    want = (bf16_bits_to_f32(g).astype(np.float64) * eN).sum(axis=0)
    assert np.array_equal(oracle.grad_gate(rows, g, eN).astype(np.float64), want)
