"""Pins of the oracle's gather-sum, int8 dequantisation, gate and rounding.

Each check compares the oracle with something other than itself: a library
routine on a case where it must agree exactly (torch's fp32->bf16 conversion,
torch's embedding_bag in float64 on integer-valued tables), exact rational
arithmetic rounded once, numpy's sequential float32 accumulation, or a
closed form (histograms of a one-hot table, linearity).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.exact import bf16_bits_to_f32, f, round_to_f32


def _torch_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------- bf16 rounding -------------------------------

def test_bf16_rne_matches_torch_on_random_and_edge_patterns():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    edge = np.array([0x00000000, 0x80000000, 0x00008000, 0x00018000, 0x3F808000,
                     0x3F818000, 0x3F807FFF, 0x3F80C000, 0x7F7FFFFF, 0xFF7FFFFF,
                     0x7F7F8000, 0x7F800000, 0xFF800000, 0x00000001, 0x007FFFFF,
                     0x00800000, 0x807FFFFF, 0x4B7FFFFF], dtype=np.uint32)
    x = np.concatenate([bits, edge]).view(np.float32)
    finite = ~np.isnan(x)
    got = oracle.bf16_rne(x)
    assert np.array_equal(got[finite], _torch_bf16_bits(x[finite]))
    # NaN: the oracle's choice is the canonical quiet NaN 0x7FC0; torch only
    # guarantees some NaN (exponent all ones, non-zero fraction)
    nans = np.array([0x7FC00000, 0xFFC00001, 0x7F800001, 0x7FBFFFFF], dtype=np.uint32).view(np.float32)
    assert np.all(oracle.bf16_rne(nans) == 0x7FC0)
    tn = _torch_bf16_bits(nans)
    assert np.all((tn & 0x7F80 == 0x7F80) & (tn & 0x7F != 0))


def test_bf16_rne_is_nearest_ties_even_exactly():
    # every tie between two bf16 neighbours resolves to the even one
    rng = np.random.default_rng(2)
    hi = rng.integers(0x0080, 0x7F7F, size=4096).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    got = oracle.bf16_rne(ties).astype(np.uint32)
    want = np.where(hi % 2 == 0, hi, hi + 1)
    assert np.array_equal(got, want)


# -------------------------------- gather-sum ---------------------------------

def _bf16_of_ints(v):
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_one_hot_table_gives_row_histogram():
    R = d = 64
    T = np.zeros((R, d), dtype=np.float32)
    T[np.arange(R), np.arange(R)] = 1.0
    offs = synth.seq_offsets(2, 128)
    toks = synth.tokens(20, 256, 1024, 1.1)
    rows = oracle.hash_rows(toks, offs, R)
    eN = oracle.embed_bag_bf16(_bf16_of_ints(T), rows)
    hist = np.stack([np.bincount(r, minlength=R) for r in rows]).astype(np.float32)
    assert np.array_equal(eN, hist)


def test_integer_table_matches_float64_and_torch_embedding_bag():
    R, d = 4096, 64
    rng = np.random.default_rng(3)
    Tint = rng.integers(-8, 9, size=(R, d))
    offs = synth.ragged_offsets([100, 1, 2, 153])
    toks = synth.tokens(21, 256, 1024, 1.1)
    rows = oracle.hash_rows(toks, offs, R)
    eN = oracle.embed_bag_bf16(_bf16_of_ints(Tint), rows)
    want64 = Tint[rows].sum(axis=1).astype(np.float64)
    assert np.array_equal(eN.astype(np.float64), want64)
    tb = torch.nn.functional.embedding_bag(
        torch.from_numpy(rows.astype(np.int64)), torch.from_numpy(Tint.astype(np.float64)),
        mode="sum")
    assert np.array_equal(eN.astype(np.float64), tb.numpy())


def test_sum_is_linear_in_the_table():
    R, d = 512, 32
    rng = np.random.default_rng(4)
    T1 = rng.integers(-100, 101, size=(R, d))
    T2 = rng.integers(-100, 101, size=(R, d))
    offs = synth.seq_offsets(1, 300)
    rows = oracle.hash_rows(synth.tokens(22, 300, 1024, 1.1), offs, R)
    e1 = oracle.embed_bag_bf16(_bf16_of_ints(T1), rows)
    e2 = oracle.embed_bag_bf16(_bf16_of_ints(T2), rows)
    e12 = oracle.embed_bag_bf16(_bf16_of_ints(T1 + T2), rows)
    assert np.array_equal(e12, e1 + e2)


def test_sum_is_sequential_fp32_in_k_order():
    R, d = 4096, 64
    T = synth.tensor(synth.KIND_BF16_WIDE, 7, synth.TAG_TABLE, R * d).reshape(R, d)
    offs = synth.seq_offsets(1, 256)
    rows = oracle.hash_rows(synth.tokens(23, 256, 1024, 1.1), offs, R)
    eN = oracle.embed_bag_bf16(T, rows)
    vals = bf16_bits_to_f32(T[rows])                  # [n, 16, d]
    seq = np.add.accumulate(vals, axis=1, dtype=np.float32)[:, -1, :]
    assert np.array_equal(eN.view(np.uint32), seq.view(np.uint32))
    # the order is observable on this table: reversed order differs somewhere
    rev = np.add.accumulate(vals[:, ::-1, :], axis=1, dtype=np.float32)[:, -1, :]
    assert np.any(rev.view(np.uint32) != seq.view(np.uint32))
    # and each partial sum is one correctly rounded fp32 add
    for (i, j) in [(0, 0), (17, 5), (255, 63)]:
        acc = np.float32(0.0)
        for k in range(16):
            acc = round_to_f32(f(acc) + f(vals[i, k, j]))
        assert acc == eN[i, j]


def _int8_case(R=1024, d=32, n=64, seed=5):
    Q = synth.tensor(synth.KIND_I8_NORMAL, seed, synth.TAG_TABLE, R * d).reshape(R, d)
    sc = synth.as_f32(synth.tensor(synth.KIND_F32_SCALE, seed, synth.TAG_SCALE, R))
    offs = synth.seq_offsets(1, n)
    rows = oracle.hash_rows(synth.tokens(seed, n, 1024, 1.2), offs, R)
    return Q, sc, rows


def test_int8_unit_scale_is_exact_integer_sum():
    Q, _, rows = _int8_case()
    eN = oracle.embed_bag_int8(Q, np.ones(Q.shape[0], dtype=np.float32), rows)
    assert np.array_equal(eN.astype(np.int64), Q.astype(np.int64)[rows].sum(axis=1))
    eN2 = oracle.embed_bag_int8(Q, np.full(Q.shape[0], 0.25, dtype=np.float32), rows)
    assert np.array_equal(eN2.astype(np.float64), Q.astype(np.float64)[rows].sum(axis=1) * 0.25)


def test_int8_dequant_is_a_chain_of_single_rounding_fmas():
    Q, sc, rows = _int8_case(n=24)
    eN = oracle.embed_bag_int8(Q, sc, rows)
    rng = np.random.default_rng(6)
    for i, j in zip(rng.integers(0, rows.shape[0], 40), rng.integers(0, Q.shape[1], 40)):
        acc = np.float32(0.0)
        for k in range(16):
            r = rows[i, k]
            acc = round_to_f32(Fraction(int(Q[r, j])) * f(sc[r]) + f(acc))
        assert acc.view(np.uint32) == eN[i, j].view(np.uint32)


# ---------------------------- gate and residual ------------------------------

def _gate_inputs(n=64, d=32, V=1024, seed=9):
    rng = np.random.default_rng(seed)
    eN = (rng.standard_normal((n, d)) * 0.1).astype(np.float32)
    ids = synth.tokens(seed, n, V, 1.1)
    e1 = synth.tensor(synth.KIND_BF16_NORMAL12, seed, synth.TAG_E1, V * d).reshape(V, d)
    W = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, seed, synth.TAG_WG, d))
    res = synth.tensor(synth.KIND_BF16_NORMAL6, seed, synth.TAG_RESIDUAL, n * d).reshape(n, d)
    return eN, ids, e1, W, res


def test_gate_is_one_fma_one_add_one_rounding():
    eN, ids, e1, W, res = _gate_inputs()
    out = oracle.gate_add(eN, ids, W, e1, res)
    out_nores = oracle.gate_add(eN, ids, W, e1, None)
    e1f = bf16_bits_to_f32(e1)
    resf = bf16_bits_to_f32(res)
    for i in range(0, eN.shape[0], 3):
        for j in range(eN.shape[1]):
            h = round_to_f32(f(W[j]) * f(eN[i, j]) + f(e1f[ids[i], j]))
            y = round_to_f32(f(resf[i, j]) + f(h))
            assert out[i, j] == _torch_bf16_bits(np.array([y]))[0]
            assert out_nores[i, j] == _torch_bf16_bits(np.array([h]))[0]


def test_gate_special_cases():
    eN, ids, e1, W, res = _gate_inputs()
    e1f = bf16_bits_to_f32(e1)
    resf = bf16_bits_to_f32(res)
    # all-zero table sum: out = bf16(e1 + res)
    zero = np.zeros_like(eN)
    assert np.array_equal(oracle.gate_add(zero, ids, W, e1, res),
                          _torch_bf16_bits(e1f[ids] + resf))
    # W_g = 0: out = bf16(e1 + res)
    assert np.array_equal(oracle.gate_add(eN, ids, np.zeros_like(W), e1, res),
                          _torch_bf16_bits(e1f[ids] + resf))
    # no e1, no residual, W_g = 1: out = bf16(eN)
    assert np.array_equal(oracle.gate_add(eN, ids, np.ones_like(W), None, None),
                          _torch_bf16_bits(eN))


def test_forward_is_the_composition_of_its_steps():
    R, d, V = 4096, 64, 1024
    T = synth.tensor(synth.KIND_BF16_WIDE, 3, synth.TAG_TABLE, R * d).reshape(R, d)
    e1 = synth.tensor(synth.KIND_BF16_NORMAL12, 3, synth.TAG_E1, V * d).reshape(V, d)
    W = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 3, synth.TAG_WG, d))
    offs = synth.ragged_offsets([30, 1, 2, 95])
    toks = synth.tokens(3, int(offs[-1]), V, 1.1)
    res = synth.tensor(synth.KIND_BF16_NORMAL6, 3, synth.TAG_RESIDUAL, toks.size * d).reshape(-1, d)
    out, rows, eN = oracle.forward(toks, offs, T, W, e1=e1, residual=res)
    r2 = oracle.hash_rows(toks, offs, R)
    e2 = oracle.embed_bag_bf16(T, r2)
    assert np.array_equal(rows, r2)
    assert np.array_equal(eN.view(np.uint32), e2.view(np.uint32))
    assert np.array_equal(out, oracle.gate_add(e2, toks, W, e1, res))


def test_zero_table_forward_equals_e1_plus_residual():
    R, d, V = 4096, 64, 1024
    e1 = synth.tensor(synth.KIND_BF16_NORMAL12, 4, synth.TAG_E1, V * d).reshape(V, d)
    W = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 4, synth.TAG_WG, d))
    offs = synth.seq_offsets(1, 256)
    toks = synth.tokens(4, 256, V, 1.1)
    res = synth.tensor(synth.KIND_BF16_NORMAL6, 4, synth.TAG_RESIDUAL, 256 * d).reshape(-1, d)
    out, _, _ = oracle.forward(toks, offs, np.zeros((R, d), np.uint16), W, e1=e1, residual=res)
    assert np.array_equal(out, _torch_bf16_bits(bf16_bits_to_f32(e1)[toks] + bf16_bits_to_f32(res)))
    out0, _, _ = oracle.forward(toks, offs, np.zeros((R, d), np.uint16), W, e1=e1)
    assert np.array_equal(out0, e1[toks])


def test_int8_forward_with_scale_one_is_integer_sum():
    R, d = 2048, 16
    Q = synth.tensor(synth.KIND_I8_NORMAL, 8, synth.TAG_TABLE, R * d).reshape(R, d)
    offs = synth.seq_offsets(2, 50)
    toks = synth.tokens(8, 100, 1024, 1.2)
    W = np.ones(d, dtype=np.float32)
    out, rows, eN = oracle.forward(toks, offs, Q, W, scale=np.ones(R, np.float32))
    assert np.array_equal(eN.astype(np.int64), Q.astype(np.int64)[rows].sum(axis=1))
    assert np.array_equal(out, _torch_bf16_bits(eN))


@pytest.mark.parametrize("n", [0])
def test_empty_input(n):
    out, rows, eN = oracle.forward(np.zeros(0, np.int32), np.array([0], np.int32),
                                   np.zeros((16, 8), np.uint16), np.ones(8, np.float32))
    assert out.shape == (0, 8) and rows.shape == (0, 16)


@pytest.mark.parametrize("scale_exp", [0, -5, 3])
def test_gate_fma_is_fused_on_a_constructed_near_tie(scale_exp):
    """W = 1 - 2^-24, eN = 2^-8 + 2^-24 + 2^-31, e1 = 1 (all scaled by 2^s):
    the exact W*eN + e1 lies just above the fp32 tie 1 + 2^-8 + 2^-24, so one
    rounding gives 1 + 2^-8 + 2^-23 and bf16 rounds that up to 1 + 2^-7; a
    separately rounded product lands on the tie, then on 1 + 2^-8, then on the
    bf16 tie, which goes to the even 1.0."""
    s = 2.0 ** scale_exp
    W = np.array([1.0 - 2.0 ** -24], dtype=np.float32)
    eN = np.array([[(2.0 ** -8 + 2.0 ** -24 + 2.0 ** -31) * s]], dtype=np.float32)
    e1 = _bf16_of_ints(np.array([[1.0 * s]]))
    exact = f(W[0]) * f(eN[0, 0]) + f(1.0 * s)
    y = round_to_f32(exact)
    assert y == np.float32((1.0 + 2.0 ** -8 + 2.0 ** -23) * s)
    want = _torch_bf16_bits(np.array([y]))
    assert want[0] == _bf16_of_ints(np.array([(1.0 + 2.0 ** -7) * s]))[0]
    unfused = np.float32(np.float32(W[0] * eN[0, 0]) + np.float32(1.0 * s))
    assert _torch_bf16_bits(np.array([unfused]))[0] != want[0]
    ids = np.array([0], dtype=np.int32)
    assert oracle.gate_add(eN, ids, W, e1, None)[0, 0] == want[0]
    zero_res = np.zeros((1, 1), dtype=np.uint16)
    assert oracle.gate_add(eN, ids, W, e1, zero_res)[0, 0] == want[0]
