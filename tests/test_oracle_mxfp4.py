"""Pins of the oracle's 4-bit (OCP MXFP4) rows: element values from the OCP MX
specification, an independent decoder written from its bit layout, numpy's
sequential float32 sums, and exact special cases."""
import json
import os
from fractions import Fraction

import numpy as np

import oracle
import synth
from tests.exact import bf16_bits_to_f32

GOLD = os.path.join(os.path.dirname(__file__), "golden", "ocp_mx_fp4.json")
K = 16


def _spec():
    with open(GOLD) as f:
        return json.load(f)


def _decode(code):
    """E2M1 from its bit fields: sign, 2-bit exponent (bias 1), 1-bit mantissa."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    v = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return -v if s else v


def _rows_values(T, d):
    """Decode MXFP4 rows [R][d/2 + d/32] to float64 [R][d] (NaN for E = 255)."""
    R = T.shape[0]
    codes = np.empty((R, d), dtype=np.int64)
    codes[:, 0::2] = T[:, : d // 2] & 15
    codes[:, 1::2] = T[:, : d // 2] >> 4
    E = np.repeat(T[:, d // 2:].astype(np.int64), 32, axis=1)
    lut = np.array([float(_decode(c)) for c in range(16)])
    v = lut[codes] * np.exp2(E - 127.0)
    v[E == 255] = np.nan
    return v


def test_e2m1_codes_match_the_specification():
    pos = _spec()["e2m1_positive_values_by_code"]
    for c in range(16):
        want = pos[c & 7] * (-1 if c & 8 else 1)
        assert oracle.e2m1(c) == want == float(_decode(c))
    assert np.signbit(oracle.e2m1(8))                    # code 8 is -0


def _table(R, d, seed, lo=100, hi=150):
    rng = np.random.default_rng(seed)
    T = np.empty((R, d // 2 + d // 32), dtype=np.uint8)
    T[:, : d // 2] = rng.integers(0, 256, size=(R, d // 2))
    T[:, d // 2:] = rng.integers(lo, hi + 1, size=(R, d // 32))
    return T


def test_sum_is_sequential_fp32_of_the_decoded_values():
    R, d = 509, 128
    T = _table(R, d, 1)
    offs = synth.seq_offsets(1, 300)
    rows = oracle.hash_rows(synth.tokens(2, 300, 1024, 1.1), offs, R)
    eN = oracle.embed_bag_mxfp4(T, d, rows)
    vals = _rows_values(T, d).astype(np.float32)         # exact: powers of two times E2M1
    seq = np.add.accumulate(vals[rows], axis=1, dtype=np.float32)[:, -1, :]
    assert np.array_equal(eN.view(np.uint32), seq.view(np.uint32))
    rev = np.add.accumulate(vals[rows][:, ::-1], axis=1, dtype=np.float32)[:, -1, :]
    assert np.any(rev.view(np.uint32) != seq.view(np.uint32))


def test_unit_scale_sums_are_exact():
    R, d = 257, 64
    T = _table(R, d, 3, lo=127, hi=127)
    rows = oracle.hash_rows(synth.tokens(4, 200, 1024, 1.1), synth.seq_offsets(2, 100), R)
    eN = oracle.embed_bag_mxfp4(T, d, rows)
    want = _rows_values(T, d)[rows].sum(axis=1)
    assert np.array_equal(eN.astype(np.float64), want)


def test_nibble_order_scale_groups_and_special_scales():
    d = 64
    T = np.zeros((3, d // 2 + d // 32), dtype=np.uint8)
    T[0, 0] = 0x42                       # element 0: code 2 (1.0), element 1: code 4 (2.0)
    T[0, 16] = 0x7F                      # elements 32, 33: codes 15 (-6), 7 (6)
    T[0, d // 2] = 127                   # scale of elements 0..31: 1
    T[0, d // 2 + 1] = 130               # scale of elements 32..63: 8
    T[1, :] = 0x11                       # every element code 1 (0.5)
    T[1, d // 2] = 0                     # scale 2^-127 (an fp32 subnormal) for 0..31
    T[1, d // 2 + 1] = 255               # NaN scale for 32..63
    T[2, :d // 2] = 0x99                 # code 9 (-0.5)
    T[2, d // 2:] = 247                  # scale 2^120
    rows = np.array([[0] * K, [1] * K, [2] * K], dtype=np.int32)
    eN = oracle.embed_bag_mxfp4(T, d, rows)
    assert eN[0, 0] == 16 * 1.0 and eN[0, 1] == 16 * 2.0
    assert eN[0, 32] == 16 * -48.0 and eN[0, 33] == 16 * 48.0
    assert np.all(eN[0, 2:32] == 0) and np.all(eN[0, 34:] == 0)
    sub = Fraction(1, 2) * Fraction(2) ** -127 * 16
    assert np.all(eN[1, :32] == np.float32(float(sub)))
    assert np.all(np.isnan(eN[1, 32:]))
    assert np.all(eN[2] == np.float32(-0.5 * 2.0 ** 120 * 16))


def test_mxfp4_forward_is_the_composition_of_its_steps():
    R, d, V = 331, 128, 64
    T = _table(R, d, 5)
    e1 = synth.tensor(synth.KIND_BF16_NORMAL12, 5, synth.TAG_E1, V * d).reshape(V, d)
    W = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 5, synth.TAG_WG, d))
    offs = synth.ragged_offsets([20, 1, 60])
    toks = synth.tokens(5, 81, V, 1.1)
    res = synth.tensor(synth.KIND_BF16_NORMAL6, 5, synth.TAG_RESIDUAL, 81 * d).reshape(81, d)
    out, rows, eN = oracle.forward(toks, offs, T, W, e1=e1, residual=res, mxfp4_d=d)
    assert np.array_equal(rows, oracle.hash_rows(toks, offs, R))
    assert np.array_equal(eN.view(np.uint32), oracle.embed_bag_mxfp4(T, d, rows).view(np.uint32))
    assert np.array_equal(out, oracle.gate_add(eN, toks, W, e1, res))
    assert bf16_bits_to_f32(out).dtype == np.float32
