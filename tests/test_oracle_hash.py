"""Pins of the oracle's context extraction and hash (CPU only).

The hash is pinned by published splitmix64 outputs; the context and key
packing by brute-force enumeration of n-gram windows on small inputs; the
row lists by invariants that any correct implementation must satisfy.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
M64 = (1 << 64) - 1


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_splitmix64_published_vectors():
    g = _gold("splitmix64_vectors.json")
    gamma = int(g["gamma"], 16)
    # Outputs 0..2 from state 0: the generator's state before output i is
    # i * gamma and the oracle's splitmix64(x) is the output from state x.
    for i, v in enumerate(g["state0_first3"]):
        assert oracle.splitmix64((i * gamma) & M64) == int(v, 16)
    s = g["rosetta_seed"]
    for v in g["rosetta_first5"]:
        assert oracle.splitmix64(s) == v
        s = (s + gamma) & M64
    s = g["rosetta_hist_seed"]
    hist = [0] * 5
    for _ in range(g["rosetta_hist_n"]):
        hist[(oracle.splitmix64(s) * 5) >> 64] += 1
        s = (s + gamma) & M64
    assert hist == g["rosetta_hist"]


def test_default_seeds_are_generator_outputs():
    g = _gold("splitmix64_vectors.json")
    seeds = [int(x) for x in oracle.default_seeds()]
    assert seeds[:3] == [int(v, 16) for v in g["state0_first3"]]
    assert len(set(seeds)) == 16


def _inv_mix(y):
    """Inverse of the splitmix64 finaliser, from the xorshift and
    odd-multiplier inverses (a bijection check on the oracle's mixer)."""
    def inv_xorshift(v, s):
        x = v
        for _ in range(64 // s + 1):
            x = v ^ (x >> s)
        return x & M64
    y = inv_xorshift(y, 31)
    y = (y * pow(0x94D049BB133111EB, -1, 1 << 64)) & M64
    y = inv_xorshift(y, 27)
    y = (y * pow(0xBF58476D1CE4E5B9, -1, 1 << 64)) & M64
    y = inv_xorshift(y, 30)
    return y


def test_mix_is_a_bijection():
    gamma = 0x9E3779B97F4A7C15
    rng = np.random.default_rng(0)
    xs = [int(v) for v in rng.integers(0, 2**63, size=2000, dtype=np.int64)]
    xs += [0, 1, M64, 1 << 63, gamma]
    for x in xs:
        assert (_inv_mix(oracle.splitmix64(x)) - gamma) & M64 == x


# ---- context and key packing: brute force over explicit n-gram windows ----

def _py_splitmix64(x):
    z = (x + 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _brute_windows(tokens, offsets, history):
    """(w_{t-2}, w_{t-1}, w_t) for every token by slicing padded sequences."""
    tokens = [int(t) for t in tokens]
    offsets = [int(o) for o in offsets]
    out = []
    for s in range(len(offsets) - 1):
        seq = tokens[offsets[s]:offsets[s + 1]]
        pre = [int(h) for h in history[s]] if history is not None else [oracle.PAD, oracle.PAD]
        padded = pre + seq
        for t in range(len(seq)):
            out.append(tuple(padded[t:t + 3]))
    return out


def _brute_rows(tokens, offsets, R, history=None, seeds=None):
    seeds = [int(s) for s in (oracle.default_seeds() if seeds is None else seeds)]
    rows = []
    for (c2, c1, c0) in _brute_windows(tokens, offsets, history):
        bigram = c0 + c1 * 2**21
        trigram = c0 + c1 * 2**21 + c2 * 2**42
        keys = [bigram] * 8 + [trigram] * 8
        rows.append([_py_splitmix64(k ^ s) % R for k, s in zip(keys, seeds)])
    return np.array(rows, dtype=np.int64).reshape(-1, 16)


@pytest.mark.parametrize("lengths,with_history", [
    ([256], False), ([1, 2, 3, 7, 0, 5], False), ([1, 2, 3, 7, 0, 5], True), ([1], True)])
def test_context_and_rows_brute_force(lengths, with_history):
    offs = synth.ragged_offsets(lengths)
    n = int(offs[-1])
    toks = synth.tokens(11, n, 1024, 1.1)
    hist = synth.tokens(12, 2 * len(lengths), 1024, 1.1).reshape(-1, 2) if with_history else None
    ctx = oracle.context(toks, offs, hist)
    brute = _brute_windows(list(toks), list(offs), None if hist is None else hist.tolist())
    assert [tuple(x) for x in ctx[:, ::-1].tolist()] == brute
    for R in (4096, 1, 7, 2**31 - 1):
        rows = oracle.hash_rows(toks, offs, R, hist)
        assert np.array_equal(rows, _brute_rows(list(toks), list(offs), R,
                                                None if hist is None else hist.tolist()))


def test_custom_seeds_brute_force():
    offs = synth.ragged_offsets([9, 4])
    toks = synth.tokens(3, 13, 151936, 1.1)
    seeds = np.array([(i * 0x1234567) ^ 0xDEADBEEF for i in range(16)], dtype=np.uint64)
    assert np.array_equal(oracle.hash_rows(toks, offs, 20_000_000, seeds=seeds),
                          _brute_rows(list(toks), list(offs), 20_000_000, seeds=list(seeds)))


def test_identical_ngrams_identical_rows():
    offs = synth.seq_offsets(4, 512)
    toks = synth.tokens(5, 2048, 64, 1.1)           # small vocab: many repeats
    ctx = oracle.context(toks, offs)
    rows = oracle.hash_rows(toks, offs, 20_000_000)
    by_bi, by_tri = {}, {}
    for i in range(len(toks)):
        c0, c1, c2 = ctx[i]
        bi, tri = tuple(rows[i, :8]), tuple(rows[i, 8:])
        assert by_bi.setdefault((c1, c0), bi) == bi
        assert by_tri.setdefault((c2, c1, c0), tri) == tri
    assert len(by_bi) > 50 and len(by_tri) > 200
    # distinct n-grams get distinct row lists
    assert len(set(by_bi.values())) == len(by_bi)
    assert len(set(by_tri.values())) == len(by_tri)


def test_pad_only_before_sequence_start():
    offs = synth.seq_offsets(8, 64)
    toks = synth.tokens(6, 512, 151936, 1.1)
    ctx = oracle.context(toks, offs)
    pos = np.arange(512) % 64
    assert np.all((ctx[:, 1] == oracle.PAD) == (pos == 0))
    assert np.all((ctx[:, 2] == oracle.PAD) == (pos < 2))
    assert np.all(ctx[:, 0] == toks)


def test_sequence_move_invariance():
    lengths = [5, 17, 3, 40]
    offs = synth.ragged_offsets(lengths)
    toks = synth.tokens(7, int(offs[-1]), 151936, 1.1)
    rows = oracle.hash_rows(toks, offs, 20_000_000)
    order = [2, 0, 3, 1]
    seqs = [toks[offs[s]:offs[s + 1]] for s in order]
    toks2 = np.concatenate(seqs)
    offs2 = synth.ragged_offsets([lengths[s] for s in order])
    rows2 = oracle.hash_rows(toks2, offs2, 20_000_000)
    for j, s in enumerate(order):
        assert np.array_equal(rows2[offs2[j]:offs2[j + 1]], rows[offs[s]:offs[s + 1]])


def test_decode_with_history_equals_prefill_position():
    toks = synth.tokens(8, 300, 151936, 1.1)
    offs = synth.seq_offsets(1, 300)
    rows = oracle.hash_rows(toks, offs, 20_000_000)
    ps = [2, 3, 100, 299]
    hist = np.array([[toks[p - 2], toks[p - 1]] for p in ps], dtype=np.int32)
    dec = oracle.hash_rows(toks[ps], synth.seq_offsets(len(ps), 1), 20_000_000, hist)
    assert np.array_equal(dec, rows[ps])
    # position 1 with history (PAD, w0) equals prefill at position 1
    dec1 = oracle.hash_rows(toks[[1]], synth.seq_offsets(1, 1), 20_000_000,
                            np.array([[oracle.PAD, toks[0]]], dtype=np.int32))
    assert np.array_equal(dec1[0], rows[1])


def test_rows_in_range_and_uniform():
    offs = synth.seq_offsets(1, 20000)
    toks = synth.tokens(9, 20000, 151936, 1.1, dist="uniform")
    R = 997
    rows = oracle.hash_rows(toks, offs, R)
    assert rows.min() >= 0 and rows.max() < R
    counts = np.bincount(rows.ravel(), minlength=R).astype(np.float64)
    expected = rows.size / R
    chi2 = ((counts - expected) ** 2 / expected).sum()
    # R-1 = 996 degrees of freedom: mean 996, sd 44.6; 6 sd either side
    assert 996 - 6 * 44.6 < chi2 < 996 + 6 * 44.6
    big = oracle.hash_rows(toks, offs, 2**31 - 1)
    assert big.min() >= 0 and big.max() < 2**31 - 1 and big.max() > 2**30
