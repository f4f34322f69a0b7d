"""The seeded input generators: Philox4x32-10 against its published
known-answer vectors, and the value recipes' exactness claims."""
import json
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLD, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)["vectors"]
    for v in kat:
        ctr = [np.array([int(x, 16)], dtype=np.uint64) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        out = synth.philox4x32_10(*ctr, *key)
        assert ["%08x" % int(o[0]) for o in out] == v["out"]


def test_bf16_normal_values_are_exact_multiples():
    x = synth.tensor(synth.KIND_BF16_NORMAL12, 1, synth.TAG_TABLE, 1 << 16)
    f = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = f * 4096.0
    assert np.all(s == np.round(s)) and np.abs(s).max() <= 254
    assert 0.016 < f.std() < 0.020


def test_wide_and_unit_and_scale_ranges():
    w = synth.tensor(synth.KIND_BF16_WIDE, 1, synth.TAG_TABLE, 4096).astype(np.uint32)
    assert np.all(((w >> 7) & 0xFF) >= 100) and np.all(((w >> 7) & 0xFF) <= 131)
    u = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 1, synth.TAG_WG, 4096))
    assert u.min() >= 0 and u.max() < 1
    sc = synth.as_f32(synth.tensor(synth.KIND_F32_SCALE, 1, synth.TAG_SCALE, 4096))
    assert sc.min() >= 2.0**-11 and sc.max() < 2.0**-10
    q = synth.tensor(synth.KIND_I8_NORMAL, 1, synth.TAG_TABLE, 4096)
    assert q.dtype == np.int8 and q.min() >= -126 and q.max() <= 126


def test_rows_on_demand_equal_the_flat_tensor():
    d = 40
    flat = synth.tensor(synth.KIND_BF16_NORMAL12, 9, synth.TAG_TABLE, 100 * d).reshape(100, d)
    ids = [0, 99, 17, 17, 3]
    assert np.array_equal(synth.rows(synth.KIND_BF16_NORMAL12, 9, synth.TAG_TABLE, d, ids), flat[ids])


def test_zipf_tokens_follow_the_rank_law():
    V = 151936
    t = synth.tokens(3, 200000, V, 1.1)
    assert t.min() >= 0 and t.max() < V
    c = np.bincount(t, minlength=V)
    # P(rank 1) / P(rank 2) = 2^1.1
    assert abs(c[0] / c[1] - 2 ** 1.1) < 0.1
    p0 = 1.0 / (np.arange(1, V + 1, dtype=np.float64) ** -1.1).sum()
    assert abs(c[0] / t.size - p0) < 0.01
    u = synth.tokens(3, 200000, V, dist="uniform")
    assert abs(np.bincount(u, minlength=V).mean() - 200000 / V) < 1e-9
