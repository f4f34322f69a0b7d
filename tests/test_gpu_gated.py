"""GPU parity of the normalised, input-gated forward (ngram_forward_gated)
against the oracle, through the C ABI.

Bar: row ids bit-exact; the normalisation factor r and the gate's logit
bit-exact (every step to them is one IEEE fp32 operation in a stated order);
bf16 outputs bit-exact except where the two sides' exp differ by an ulp and
the oracle's fp32 value y lies that close to a bf16 rounding midpoint.  Then
the two bf16 values are neighbours and y sits within 2^-20 of the size of its
terms (|residual| + |e1| + |alpha W_g n|) from their midpoint: one ulp of
alpha moves alpha W_g n by 2^-23 of itself, and the fma and the residual add
each round once.  With the gate closed, half open or fully open (alpha exactly
0, 1/2 or 1) every output is bit-exact.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_embedding_ngram_amd as ng  # noqa: E402
import synth  # noqa: E402
from synth.workloads import CONFIGS, DeviceInputs, GateParams, HostInputs, Spec, gate_params  # noqa: E402
from tests.oracle_ref import expected_gated, sample_tokens  # noqa: E402
from tests.test_gpu_parity import bits16, say  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _f32(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_gated_equal(got, want, y, mag, what, max_frac=1e-3):
    got = np.asarray(got, np.uint16).reshape(want.shape)
    diff = got != want
    nan_w = np.isnan(_f32(want))
    assert np.array_equal(np.isnan(_f32(got)), nan_w), f"{what}: NaN pattern differs"
    diff &= ~nan_w
    nd = int(diff.sum())
    assert nd <= max(2, max_frac * want.size), f"{what}: {nd} of {want.size} bf16 values differ"
    if nd:
        gi, wi = got[diff].astype(np.int32), want[diff].astype(np.int32)
        assert np.all((gi >> 15) == (wi >> 15)) and np.all(np.abs(gi - wi) == 1), \
            f"{what}: differing values are not bf16 neighbours"
        mid = (_f32(got[diff]) + _f32(want[diff])) / 2
        dist = np.abs(y[diff].astype(np.float64) - mid) / mag[diff]
        assert np.all(dist <= 2.0 ** -20), \
            f"{what}: {nd} differ, max distance from the midpoint {dist.max():.3g} of the terms' size"


def run_gated(di: DeviceInputs, gp: GateParams, out_of_place=False):
    sp = di.spec
    dev = di.tokens.device
    out = di.residual if (di.residual is not None and not out_of_place) else \
        torch.empty(sp.n * sp.d, dtype=torch.int16, device=dev)
    rows = torch.empty((sp.n, 16), dtype=torch.int32, device=dev)
    stats = torch.empty((sp.n, 2), dtype=torch.float32, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ng.ngram_forward_gated(di.tokens, di.offsets, di.table_obj(), di.W_g, t(gp.gamma), t(gp.u), t(gp.v),
                           gp.b, gp.eps, out, di.e1, residual=di.residual, history=di.history,
                           rows_out=rows, stats_out=stats)
    torch.cuda.synchronize()
    return bits16(out).reshape(sp.n, sp.d), rows.cpu().numpy(), stats.cpu().numpy()


def check(sp: Spec, gp=None, sample=None, exact=False, **kw):
    gp = gp or gate_params(sp)
    say(f"gated {sp.name} n={sp.n} R={sp.R} d={sp.d} table={sp.table} res={sp.residual} hist={sp.history} "
        f"b={gp.b} {kw}")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    out, rows, stats = run_gated(di, gp, **kw)
    want_rows, want, want_stats, y, mag = expected_gated(h, gp, sample=sample)
    assert np.array_equal(rows, want_rows), "row ids differ"
    if sample is not None:
        out, stats = out[sample], stats[sample]
    assert np.array_equal(stats.view(np.uint32), want_stats.view(np.uint32)), \
        f"r or logit differ: {np.argwhere(stats.view(np.uint32) != want_stats.view(np.uint32))[:5]}"
    if exact:
        assert np.array_equal(out, want), f"{int((out != want).sum())} outputs differ"
    else:
        assert_gated_equal(out, want, y, mag, sp.name)
    return h, di, out


RAGGED = Spec("g_ragged", (1, 2, 3, 5, 0, 250, 33), 151936, 1_000_003, 2560,
              table_kind=synth.KIND_BF16_WIDE, residual=True, config_id=41)


@pytest.mark.parametrize("b", [200.0, -200.0, 0.0])
def test_gated_open_closed_and_half_gate_bit_exact(b):
    """u = v = 0: logit = b exactly; alpha = 1 (b = 200), 0 (b = -200) or 1/2
    (b = 0) on both sides, so every output is bit-exact."""
    sp = Spec(f"g_open{b}", (200, 56), 151936, 100_003, 2560, table_kind=synth.KIND_BF16_WIDE,
              residual=True, config_id=46)
    gp0 = gate_params(sp)
    z = np.zeros(sp.d, np.float32)
    check(sp, gp=GateParams(gp0.gamma, z, z, b, gp0.eps), exact=True)


def test_gated_tiny():
    check(CONFIGS["tiny"])


def test_gated_ragged_wide_in_place():
    check(RAGGED)


def test_gated_out_of_place_keeps_residual():
    h, di, _ = check(RAGGED.replace(batch=1), out_of_place=True)
    assert np.array_equal(bits16(di.residual).reshape(h.spec.n, -1), h.full_residual())


@pytest.mark.parametrize("d", [8, 64, 520, 1032, 2568, 4104, 8192])
def test_gated_row_widths(d):
    check(Spec(f"gd{d}", (1, 40, 0, 2, 57), 5000, 5003, d, table_kind=synth.KIND_BF16_WIDE,
               residual=True, config_id=42))


@pytest.mark.parametrize("table,kind,d", [("int8", synth.KIND_I8_NORMAL, 2560), ("mxfp4", synth.KIND_MXFP4, 2560),
                                          ("mxfp4", synth.KIND_MXFP4_WIDE, 640), ("int8", synth.KIND_I8_NORMAL, 136)])
def test_gated_quantised_tables(table, kind, d):
    check(Spec(f"g{table}{d}", (130, 70), 151936, 100_003, d, table=table, table_kind=kind,
               residual=True, config_id=43))


@pytest.mark.parametrize("tpw", ["1", "3", "64"])
def test_gated_tokens_per_workgroup(tpw, monkeypatch):
    monkeypatch.setenv("NGRAM_TOKENS_PER_WG", tpw)
    check(Spec(f"gtpw{tpw}", (300, 7), 151936, 100_003, 2560, table_kind=synth.KIND_BF16_WIDE,
               residual=True, config_id=44))


def test_gated_decode_with_history_no_residual():
    check(Spec("g_decode", (1, 1, 1, 1), 151936, 100_003, 2560, history=True,
               table_kind=synth.KIND_BF16_WIDE, config_id=45))


def test_gated_invalid_tokens_give_nan():
    """An id >= V makes its own token invalid; an id above the pad id (or
    negative) also makes the next two tokens of its sequence invalid (their
    context holds it).  Tokens whose context holds no changed id equal the
    oracle on the unchanged batch."""
    sp = Spec("g_bad", (40, 24), 5000, 5003, 512, residual=True, config_id=47)
    gp = gate_params(sp)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    changed = {0: 5000, 17: -1, 41: 1 << 22, 63: 5001}
    for i, t in changed.items():
        di.tokens[i] = t
    say("gated invalid token ids")
    out, rows, stats = run_gated(di, gp, out_of_place=True)
    invalid = {0, 17, 18, 19, 41, 42, 43, 63}
    nan_tok = set(np.nonzero(np.isnan(stats[:, 0]))[0].tolist())
    assert nan_tok == invalid
    inv = sorted(invalid)
    assert np.all(rows[inv] == -1) and np.all(np.isnan(stats[inv])) and np.all(np.isnan(_f32(out[inv])))
    starts = {0, 40}
    clean = [i for i in range(sp.n) if not any(i - k in changed and not any(s in range(i - k + 1, i + 1)
                                                                            for s in starts) for k in (0, 1, 2))]
    assert len(clean) > 40
    _, want, want_stats, y, mag = expected_gated(h, gp, sample=np.array(clean))
    assert np.array_equal(stats[clean].view(np.uint32), want_stats.view(np.uint32))
    assert_gated_equal(out[clean], want, y, mag, "g_bad clean tokens")


@pytest.mark.parametrize("table,kind,d", [("bf16", synth.KIND_BF16_WIDE, 2560), ("int8", synth.KIND_I8_NORMAL, 2560),
                                          ("mxfp4", synth.KIND_MXFP4_WIDE, 640)])
def test_gated_host_table_equals_device_table(table, kind, d, monkeypatch):
    """The same table in pinned host memory (capped persistent grid) and in
    HBM gives bit-identical gated outputs and statistics."""
    from synth.workloads import fill_host_table
    monkeypatch.setenv("NGRAM_HOST_WORKGROUPS", "5")
    sp = Spec(f"g_host_{table}", (300, 212), 151936, 20_003, d, table=table, table_kind=kind,
              residual=True, config_id=48)
    gp = gate_params(sp)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    out_dev, _, st_dev = run_gated(di, gp, out_of_place=True)
    rb = {"bf16": 2 * d, "int8": d, "mxfp4": synth.mxfp4_row_bytes(d)}[table]
    hb = ng.HostBuffer(sp.R * rb)
    try:
        npdt = {"bf16": np.int16, "int8": np.int8, "mxfp4": np.uint8}[table]
        fill_host_table(sp, hb.numpy(npdt, (sp.R, rb // np.dtype(npdt).itemsize)))
        dt = {"bf16": ng.TABLE_BF16, "int8": ng.TABLE_INT8_ROWSCALE, "mxfp4": ng.TABLE_MXFP4}[table]
        di.table_obj = lambda: ng.Table(hb, sp.R, sp.d, dt, row_scale=di.scale)
        out_host, _, st_host = run_gated(di, gp, out_of_place=True)
    finally:
        hb.free()
    assert np.array_equal(out_dev, out_host) and np.array_equal(st_dev.view(np.uint32), st_host.view(np.uint32))


def test_gated_empty_batch():
    sp = Spec("g_empty", (0,), 100, 101, 64, config_id=49)
    gp = gate_params(sp)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    out = torch.empty(0, dtype=torch.int16, device=DEV)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    ng.ngram_forward_gated(di.tokens, di.offsets, di.table_obj(), di.W_g, t(gp.gamma), t(gp.u), t(gp.v),
                           gp.b, gp.eps, out, di.e1)
    torch.cuda.synchronize()


def test_gated_prefill_full_size_sampled():
    sp = CONFIGS["gated"]
    idx = sample_tokens(sp, m=96)
    check(sp, sample=idx)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
