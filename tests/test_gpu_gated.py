"""GPU parity of the normalised, input-gated forward (ngram_forward_gated)
against the oracle, through the C ABI.

The oracle evaluates the fusion in float64 with each sum over ascending
columns; the kernel evaluates it in float64 with its own order of the sums.
Bar: row ids bit-exact; r and the logit within the bound two float64
evaluations of those sums can differ by (tests.tolerance.gated_bounds, each
step's error derived from the arithmetic, times a safety factor); bf16
outputs equal to the oracle's except where the oracle's float64 y lies
within its bound of a bf16 rounding midpoint, and then only the neighbour on
the other side.  The number of such outputs is printed (it is expected to be
0: the bounds are about 1e-12 of the values, against a bf16 spacing of about
4e-3).
"""
from fractions import Fraction

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_embedding_ngram_amd as ng  # noqa: E402
import synth  # noqa: E402
from synth.workloads import CONFIGS, DeviceInputs, GateParams, HostInputs, Spec, gate_params  # noqa: E402
from tests.oracle_ref import expected_gated, sample_tokens  # noqa: E402
from tests.test_gpu_parity import bits16, say  # noqa: E402
from tests.exact import round_to_bf16  # noqa: E402
from tests.tolerance import assert_bf16_rounded_once, assert_f64_close  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _f32(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def run_gated(di: DeviceInputs, gp: GateParams, out_of_place=False, launch=None):
    sp = di.spec
    dev = di.tokens.device
    out = di.residual if (di.residual is not None and not out_of_place) else \
        torch.empty(sp.n * sp.d, dtype=torch.int16, device=dev)
    rows = torch.empty((sp.n, 16), dtype=torch.int32, device=dev)
    stats = torch.empty((sp.n, 2), dtype=torch.float64, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ng.ngram_forward_gated(di.tokens, di.offsets, di.table_obj(), di.W_g, t(gp.gamma), t(gp.u), t(gp.v),
                           gp.b, gp.eps, out, di.e1, residual=di.residual, history=di.history,
                           rows_out=rows, stats_out=stats, launch=launch)
    torch.cuda.synchronize()
    return bits16(out).reshape(sp.n, sp.d), rows.cpu().numpy(), stats.cpu().numpy()


def compare(out, stats, want, want_stats, y, bounds, what):
    b_r, b_logit, b_y = bounds
    assert_f64_close(stats[:, 0], want_stats[:, 0], b_r, f"{what} r")
    assert_f64_close(stats[:, 1], want_stats[:, 1], b_logit, f"{what} logit")
    near = assert_bf16_rounded_once(out, want, y, b_y, what)
    say(f"{what}: {out.size} outputs, {near} at a bf16 midpoint within the bound")
    return near


def check(sp: Spec, gp=None, sample=None, **kw):
    gp = gp or gate_params(sp)
    say(f"gated {sp.name} n={sp.n} R={sp.R} d={sp.d} table={sp.table} res={sp.residual} hist={sp.history} "
        f"b={gp.b} {kw}")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    out, rows, stats = run_gated(di, gp, **kw)
    want_rows, want, want_stats, y, bounds = expected_gated(h, gp, sample=sample)
    assert np.array_equal(rows, want_rows), "row ids differ"
    if sample is not None:
        out, stats = out[sample], stats[sample]
    compare(out, stats, want, want_stats, y, bounds, sp.name)
    return h, di, out


RAGGED = Spec("g_ragged", (1, 2, 3, 5, 0, 250, 33), 151936, 1_000_003, 2560,
              table_kind=synth.KIND_BF16_WIDE, residual=True, config_id=41)


@pytest.mark.parametrize("b", [200.0, -800.0, 0.0])
def test_gated_open_closed_and_half_gate(b):
    """u = v = 0: logit = b exactly on both sides, and alpha = 1 (b = 200),
    0 (b = -800) or 1/2 (b = 0) exactly."""
    sp = Spec(f"g_open{b}", (200, 56), 151936, 100_003, 2560, table_kind=synth.KIND_BF16_WIDE,
              residual=True, config_id=46)
    gp0 = gate_params(sp)
    z = np.zeros(sp.d, np.float32)
    h, di, _ = check(sp, gp=GateParams(gp0.gamma, z, z, b, gp0.eps))
    if b == -800.0:
        # a closed gate leaves residual + e1 rounded once to bf16, exactly
        out, _, stats = run_gated(DeviceInputs(sp, h), GateParams(gp0.gamma, z, z, b, gp0.eps), out_of_place=True)
        assert np.all(stats[:, 1] == b)
        e1v, res = _f32(h.e1_rows(h.tokens)), _f32(h.full_residual())
        for i in (0, 1, 100, sp.n - 1):
            for j in (0, 1, sp.d - 1):
                assert out[i, j] == round_to_bf16(Fraction(float(res[i, j])) + Fraction(float(e1v[i, j])))


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


@pytest.mark.parametrize("tpw", [1, 3, 64])
def test_gated_tokens_per_workgroup(tpw):
    check(Spec(f"gtpw{tpw}", (300, 7), 151936, 100_003, 2560, table_kind=synth.KIND_BF16_WIDE,
               residual=True, config_id=44), launch=(tpw, 0))


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
    _, want, want_stats, y, bounds = expected_gated(h, gp, sample=np.array(clean))
    compare(out[clean], stats[clean], want, want_stats, y, bounds, "g_bad clean tokens")


@pytest.mark.parametrize("table,kind,d", [("bf16", synth.KIND_BF16_WIDE, 2560), ("int8", synth.KIND_I8_NORMAL, 2560),
                                          ("mxfp4", synth.KIND_MXFP4_WIDE, 640)])
def test_gated_host_table_equals_device_table(table, kind, d):
    """The same table in pinned host memory (capped persistent grid) and in
    HBM gives bit-identical gated outputs and statistics."""
    from synth.workloads import fill_host_table
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
        out_host, _, st_host = run_gated(di, gp, out_of_place=True, launch=(0, 5))
    finally:
        hb.free()
    assert np.array_equal(out_dev, out_host) and np.array_equal(st_dev.view(np.uint64), st_host.view(np.uint64))


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
