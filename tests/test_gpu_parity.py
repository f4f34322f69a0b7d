"""GPU parity against the oracle at sizes the oracle finishes in seconds,
through the C ABI (the Python binding only marshals pointers).

Bar: row ids bit-exact, fp32 sums bit-exact, bf16 outputs bit-exact (the
relative-error bound of 1e-3 is below one bf16 ulp, so only identical bits
meet it; the observed maximum relative error is asserted too).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_embedding_ngram_amd as ng  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from synth.workloads import CONFIGS, DeviceInputs, HostInputs, Spec  # noqa: E402
from tests.oracle_ref import expected  # noqa: E402

pytestmark = pytest.mark.gpu
REL_TOL = 1e-3


def say(msg):
    print(f"[case] {msg}", flush=True)


def bits16(t):
    return t.cpu().numpy().view(np.uint16)


def assert_bf16_equal(got, want, what):
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    g = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = (want.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    finite = np.isfinite(w)
    rel = np.abs(g[finite] - w[finite]) / np.maximum(np.abs(w[finite]), 2.0 ** -14)
    ndiff = int((got != want).sum())
    assert ndiff == 0, f"{what}: {ndiff} bf16 values differ, max rel err {rel.max():.3g}"
    assert rel.size == 0 or rel.max() <= REL_TOL


def check_staged(T, hb, rows, want_rows, want_eN, mode, scale=None):
    """ngram_gather_host in ``mode`` on the host table T (pinned buffer hb):
    each distinct valid row staged once, byte for byte, the remap pointing at
    it, and the sums from the stage equal to the oracle's ``want_eN``."""
    say(f"staged gather mode {mode}: R={T.R} d={T.d} dtype={T.dtype}")
    n = rows.shape[0]
    rb = ng.row_bytes(T.d, T.dtype)
    stage = torch.empty(n * 16 * rb, dtype=torch.uint8, device="cuda:0")
    remap = torch.empty((n, 16), dtype=torch.int32, device="cuda:0")
    sscale = torch.empty(n * 16, dtype=torch.float32, device="cuda:0") if T.dtype == ng.TABLE_INT8_ROWSCALE else None
    _, _, nst = ng.ngram_gather_host(T, rows, stage, remap, stage_scale_out=sscale, mode=mode)
    view = {ng.TABLE_BF16: stage.view(torch.int16), ng.TABLE_INT8_ROWSCALE: stage.view(torch.int8)}.get(T.dtype, stage)
    eN2 = ng.ngram_embed_bag(ng.Table(view, n * 16, T.d, T.dtype, row_scale=sscale), remap)
    torch.cuda.synchronize()
    U = int(nst.item())
    valid = want_rows[(want_rows >= 0) & (want_rows < T.R)]
    assert U == np.unique(valid).size
    rm = remap.cpu().numpy()
    assert np.array_equal(rm < 0, (want_rows < 0) | (want_rows >= T.R))
    assert rm.max() == U - 1 and np.unique(rm[rm >= 0]).size == U          # stage rows 0..U-1, each used
    host = hb.numpy(np.uint8, (T.R, rb))
    st = stage.cpu().numpy().reshape(n * 16, rb)
    ok = rm >= 0
    assert np.array_equal(st[rm[ok]], host[want_rows[ok]])                   # staged rows are the table's bytes
    if sscale is not None:
        assert np.array_equal(sscale.cpu().numpy()[rm[ok]], scale.cpu().numpy()[want_rows[ok]])
    assert np.array_equal(eN2.cpu().numpy().view(np.uint32), want_eN.view(np.uint32))


def run_forward(di: DeviceInputs, out_of_place=False, seeds=None, launch=None):
    sp = di.spec
    if di.residual is not None and not out_of_place:
        out = di.residual
    else:
        out = torch.empty(sp.n * sp.d, dtype=torch.int16, device=di.tokens.device)
    rows = torch.empty((sp.n, 16), dtype=torch.int32, device=di.tokens.device)
    ng.ngram_forward(di.tokens, di.offsets, di.table_obj(), di.W_g, out, e1=di.e1,
                     residual=di.residual, history=di.history, rows_out=rows, seeds=seeds, launch=launch)
    torch.cuda.synchronize()
    return bits16(out).reshape(sp.n, sp.d), rows.cpu().numpy()


def check_spec(sp: Spec, **kw):
    say(f"{sp.name} n={sp.n} R={sp.R} d={sp.d} table={sp.table} e1={sp.e1} res={sp.residual} "
        f"hist={sp.history} {kw}")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    out, rows = run_forward(di, **kw)
    want_rows, _, want_out = expected(h)
    assert np.array_equal(rows, want_rows), "row ids differ"
    assert_bf16_equal(out, want_out, sp.name)
    return h, di


RAGGED = Spec("ragged_wide", (1, 2, 3, 5, 0, 250, 33), 151936, 1_000_003, 2560,
              table_kind=synth.KIND_BF16_WIDE, residual=True, config_id=11)


def test_tiny_config_fused():
    check_spec(CONFIGS["tiny"])


def test_ragged_wide_in_place():
    check_spec(RAGGED)


def test_ragged_wide_out_of_place_keeps_residual():
    h, di = check_spec(RAGGED.replace(batch=1), out_of_place=True)
    assert np.array_equal(bits16(di.residual).reshape(h.spec.n, -1), h.full_residual())


@pytest.mark.parametrize("d", [8, 64, 520, 1032, 2568, 4104])
def test_row_widths(d):
    check_spec(Spec(f"d{d}", (1, 40, 0, 2, 57), 5000, 5003, d,
                    table_kind=synth.KIND_BF16_WIDE, residual=True, config_id=12))


@pytest.mark.parametrize("e1,res", [(False, False), (True, False), (False, True), (True, True)])
def test_optional_e1_and_residual(e1, res):
    check_spec(Spec(f"opt{int(e1)}{int(res)}", (130,), 2048, 4096, 256,
                    table_kind=synth.KIND_BF16_WIDE, e1=e1, residual=res, config_id=13))


@pytest.mark.parametrize("tpw", [1, 3, 64])
def test_tokens_per_workgroup(tpw):
    check_spec(Spec(f"tpw{tpw}", (300, 7), 151936, 100_003, 2560,
                    table_kind=synth.KIND_BF16_WIDE, residual=True, config_id=14), launch=(tpw, 0))


def test_launch_override_out_of_range_is_refused():
    sp = Spec("launch_bad", (8,), 100, 101, 64, config_id=14)
    di = DeviceInputs(sp, HostInputs(sp))
    for bad in ((65, 0), (-1, 0), (0, -2)):
        with pytest.raises(ng.NgramError, match="EINVAL"):
            run_forward(di, launch=bad)


def test_decode_with_history():
    check_spec(Spec("decode_hist", (1, 1, 1, 1), 151936, 100_003, 2560, history=True,
                    table_kind=synth.KIND_BF16_WIDE, config_id=15))


def test_history_of_pads_equals_no_history():
    sp = Spec("pads", (5, 9), 1024, 4096, 64, config_id=16)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    out0, rows0 = run_forward(di)
    di.history = torch.full((2, 2), ng.PAD_ID, dtype=torch.int32, device="cuda:0")
    out1, rows1 = run_forward(di)
    assert np.array_equal(rows0, rows1) and np.array_equal(out0, out1)


def test_int8_ragged():
    check_spec(Spec("int8_ragged", (3, 0, 200, 1), 151936, 1_000_003, 2560, zipf_s=1.2,
                    table="int8", table_kind=synth.KIND_I8_NORMAL, residual=True, config_id=17))


def test_int8_small_widths():
    check_spec(Spec("int8_d72", (33, 1), 1000, 777, 72, table="int8",
                    table_kind=synth.KIND_I8_NORMAL, residual=True, config_id=18))


def test_custom_seeds():
    sp = Spec("seeds", (77,), 1024, 4096, 64, table_kind=synth.KIND_BF16_WIDE, config_id=19)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    seeds = [(k * 0x9E3779B97F4A7C15 + 12345) & 0xFFFFFFFFFFFFFFFF for k in range(16)]
    say("custom seeds")
    out, rows = run_forward(di, seeds=seeds)
    want_out, want_rows, _ = oracle.forward(h.tokens, h.offsets, h.full_table(), h.W_g,
                                            e1=h.full_e1(), seeds=np.array(seeds, dtype=np.uint64))
    assert np.array_equal(rows, want_rows)
    assert_bf16_equal(out, want_out, "custom seeds")


def test_unfused_pipeline_equals_fused_and_oracle():
    sp = RAGGED.replace(batch=2)
    say("unfused pipeline")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
    eN = ng.ngram_embed_bag(di.table_obj(), rows)
    out = torch.empty(sp.n * sp.d, dtype=torch.int16, device="cuda:0")
    ng.ngram_gate_add(eN, di.tokens, di.W_g, out, e1=di.e1, residual=di.residual)
    torch.cuda.synchronize()
    want_rows, want_eN, want_out = expected(h)
    assert np.array_equal(rows.cpu().numpy(), want_rows)
    assert np.array_equal(eN.cpu().numpy().view(np.uint32), want_eN.view(np.uint32))
    assert_bf16_equal(bits16(out).reshape(sp.n, -1), want_out, "unfused")
    fused, _ = run_forward(di, out_of_place=True)
    assert np.array_equal(fused, bits16(out).reshape(sp.n, -1))


def test_unfused_int8_sum_bits():
    sp = Spec("int8_bag", (64, 64), 151936, 1_000_003, 2560, zipf_s=1.2, table="int8",
              table_kind=synth.KIND_I8_NORMAL, config_id=20)
    say("int8 embed_bag")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
    eN = ng.ngram_embed_bag(di.table_obj(), rows)
    torch.cuda.synchronize()
    _, want_eN, _ = expected(h)
    assert np.array_equal(eN.cpu().numpy().view(np.uint32), want_eN.view(np.uint32))


@pytest.mark.parametrize("table,d", [("bf16", 1536), ("bf16", 9216), ("int8", 1024), ("int8", 9216),
                                     ("int8", 1032)])
def test_unfused_and_fused_whole_and_looped_slices(table, d):
    """Widths made of whole 512-column slices (the int8 scales by one load
    per token, the bag kernel's fp32 sums through LDS), up to 18 slices, so
    each of 16 wavefronts takes two in turn; 1032 leaves an 8-column last
    slice beside whole ones.  fp32 sums and bf16 outputs bit-exact."""
    kw = dict(table="int8", table_kind=synth.KIND_I8_NORMAL) if table == "int8" else \
        dict(table_kind=synth.KIND_BF16_WIDE)
    sp = Spec(f"slices_{table}_{d}", (3, 0, 40, 1), 151936, 20_011, d, residual=True, config_id=61, **kw)
    h, di = check_spec(sp)
    rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
    eN = ng.ngram_embed_bag(di.table_obj(), rows)
    torch.cuda.synchronize()
    _, want_eN, _ = expected(h)
    assert np.array_equal(eN.cpu().numpy().view(np.uint32), want_eN.view(np.uint32))


def test_hash_extreme_R():
    sp = Spec("hashR", (1, 2, 300), 151936, 4096, 64, config_id=21)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h, table=False, e1=False)
    for R in (1, 2, 3, 1 << 20, 2**31 - 1):
        say(f"ngram_hash R={R}")
        rows = ng.ngram_hash(di.tokens, di.offsets, R)
        torch.cuda.synchronize()
        assert np.array_equal(rows.cpu().numpy(), oracle.hash_rows(h.tokens, h.offsets, R))


def test_table_with_one_row():
    check_spec(Spec("R1", (20,), 64, 1, 64, table_kind=synth.KIND_BF16_WIDE, config_id=22))


def test_vocab_boundary_tokens():
    sp = Spec("vb", (6,), 1000, 4096, 64, config_id=23)
    h = HostInputs(sp)
    h.tokens = np.array([0, 999, 999, 0, 998, 1], dtype=np.int32)
    di = DeviceInputs(sp, h)
    say("vocab boundary tokens")
    out, rows = run_forward(di)
    want_out, want_rows, _ = oracle.forward(h.tokens, h.offsets, h.full_table(), h.W_g, e1=h.full_e1())
    assert np.array_equal(rows, want_rows)
    assert_bf16_equal(out, want_out, "vocab boundary")


def test_invalid_ids_give_nan_and_leave_others_exact():
    sp = Spec("bad", (8,), 1000, 4096, 64, residual=True, config_id=24)
    h = HostInputs(sp)
    good = h.tokens.copy()
    bad = good.copy()
    bad[3] = 1000            # == V: out of range
    bad[6] = -5
    di = DeviceInputs(sp, h)
    di.tokens = torch.from_numpy(bad).to("cuda:0")
    say("invalid token ids")
    out, rows = run_forward(di, out_of_place=True)
    assert np.all(out[3] == 0x7FC0) and np.all(out[6] == 0x7FC0)
    assert np.all(rows[3] == -1) and np.all(rows[6] == -1)
    # tokens whose context holds no invalid id are exact
    want_out, want_rows, _ = oracle.forward(good, h.offsets, h.full_table(), h.W_g,
                                            e1=h.full_e1(), residual=h.full_residual())
    for i in (0, 1, 2):
        assert np.array_equal(rows[i], want_rows[i]) and np.array_equal(out[i], want_out[i])
    # embed_bag with out-of-range row ids: NaN sums for those tokens only
    rr = torch.from_numpy(want_rows.copy()).to("cuda:0")
    rr[2, 5] = sp.R
    rr[4, 0] = -1
    eN = ng.ngram_embed_bag(di.table_obj(), rr)
    torch.cuda.synchronize()
    e = eN.cpu().numpy()
    assert np.all(np.isnan(e[2])) and np.all(np.isnan(e[4]))
    assert np.array_equal(e[0].view(np.uint32), oracle.embed_bag_bf16(h.full_table(), want_rows[:1])[0].view(np.uint32))


def test_empty_batch_launches_nothing():
    sp = Spec("empty", (4,), 1000, 4096, 64, config_id=25)
    di = DeviceInputs(sp)
    z = torch.zeros(0, dtype=torch.int32, device="cuda:0")
    out = torch.zeros(0, dtype=torch.int16, device="cuda:0")
    say("n = 0")
    ng.ngram_forward(z, torch.zeros(1, dtype=torch.int32, device="cuda:0"), di.table_obj(),
                     di.W_g, out, e1=di.e1)
    r = ng.ngram_hash(z, torch.zeros(1, dtype=torch.int32, device="cuda:0"), 4096)
    assert r.shape == (0, 16)
    e = ng.ngram_embed_bag(di.table_obj(), torch.zeros((0, 16), dtype=torch.int32, device="cuda:0"))
    assert e.shape == (0, 64)
    torch.cuda.synchronize()


def test_default_seeds_match_oracle():
    assert ng.default_seeds() == [int(s) for s in oracle.default_seeds()]


def test_repeated_calls_are_deterministic():
    sp = Spec("det", (512, 100), 151936, 100_003, 2560, table_kind=synth.KIND_BF16_WIDE, config_id=26)
    di = DeviceInputs(sp)
    say("determinism")
    a, ra = run_forward(di)
    b, rb = run_forward(di)
    assert np.array_equal(a, b) and np.array_equal(ra, rb)


@pytest.mark.parametrize("wgs,tpw,table", [(3, 1, "bf16"), (5, 3, "bf16"), (64, 4, "bf16"), (7, 2, "int8")])
def test_host_table_paths(wgs, tpw, table):
    """Pinned-host table with a capped, persistent grid (several ragged tiles
    per workgroup): fused forward, zero-copy sum and staged gather all equal
    the oracle."""
    from synth.workloads import fill_host_table
    kw = dict(table="int8", table_kind=synth.KIND_I8_NORMAL) if table == "int8" else \
        dict(table_kind=synth.KIND_BF16_WIDE)
    sp = Spec(f"host_{table}_{wgs}_{tpw}", (1, 40, 0, 300, 2), 151936, 20_011, 2560, residual=True,
              config_id=27, **kw)
    say(sp.name)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h, table=False)
    esize = 2 if table == "bf16" else 1
    hb = ng.HostBuffer(sp.R * sp.d * esize)
    try:
        fill_host_table(sp, hb.numpy(np.int16 if table == "bf16" else np.int8, (sp.R, sp.d)))
        scale = None
        if table == "int8":
            scale = synth.fill_gpu(synth.KIND_F32_SCALE, sp.seed, synth.TAG_SCALE,
                                   torch.empty(sp.R, dtype=torch.float32, device="cuda:0"))
        T = ng.Table(hb, sp.R, sp.d, ng.TABLE_INT8_ROWSCALE if table == "int8" else ng.TABLE_BF16,
                     row_scale=scale)
        want_rows, want_eN, want_out = expected(h)
        out = torch.empty(sp.n * sp.d, dtype=torch.int16, device="cuda:0")
        rows = torch.empty((sp.n, 16), dtype=torch.int32, device="cuda:0")
        ng.ngram_forward(di.tokens, di.offsets, T, di.W_g, out, e1=di.e1, residual=di.residual, rows_out=rows,
                         launch=(tpw, wgs))
        eN = ng.ngram_embed_bag(T, rows, launch=(tpw, wgs))
        torch.cuda.synchronize()
        assert np.array_equal(rows.cpu().numpy(), want_rows)
        assert_bf16_equal(bits16(out).reshape(sp.n, -1), want_out, sp.name)
        assert np.array_equal(eN.cpu().numpy().view(np.uint32), want_eN.view(np.uint32))
        for mode in (ng.GATHER_ZERO_COPY, ng.GATHER_ASYNC_COPY):
            check_staged(T, hb, rows, want_rows, want_eN, mode, scale=scale)
    finally:
        hb.free()


@pytest.mark.parametrize("table,C", [("bf16", 500), ("bf16", 0), ("int8", 300)])
def test_row_pool(table, C):
    """Hot-row cache + per-batch dedup in front of a host table: the sums from
    the pool equal the oracle's bit for bit, every pool row is an exact copy
    of its table row, and each distinct uncached row is fetched exactly once."""
    from synth.workloads import fill_host_table
    kw = dict(table="int8", table_kind=synth.KIND_I8_NORMAL) if table == "int8" else \
        dict(table_kind=synth.KIND_BF16_WIDE)
    sp = Spec(f"pool_{table}_{C}", (40, 0, 300, 3), 151936, 20_011, 2560, config_id=28, **kw)
    say(sp.name)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h, table=False)
    npdt = np.int16 if table == "bf16" else np.int8
    hb = ng.HostBuffer(sp.R * sp.d * np.dtype(npdt).itemsize)
    try:
        host_np = hb.numpy(npdt, (sp.R, sp.d))
        fill_host_table(sp, host_np)
        scale = None
        if table == "int8":
            scale = synth.fill_gpu(synth.KIND_F32_SCALE, sp.seed, synth.TAG_SCALE,
                                   torch.empty(sp.R, dtype=torch.float32, device="cuda:0"))
        T = ng.Table(hb, sp.R, sp.d, ng.TABLE_INT8_ROWSCALE if table == "int8" else ng.TABLE_BF16, row_scale=scale)
        # frequencies from two other batches choose the cached rows
        counts = None
        for b in (1, 2):
            hb_in = HostInputs(sp.replace(batch=b))
            r_b = ng.ngram_hash(torch.from_numpy(hb_in.tokens).cuda(), torch.from_numpy(hb_in.offsets).cuda(), sp.R)
            counts = ng.ngram_count_rows(r_b, sp.R, counts=counts, accumulate=counts is not None)
        pool = ng.RowPool(T, C + 16 * sp.n)
        hot, selected = ng.ngram_select_hot_rows(counts, C)
        ng.ngram_pool_cache_rows(pool, hot, selected)
        rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
        rows_bad = rows.clone()
        rows_bad[5, 3] = sp.R
        rows_bad[7, 0] = -1
        fetched = torch.zeros(1, dtype=torch.int64, device="cuda:0")
        prow = ng.ngram_pool_gather(pool, rows_bad, fetched_out=fetched)
        eN = ng.ngram_embed_bag(pool.device_table(), prow)
        torch.cuda.synchronize()

        want_rows, want_eN, _ = expected(h)
        assert np.array_equal(rows.cpu().numpy(), want_rows)
        e = eN.cpu().numpy()
        good = np.ones(sp.n, bool)
        good[[5, 7]] = False
        assert np.all(np.isnan(e[~good]))
        assert np.array_equal(e[good].view(np.uint32), want_eN[good].view(np.uint32))

        cnt = counts.cpu().numpy()
        hot_np = hot.cpu().numpy()[:selected]
        assert selected <= C and len(set(hot_np.tolist())) == selected and np.all(cnt[hot_np] > 0)
        if selected:
            rest = np.ones(sp.R, bool)
            rest[hot_np] = False
            u = cnt[rest].max()
            assert cnt[hot_np].min() > u                            # a threshold set
            assert u == 0 or selected + int((cnt == u).sum()) > C   # the next level would not fit
        slots = pool.slot_of_row.cpu().numpy()
        assert set(np.nonzero(slots >= 0)[0].tolist()) == set(hot_np.tolist())
        rb = rows_bad.cpu().numpy()
        valid = (rb >= 0) & (rb < sp.R)
        distinct = np.unique(rb[valid])
        assert int(fetched.item()) == int((slots[distinct] < 0).sum())
        pr = prow.cpu().numpy()
        assert np.all(pr[~valid] == -1) and np.all(pr[valid] >= 0)
        pool_np = pool.data.view(pool.pool_rows, sp.d).cpu().numpy()
        assert np.array_equal(pool_np[pr[valid]].view(npdt), host_np[rb[valid]])
        if table == "int8":
            assert np.array_equal(pool.row_scale.cpu().numpy()[pr[valid]], scale.cpu().numpy()[rb[valid]])
    finally:
        hb.free()


@pytest.mark.parametrize("d", [128, 384, 640, 2560])
def test_mxfp4_table(d):
    sp = Spec(f"mxfp4_d{d}", (1, 40, 0, 200, 3), 151936, 20_011, d, table="mxfp4",
              table_kind=synth.KIND_MXFP4_WIDE, residual=True, config_id=29)
    h, di = check_spec(sp)
    say(f"mxfp4 embed_bag d={d}")
    rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
    eN = ng.ngram_embed_bag(di.table_obj(), rows)
    torch.cuda.synchronize()
    _, want_eN, _ = expected(h)
    assert np.array_equal(eN.cpu().numpy().view(np.uint32), want_eN.view(np.uint32))


def test_mxfp4_special_scales():
    """E8M0 = 255 makes the row's 32-element group NaN; E8M0 = 0 (2^-127, an
    fp32 subnormal) and large exponents decode exactly."""
    d, R = 128, 5
    rb = synth.mxfp4_row_bytes(d)
    rng = np.random.default_rng(0)
    T = rng.integers(0, 256, size=(R, rb)).astype(np.uint8)
    T[0, d // 2:] = 0
    T[1, d // 2:] = [255, 127, 200, 0]
    T[2, d // 2:] = 254
    T[3, d // 2:] = [1, 2, 3, 4]
    T[4, d // 2:] = 127
    rows = np.array([[0] * 16, [1] * 8 + [4] * 8, [2, 3] * 8, [4] * 16], dtype=np.int32)
    say("mxfp4 special scales")
    t = torch.from_numpy(T.reshape(-1)).cuda()
    eN = ng.ngram_embed_bag(ng.Table(t, R, d, ng.TABLE_MXFP4), torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    got = eN.cpu().numpy()
    want = oracle.embed_bag_mxfp4(T, d, rows)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan[1, :32].all() and not nan[1, 32:].any()
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("d", [640, 1024])
def test_mxfp4_forward_every_scale_byte(d):
    """The fused forward (e1 and residual) on an MXFP4 table whose scale
    bytes take every value 0..255: E = 0 (2^-127), large exponents (sums
    that overflow to inf, and inf - inf), and E = 255 (NaN groups), over
    whole 512-column slices and a partial one (d = 640)."""
    R, V, lengths = 97, 500, (1, 3, 200, 57)
    rb = synth.mxfp4_row_bytes(d)
    rng = np.random.default_rng(d)
    T = rng.integers(0, 256, size=(R, rb)).astype(np.uint8)
    T[:, d // 2:] = rng.permutation(np.resize(np.arange(256), R * (d // 32))).reshape(R, d // 32)
    n = sum(lengths)
    tokens = rng.integers(0, V, size=n).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    W_g = rng.standard_normal(d).astype(np.float32)
    e1 = (rng.standard_normal((V, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    res = (rng.standard_normal((n, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    want, want_rows, want_eN = oracle.forward(tokens, offsets, T, W_g, e1=e1, residual=res, mxfp4_d=d)
    assert np.isnan(want_eN).any() and np.isinf(want_eN).any()
    say(f"mxfp4 forward, every scale byte: d={d} n={n}")
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).cuda()
    out = torch.empty(n * d, dtype=torch.int16, device="cuda:0")
    rows = torch.empty((n, 16), dtype=torch.int32, device="cuda:0")
    ng.ngram_forward(dev(tokens, np.int32), dev(offsets, np.int32), ng.Table(dev(T.reshape(-1), np.uint8), R, d,
                     ng.TABLE_MXFP4), dev(W_g, np.float32), out, e1=dev(e1, np.int16),
                     residual=dev(res, np.int16), rows_out=rows)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), want_rows)
    got = bits16(out).reshape(n, d)
    nan = (want & 0x7FFF) > 0x7F80
    assert np.array_equal((got & 0x7FFF) > 0x7F80, nan)
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("d", [128, 2560])
def test_mxfp4_host_table_paths(d):
    from synth.workloads import fill_host_table
    sp = Spec(f"mxfp4_host_d{d}", (40, 0, 90), 151936, 20_011, d, table="mxfp4",
              table_kind=synth.KIND_MXFP4_WIDE, config_id=30)
    say(sp.name)
    h = HostInputs(sp)
    rb = synth.mxfp4_row_bytes(d)
    hb = ng.HostBuffer(sp.R * rb)
    try:
        fill_host_table(sp, hb.numpy(np.uint8, (sp.R, rb)))
        T = ng.Table(hb, sp.R, d, ng.TABLE_MXFP4)
        di = DeviceInputs(sp, h, table=False)
        rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
        eN = ng.ngram_embed_bag(T, rows, launch=(0, 3))
        torch.cuda.synchronize()
        want_rows, want, want_out = expected(h)
        for mode in (ng.GATHER_ZERO_COPY, ng.GATHER_ASYNC_COPY):
            check_staged(T, hb, rows, want_rows, want, mode)
        pool = ng.RowPool(T, 50 + 16 * sp.n)
        counts = ng.ngram_count_rows(rows, sp.R)
        hot, sel = ng.ngram_select_hot_rows(counts, 50)
        ng.ngram_pool_cache_rows(pool, hot, sel)
        prow = ng.ngram_pool_gather(pool, rows)
        eN3 = ng.ngram_embed_bag(pool.device_table(), prow)
        out = torch.empty(sp.n * d, dtype=torch.int16, device="cuda:0")
        ng.ngram_forward(di.tokens, di.offsets, T, di.W_g, out, e1=di.e1)     # fused, persistent grid
        torch.cuda.synchronize()
        for e in (eN, eN3):
            assert np.array_equal(e.cpu().numpy().view(np.uint32), want.view(np.uint32))
        assert_bf16_equal(bits16(out).reshape(sp.n, d), want_out, sp.name)
    finally:
        hb.free()


def test_unpinned_host_table_is_rejected_and_leaves_no_error_behind():
    """A host table in ordinary (not pinned, not device-mapped) memory: the
    host-side pointer lookup fails, the call returns NGRAM_EHIP without a
    launch, and the next call runs normally."""
    import ctypes
    sp = Spec("unpinned", (40,), 1000, 64, 64, table_kind=synth.KIND_BF16_WIDE, config_id=26)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
    plain = np.ascontiguousarray(h.full_table())                    # pageable host memory
    t = ng._Table(plain.ctypes.data, None, sp.R, sp.d, ng.TABLE_BF16, ng.IN_HOST, 0)
    eN = torch.empty((sp.n, sp.d), dtype=torch.float32, device="cuda:0")
    say("unpinned host table")
    rc = ng.lib().ngram_embed_bag(ctypes.byref(t), rows.data_ptr(), sp.n, eN.data_ptr(), None)
    assert rc == -4, rc                                                # NGRAM_EHIP
    assert b"pinned" in ng.lib().ngram_last_error()
    eN2 = ng.ngram_embed_bag(di.table_obj(), rows)                   # a valid call still succeeds
    torch.cuda.synchronize()
    _, want_eN, _ = expected(h)
    assert np.array_equal(eN2.cpu().numpy().view(np.uint32), want_eN.view(np.uint32))


@pytest.mark.parametrize("lengths,history", [
    ((600, 0, 1, 2, 450, 3), False),          # 1056 tokens, 6 sequences: offsets staged in LDS
    ((6,) * 200, True),                       # 1200 tokens, 200 sequences with history: both staged
    ((4,) * 300, True),                       # 300 sequences: above the staging limit, global search
    ((1023, 1), False),                       # 1024 tokens exactly, 2 sequences
])
def test_sequence_lookup_staged_and_global(lengths, history):
    """Batches of at least 1024 tokens with 2..255 sequences look their
    sequence up in LDS copies of seq_offsets (and the history); more
    sequences, or smaller batches, search in global memory.  Both give the
    oracle's rows and outputs, through the fused and the unfused hash."""
    sp = Spec(f"seqs{len(lengths)}", lengths, 151936, 100_003, 64, table_kind=synth.KIND_BF16_WIDE,
              residual=True, history=history, config_id=27)
    h, di = check_spec(sp)
    rows = ng.ngram_hash(di.tokens, di.offsets, sp.R, history=di.history)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), oracle.hash_rows(h.tokens, h.offsets, sp.R, h.history))
