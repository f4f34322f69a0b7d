"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: every row id of the batch bit-exact against the oracle's
hash, and the bf16 outputs of 1024 sampled tokens (plus each sequence's first
three and last tokens) bit-exact against the oracle run on those tokens'
rows; on tables whose fp32 sums round, the test also shows that the checked
sums depend on the k = 0..15 order.

Memory: the 20M x 2560 bf16 table is 95.4 GiB of HBM; each test frees its
tensors before the next one allocates.
"""
import gc

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_embedding_ngram_amd as ng  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from synth.workloads import CONFIGS, DeviceInputs, HostInputs, Spec, fill_host_table  # noqa: E402
from tests.oracle_ref import expected, sample_tokens  # noqa: E402
from tests.test_gpu_parity import assert_bf16_equal, bits16, say  # noqa: E402

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _order_observable(h, idx, rows_all):
    """Fraction of the sampled tokens' fp32 sums that change when their 16
    rows are added in reversed order (the oracle on both orders): how much
    of the check below depends on the k = 0..15 order."""
    sp = h.spec
    rows_s = rows_all[idx]
    uniq, inv = np.unique(rows_s, return_inverse=True)
    remap = inv.reshape(rows_s.shape).astype(np.int32)
    rev = np.ascontiguousarray(remap[:, ::-1])
    Tc = h.table_rows(uniq)
    if sp.table == "int8":
        sc = h.scale_rows(uniq)
        a, b = oracle.embed_bag_int8(Tc, sc, remap), oracle.embed_bag_int8(Tc, sc, rev)
    elif sp.table == "mxfp4":
        a, b = oracle.embed_bag_mxfp4(Tc, sp.d, remap), oracle.embed_bag_mxfp4(Tc, sp.d, rev)
    else:
        a, b = oracle.embed_bag_bf16(Tc, remap), oracle.embed_bag_bf16(Tc, rev)
    return float(np.mean(a.view(np.uint32) != b.view(np.uint32)))


def _check_forward(name, table_kind=None, m=1024, min_order_share=None):
    sp = CONFIGS[name] if table_kind is None else CONFIGS[name].replace(table_kind=table_kind)
    say(f"full size {name}: n={sp.n} R={sp.R} d={sp.d} table={sp.table} kind={sp.table_kind}")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    out = di.residual if di.residual is not None else torch.empty(sp.n * sp.d, dtype=torch.int16, device="cuda:0")
    rows = torch.empty((sp.n, 16), dtype=torch.int32, device="cuda:0")
    ng.ngram_forward(di.tokens, di.offsets, di.table_obj(), di.W_g, out, e1=di.e1,
                     residual=di.residual, history=di.history, rows_out=rows)
    torch.cuda.synchronize()
    got_rows = rows.cpu().numpy()
    want_rows = oracle.hash_rows(h.tokens, h.offsets, sp.R, h.history)
    assert np.array_equal(got_rows, want_rows), "row ids differ"
    idx = sample_tokens(sp, m=m) if sp.n > m else np.arange(sp.n)
    _, _, want = expected(h, idx, rows_all=want_rows)
    got = bits16(out.view(sp.n, sp.d)[torch.from_numpy(idx).to("cuda:0")])
    assert_bf16_equal(got, want, name)
    if min_order_share is not None:
        share = _order_observable(h, idx, want_rows)
        say(f"full size {name}: {idx.size} tokens checked, {share:.0%} of their sums depend on the k order")
        assert share >= min_order_share
    del di, out, rows
    _free()


def test_prefill_full_size():
    _check_forward("prefill")


def test_prefill_full_size_wide_values():
    """The same 20M x 2560 table filled with wide-exponent bf16 values, whose
    fp32 sums round, so the check sees the k = 0..15 order."""
    _check_forward("prefill", table_kind=synth.KIND_BF16_WIDE, min_order_share=0.4)


@pytest.mark.parametrize("name", ["decode1", "decode2", "decode4"])
def test_decode_full_size(name):
    _check_forward(name)


def test_int8_full_size():
    """Row scales in [2^-11, 2^-10) make every fused multiply-add round, so
    the order is observable with the workload's own table."""
    _check_forward("int8", min_order_share=0.4)


def test_mxfp4_full_size():
    _check_forward("fp4")


def test_mxfp4_full_size_wide_scales():
    _check_forward("fp4", table_kind=synth.KIND_MXFP4_WIDE, min_order_share=0.2)


def test_host_table_full_size():
    """R = 5M x 2560 bf16 (23.8 GiB) in pinned host memory: the zero-copy sum
    and the staged path both equal the oracle on sampled tokens, and the host
    table gives bit-identical results to the same table resident in HBM."""
    sp = CONFIGS["host"]
    say(f"full size host: n={sp.n} R={sp.R} d={sp.d}")
    h = HostInputs(sp)
    hb = ng.HostBuffer(sp.R * sp.d * 2)
    try:
        fill_host_table(sp, hb.numpy(np.int16, (sp.R, sp.d)))
        di = DeviceInputs(sp, h, table=False)
        th = ng.Table(hb, sp.R, sp.d)
        rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
        eN_host = ng.ngram_embed_bag(th, rows)
        out = torch.empty(sp.n * sp.d, dtype=torch.int16, device="cuda:0")
        ng.ngram_gate_add(eN_host, di.tokens, di.W_g, out, e1=di.e1, residual=di.residual)
        torch.cuda.synchronize()
        want_rows = oracle.hash_rows(h.tokens, h.offsets, sp.R)
        assert np.array_equal(rows.cpu().numpy(), want_rows)
        idx = sample_tokens(sp, m=64)
        _, want_eN, want = expected(h, idx, rows_all=want_rows)
        tidx = torch.from_numpy(idx).to("cuda:0")
        assert np.array_equal(eN_host[tidx].cpu().numpy().view(np.uint32), want_eN.view(np.uint32))
        assert_bf16_equal(bits16(out.view(sp.n, sp.d)[tidx]), want, "host")

        for mode in (ng.GATHER_ZERO_COPY, ng.GATHER_ASYNC_COPY):
            say(f"host: staged gather, mode {mode}")
            stage = torch.empty((sp.n * 16, sp.d), dtype=torch.int16, device="cuda:0")
            remap = torch.empty((sp.n, 16), dtype=torch.int32, device="cuda:0")
            _, _, nst = ng.ngram_gather_host(th, rows, stage, remap, mode=mode)
            eN_stage = ng.ngram_embed_bag(ng.Table(stage, sp.n * 16, sp.d), remap)
            torch.cuda.synchronize()
            U = int(nst.item())
            assert U == np.unique(want_rows).size
            rm = remap.cpu().numpy()
            host = hb.numpy(np.int16, (sp.R, sp.d))
            pick = np.random.default_rng(mode).integers(0, sp.n * 16, 2000)
            assert np.array_equal(stage.cpu().numpy()[rm.reshape(-1)[pick]], host[want_rows.reshape(-1)[pick]])
            assert torch.equal(eN_stage.view(torch.int32), eN_host.view(torch.int32))
            del stage, remap, eN_stage
            _free()

        say("host: same table in HBM")
        dev_table = torch.from_numpy(hb.numpy(np.int16, (sp.R * sp.d,))).to("cuda:0")
        eN_dev = ng.ngram_embed_bag(ng.Table(dev_table, sp.R, sp.d), rows)
        torch.cuda.synchronize()
        assert torch.equal(eN_dev.view(torch.int32), eN_host.view(torch.int32))
        del dev_table, eN_dev, eN_host, out, rows, di
        _free()
    finally:
        hb.free()


@pytest.mark.parametrize("table,kind,d", [("bf16", 2, 8), ("int8", 4, 8), ("mxfp4", 7, 128)])
def test_forward_at_the_largest_row_count(table, kind, d):
    """R = 2^31 - 1 rows (the largest the ABI takes): row byte offsets pass
    2^32 (bf16: 32 GiB table; int8: 16 GiB + 8 GiB of scales; MXFP4 at 68 B
    per row: 136 GiB).  Every row id and every output equals the oracle."""
    sp = Spec(f"maxR_{table}", (300, 17, 1), 151936, 2**31 - 1, d, table=table, table_kind=kind,
              residual=True, config_id=31)
    say(f"largest R: {table} d={d}")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    out, rows = torch.empty(sp.n * d, dtype=torch.int16, device="cuda:0"), \
        torch.empty((sp.n, 16), dtype=torch.int32, device="cuda:0")
    ng.ngram_forward(di.tokens, di.offsets, di.table_obj(), di.W_g, out, e1=di.e1, residual=di.residual,
                     rows_out=rows)
    torch.cuda.synchronize()
    want_rows, _, want = expected(h)
    got_rows = rows.cpu().numpy()
    assert np.array_equal(got_rows, want_rows)
    assert got_rows.max() > 2**31 - 2**28                  # rows near the end of the table are read
    assert_bf16_equal(bits16(out).reshape(sp.n, d), want, sp.name)
    del di, out, rows
    _free()


def test_forward_output_beyond_2_31_elements():
    """2^22 tokens x d = 1024: the output holds 2^32 elements (8 GiB), so the
    output offsets pass 2^31; sampled tokens, including the last ones, equal
    the oracle, and every row id is checked."""
    n = 1 << 22
    sp = Spec("big_n", (n // 2, n // 2), 151936, 100_003, 1024, residual=True, config_id=32)
    say(f"output beyond 2^31 elements: n={sp.n} d={sp.d}")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    rows = torch.empty((sp.n, 16), dtype=torch.int32, device="cuda:0")
    ng.ngram_forward(di.tokens, di.offsets, di.table_obj(), di.W_g, di.residual, e1=di.e1,
                     residual=di.residual, rows_out=rows)
    torch.cuda.synchronize()
    want_rows = oracle.hash_rows(h.tokens, h.offsets, sp.R)
    assert np.array_equal(rows.cpu().numpy(), want_rows)
    idx = np.unique(np.concatenate([sample_tokens(sp, m=64), np.arange(n - 8, n)]))
    _, _, want = expected(h, idx, rows_all=want_rows)
    got = bits16(di.residual.view(sp.n, sp.d)[torch.from_numpy(idx).to("cuda:0")])
    assert_bf16_equal(got, want, sp.name)
    del di, rows
    _free()
