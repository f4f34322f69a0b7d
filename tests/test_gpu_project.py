"""GPU parity of the projection (ngram_project) and of the normalised, gated
epilogue on given sums (ngram_norm_gate_add), through the C ABI.

Projection bar: the oracle gives the exact-product sum in float64; the GPU
sums the same exact products in fp32 in its own order, so each output must
lie within tests.tolerance.project_bound of the oracle's value.  Where every
partial sum is an integer below 2^24 the fp32 result is exact in any order,
and there the outputs must be bit-identical; so must an identity weight's
(each output is one rounded input).

Epilogue bar: bit-identical to ngram_forward_gated for the same sums (the
same kernel code reads them instead of gathering them), and against the
oracle the gated path's bar (tests/test_gpu_gated.py).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_embedding_ngram_amd as ng  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from synth.workloads import DeviceInputs, HostInputs, Spec, gate_params  # noqa: E402
from tests.test_gpu_gated import compare  # noqa: E402
from tests.test_gpu_parity import bits16, say  # noqa: E402
from tests.tolerance import assert_project_close, gated_bounds  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a, dt=None):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a if dt is None else a.view(dt)).to(DEV)


def weights(d_out, d_in, seed):
    """bf16 bits of N(0, 1/d_in) weights."""
    w = (np.random.default_rng(seed).standard_normal((d_out, d_in)) / np.sqrt(d_in)).astype(np.float32)
    return (w.view(np.uint32) >> 16).astype(np.uint16)


def bf16_inputs(shape, scale, seed):
    """(bf16 bits, the same values as fp32) of scaled normal values, cut to
    bf16 by dropping the low half of each fp32."""
    v = (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)


def run_project(x_bits, P):
    y = ng.ngram_project(dev(x_bits, np.int16), dev(P, np.int16))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("n,d_in,d_out", [(300, 256, 384), (129, 2560, 256), (1, 64, 128), (128, 128, 2560),
                                          (4096, 128, 768),     # XCD runs of whole tile rows: column order
                                          (517, 640, 640), (65, 128, 72), (1000, 2560, 2560), (257, 64, 512),
                                          (40, 192, 8)])
def test_project_matches_oracle_within_the_fp32_bound(n, d_in, d_out):
    """Several 256 x 256 tiles, ragged last row and column tiles, K from one
    step of 64 to forty."""
    say(f"project n={n} d_in={d_in} d_out={d_out}")
    xb, x = bf16_inputs((n, d_in), 0.08, n * 7 + d_in)
    P = weights(d_out, d_in, d_out)
    got = run_project(xb, P)
    y64, a64 = oracle.project(x, P)
    r = assert_project_close(got, y64, a64, d_in, f"project {n}x{d_in}x{d_out}")
    say(f"  largest error {r:.3g} of the bound")


def test_project_integer_data_is_exact_in_any_order():
    """x, P integers in [-8, 8]: every partial sum is an integer below 2^24,
    so any fp32 order gives the exact value, bit for bit."""
    n, d_in, d_out = 333, 2560, 384
    rng = np.random.default_rng(11)
    x = rng.integers(-8, 9, size=(n, d_in)).astype(np.float32)
    Pf = rng.integers(-8, 9, size=(d_out, d_in)).astype(np.float32)
    P = (Pf.view(np.uint32) >> 16).astype(np.uint16)
    say("project integer data")
    got = run_project((x.view(np.uint32) >> 16).astype(np.uint16), P)
    y64, _ = oracle.project(x, P)
    assert np.array_equal(got.astype(np.float64), y64)


def test_project_identity_passes_each_input_through():
    """P = I: y = x exactly (each output is one input: the operand layouts
    and the output mapping, bit for bit), over large and subnormal values."""
    d = 256
    rng = np.random.default_rng(12)
    v = (rng.standard_normal((200, d)) * np.exp2(rng.integers(-30, 30, size=(200, d)))).astype(np.float32)
    v[0, :3] = [2.0 ** -130, 0.0, -(2.0 ** 100)]
    xb = (v.view(np.uint32) >> 16).astype(np.uint16)
    x = (xb.astype(np.uint32) << 16).view(np.float32)
    P = np.zeros((d, d), np.uint16)
    P[np.arange(d), np.arange(d)] = 0x3F80
    say("project identity")
    got = run_project(xb, P)
    want, _ = oracle.project(x, P)
    assert np.array_equal(got.astype(np.float64), want)
    assert np.array_equal(got, x)


def test_embed_bag_bf16_is_the_rounded_sum():
    """ngram_embed_bag_bf16 gives the oracle's fp32 sum rounded to bf16,
    bit for bit, with ties to even (1 + 2^-8 -> 1, 1 + 3 * 2^-8 ->
    1 + 2^-6), NaN for an invalid row, and on a workload's rows."""
    d = 64
    T = np.zeros((5, d), np.uint16)
    T[0] = 0x3F80                                   # 1.0
    T[1] = 0x3B80                                   # 2^-8
    T[2] = 0x3C40                                   # 3 * 2^-8
    rows = np.array([[0, 1] + [4] * 14, [0, 2] + [4] * 14, [3] * 15 + [-1], [0] * 16], np.int32)
    say("embed_bag_bf16 ties")
    out = ng.ngram_embed_bag_bf16(ng.Table(dev(T, np.int16), 5, d), dev(rows))
    torch.cuda.synchronize()
    got = bits16(out).reshape(4, d)
    assert np.all(got[0] == 0x3F80) and np.all(got[1] == 0x3F82) and np.all(got[2] == 0x7FC0)
    assert np.all(got[3] == 0x4180)                 # 16
    sp = GSPEC.replace(d=640)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
    out = ng.ngram_embed_bag_bf16(di.table_obj(), rows)
    torch.cuda.synchronize()
    from tests.oracle_ref import expected
    _, want_eN, _ = expected(h)
    assert np.array_equal(bits16(out).reshape(sp.n, sp.d), oracle.bf16_rne(want_eN).reshape(sp.n, sp.d))


def test_forward_without_gate_terms_gives_the_rounded_sums():
    """ngram_forward with W_g = 1 and neither e1 nor residual writes
    bf16(fmaf(1, s, +0)) = bf16(s) for every fp32 sum s (a sum that starts
    from +0 is never -0): the same bits as ngram_hash + ngram_embed_bag_bf16,
    also around invalid tokens (their rows NaN both ways).  The projected
    path's benchmark takes its sums this way, in one launch."""
    sp = GSPEC.replace(d=640)
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    tok = di.tokens.clone()
    tok[5] = -1
    tok[17] = (1 << 21) - 1                          # the pad id is not a real token
    say("forward W_g = 1 against embed_bag_bf16")
    rows = ng.ngram_hash(tok, di.offsets, sp.R)
    want = ng.ngram_embed_bag_bf16(di.table_obj(), rows)
    got = torch.empty(sp.n * sp.d, dtype=torch.int16, device=DEV)
    ng.ngram_forward(tok, di.offsets, di.table_obj(), torch.ones(sp.d, dtype=torch.float32, device=DEV), got)
    torch.cuda.synchronize()
    w, g = bits16(want).reshape(sp.n, sp.d), bits16(got).reshape(sp.n, sp.d)
    assert np.all(w[5] == 0x7FC0) and np.all(w[17] == 0x7FC0)
    assert np.array_equal(g, w)


def test_project_full_size_sampled():
    """32,768 x 2560 x 2560 (the prefill batch's sums): every output of 96
    sampled rows, including the first and the last, against the oracle."""
    n, d = 32768, 2560
    xb, x = bf16_inputs((n, d), 0.08, 5)
    P = weights(d, d, 13)
    say("project full size")
    y = ng.ngram_project(dev(xb, np.int16), dev(P, np.int16))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, n - 1], np.random.default_rng(3).integers(0, n, 91)]))
    y64, a64 = oracle.project(x[rows], P)
    got = y[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    r = assert_project_close(got, y64, a64, d, "project full size")
    say(f"  largest error {r:.3g} of the bound")


def test_project_empty_and_argument_errors():
    P = dev(weights(128, 64, 1), np.int16)
    y = ng.ngram_project(torch.empty((0, 64), dtype=torch.int16, device=DEV), P)
    assert y.shape == (0, 128)
    x = torch.zeros((4, 96), dtype=torch.int16, device=DEV)
    with pytest.raises(ng.NgramError, match="EINVAL"):
        ng.ngram_project(x, torch.zeros((128, 96), dtype=torch.int16, device=DEV))       # d_in not a multiple of 64
    x = torch.zeros((4, 64), dtype=torch.int16, device=DEV)
    with pytest.raises(ng.NgramError, match="EINVAL"):
        ng.ngram_project(x, torch.zeros((100, 64), dtype=torch.int16, device=DEV))       # d_out not a multiple of 8
    buf = torch.zeros(4 * 64 + 1, dtype=torch.int16, device=DEV)
    with pytest.raises(ng.NgramError, match="EALIGN"):
        ng.ngram_project(buf[1:].view(4, 64), P)


GSPEC = Spec("g_unfused", (1, 2, 250, 33, 300), 151936, 1_000_003, 2560, table_kind=synth.KIND_BF16_WIDE,
             residual=True, config_id=47)


@pytest.mark.parametrize("d,res", [(2560, True), (520, False), (8, True)])
def test_norm_gate_add_on_gathered_sums_equals_the_fused_kernel(d, res):
    sp = GSPEC.replace(d=d, residual=res)
    gp = gate_params(sp)
    say(f"norm_gate_add vs fused: d={d} res={res}")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    n = sp.n
    out_f = torch.empty(n * d, dtype=torch.int16, device=DEV)
    stats_f = torch.empty((n, 2), dtype=torch.float64, device=DEV)
    rows = torch.empty((n, 16), dtype=torch.int32, device=DEV)
    ng.ngram_forward_gated(di.tokens, di.offsets, di.table_obj(), di.W_g, t(gp.gamma), t(gp.u), t(gp.v), gp.b,
                           gp.eps, out_f, di.e1, residual=di.residual, history=di.history, rows_out=rows,
                           stats_out=stats_f)
    eN = ng.ngram_embed_bag(di.table_obj(), rows)
    out_u = torch.empty(n * d, dtype=torch.int16, device=DEV)
    stats_u = torch.empty((n, 2), dtype=torch.float64, device=DEV)
    ng.ngram_norm_gate_add(eN, di.tokens, di.e1, di.W_g, t(gp.gamma), t(gp.u), t(gp.v), gp.b, gp.eps, out_u,
                           residual=di.residual, stats_out=stats_u)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(out_u), bits16(out_f))
    assert np.array_equal(stats_u.cpu().numpy().view(np.uint64), stats_f.cpu().numpy().view(np.uint64))


def test_norm_gate_add_matches_oracle_and_invalid_ids_give_nan():
    """Sums from the seeded generator (not from a lookup), some token ids
    out of [0, V)."""
    n, d, V = 400, 1032, 5000
    rng = np.random.default_rng(21)
    eN = (rng.standard_normal((n, d)) * 0.1).astype(np.float32)
    tokens = rng.integers(0, V, size=n).astype(np.int32)
    tokens[[3, 77, n - 1]] = [V, -1, V + 100]
    e1 = ((rng.standard_normal((V, d)) * 0.02).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    res = ((rng.standard_normal((n, d)) * 0.5).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    W = rng.standard_normal(d).astype(np.float32)
    gp = gate_params(GSPEC.replace(d=d))
    say("norm_gate_add vs oracle")
    out = torch.empty(n * d, dtype=torch.int16, device=DEV)
    stats = torch.empty((n, 2), dtype=torch.float64, device=DEV)
    ng.ngram_norm_gate_add(dev(eN), dev(tokens), dev(e1, np.int16), dev(W), dev(gp.gamma), dev(gp.u), dev(gp.v),
                           gp.b, gp.eps, out, residual=dev(res, np.int16), stats_out=stats)
    torch.cuda.synchronize()
    got, st = bits16(out).reshape(n, d), stats.cpu().numpy()
    bad = (tokens < 0) | (tokens >= V)
    assert np.all((got[bad] & 0x7FFF) > 0x7F80) and np.all(np.isnan(st[bad]))
    ok = ~bad
    want, want_stats, y = oracle.norm_gate_add(eN[ok], tokens[ok], e1, W, gp.gamma, gp.u, gp.v, gp.b, gp.eps,
                                               res[ok])
    f = lambda b: (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    bounds = gated_bounds(eN[ok], f(e1[tokens[ok]]), f(res[ok]), W, gp.gamma, gp.u, gp.v, want_stats)
    compare(got[ok], st[ok], want, want_stats, y, bounds, "norm_gate_add")


def test_projected_path_stages():
    """Lookup, projection, normalisation and gate at a small shape: the GPU's
    bf16 sums equal the oracle's sums rounded to bf16 bit for bit, their
    projection lies within the bound of the oracle's projection, and the
    gated epilogue on the projected sums gives finite outputs for every
    (valid) token."""
    sp = GSPEC.replace(d=640)
    gp = gate_params(sp)
    say("projected path")
    h = HostInputs(sp)
    di = DeviceInputs(sp, h)
    rows = ng.ngram_hash(di.tokens, di.offsets, sp.R)
    x = ng.ngram_embed_bag_bf16(di.table_obj(), rows)
    P = weights(sp.d, sp.d, 31)
    p = ng.ngram_project(x, dev(P, np.int16))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = torch.empty(sp.n * sp.d, dtype=torch.int16, device=DEV)
    ng.ngram_norm_gate_add(p, di.tokens, di.e1, di.W_g, t(gp.gamma), t(gp.u), t(gp.v), gp.b, gp.eps, out,
                           residual=di.residual)
    torch.cuda.synchronize()
    from tests.oracle_ref import expected
    _, want_eN, _ = expected(h)
    assert np.array_equal(bits16(x).reshape(sp.n, sp.d), oracle.bf16_rne(want_eN).reshape(sp.n, sp.d))
    y64, a64 = oracle.project(want_eN, P)
    assert_project_close(p.cpu().numpy(), y64, a64, sp.d, "projected path: projection")
    o = bits16(out)
    assert not np.any((o & 0x7FFF) > 0x7F80)
