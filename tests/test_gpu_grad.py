"""GPU gradients against the oracle: the distinct row and token lists
(ascending) and every fp32 table and e1 gradient value bit for bit (both sides
run the same stated fp32 order); the gate gradient, a plain sum accumulated in
float64 and rounded once, equal to the oracle's rounding except where an fp32
midpoint lies within the bound two float64 sums of the same terms can differ
by (tests.tolerance)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_embedding_ngram_amd as ng  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from tests.test_gpu_parity import say  # noqa: E402
from tests.tolerance import assert_f32_rounded_once, sum_bound  # noqa: E402

pytestmark = pytest.mark.gpu


def _inputs(lengths, R, V, d, seed, kind=synth.KIND_BF16_WIDE, bad=()):
    offs = synth.ragged_offsets(lengths)
    n = int(offs[-1])
    toks = synth.tokens(seed, n, V, 1.1)
    rows = oracle.hash_rows(toks, offs, R)
    for b in bad:
        rows[b] = -1
    g = synth.tensor(kind, seed, synth.TAG_RESIDUAL, n * d).reshape(n, d)
    W = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, seed, synth.TAG_WG, d))
    return toks, rows, g, W


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a).view(dt) if a.dtype != dt else a).to("cuda:0")


@pytest.mark.parametrize("lengths,R,d,bad", [
    ((40, 0, 57), 61, 64, ()),              # long groups, ragged unroll tails
    ((300, 7), 100_003, 520, (3, 17)),      # invalid tokens, ragged slices
    ((2000,), 4001, 2560, ()),              # 16 sort tiles, 8 group-numbering tiles (32000 items)
    ((1,), 7, 8, ()),
    ((50,), 3, 136, ()),                    # groups of hundreds of items (several 64-item blocks)
    ((200,), 3, 136, (7,)),                 # groups of about 1000 items: the long-group walk
    ((700, 333), 11, 2568, ()),             # long groups, a ragged last column block
    ((90, 3), 500, 9216, (2,)),             # 18 whole slices: each of 16 wavefronts walks two in turn
])
def test_table_grad(lengths, R, d, bad):
    say(f"grad table {lengths} R={R} d={d}")
    toks, rows, g, W = _inputs(lengths, R, 151936, d, seed=len(lengths) + R, bad=bad)
    gr, gv, nu = ng.ngram_grad_table(_dev(rows, np.int32), _dev(W, np.float32), _dev(g.view(np.int16), np.int16), R)
    torch.cuda.synchronize()
    U = int(nu.item())
    q, want = oracle.grad_table(rows, W, g)
    assert U == q.size
    assert np.array_equal(gr.cpu().numpy()[:U], q)
    assert np.array_equal(gv.cpu().numpy()[:U].view(np.uint32), want.view(np.uint32))


def test_table_grad_long_group_edges():
    """The long-group walk at its edges: groups of exactly 512 (walked
    with the short groups), 513 and 577 items (nine and ten 64-item units,
    the last one ragged), spread over the batch's positions, beside random
    short groups; d = 200 leaves a ragged 64-column slice."""
    n, R, d = 120, 50, 200
    rng = np.random.default_rng(11)
    ids = np.concatenate([np.full(513, 5), np.full(512, 9), np.full(577, 2),
                          rng.choice([r for r in range(R) if r not in (2, 5, 9)], n * 16 - 1602)])
    rows = rng.permutation(ids).astype(np.int32).reshape(n, 16)
    say("grad table long-group edges")
    g = synth.tensor(synth.KIND_BF16_WIDE, 12, synth.TAG_RESIDUAL, n * d).reshape(n, d)
    W = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 12, synth.TAG_WG, d))
    gr, gv, nu = ng.ngram_grad_table(_dev(rows, np.int32), _dev(W, np.float32), _dev(g.view(np.int16), np.int16), R)
    torch.cuda.synchronize()
    U = int(nu.item())
    q, want = oracle.grad_table(rows, W, g)
    assert U == q.size
    assert np.array_equal(gr.cpu().numpy()[:U], q)
    assert np.array_equal(gv.cpu().numpy()[:U].view(np.uint32), want.view(np.uint32))


def test_table_grad_more_long_groups_than_walkers():
    """About 100 groups longer than 512 items, more than the long-group
    walk's 64 workgroup rows, so each row takes several groups in turn;
    d = 72 (a 64-column slice and an 8-column one)."""
    n, R, d = 5000, 100, 72
    say("grad table 5000 tokens R=100")
    toks, rows, g, W = _inputs((n,), R, 151936, d, seed=13)
    assert (np.unique(rows, return_counts=True)[1] > 512).sum() > 64
    gr, gv, nu = ng.ngram_grad_table(_dev(rows, np.int32), _dev(W, np.float32), _dev(g.view(np.int16), np.int16), R)
    torch.cuda.synchronize()
    U = int(nu.item())
    q, want = oracle.grad_table(rows, W, g)
    assert U == q.size
    assert np.array_equal(gr.cpu().numpy()[:U], q)
    assert np.array_equal(gv.cpu().numpy()[:U].view(np.uint32), want.view(np.uint32))


def test_table_grad_many_items_sampled():
    """70000 tokens (1.12M sort items, multi-tile histogram scans): the
    distinct-row list in full, gradients of sampled rows (the most frequent
    ones and random ones)."""
    n, R, d = 70_000, 2_000_003, 64
    say("grad table 70000 tokens")
    toks, rows, g, W = _inputs((n,), R, 151936, d, seed=5)
    gr, gv, nu = ng.ngram_grad_table(_dev(rows, np.int32), _dev(W, np.float32), _dev(g.view(np.int16), np.int16), R)
    torch.cuda.synchronize()
    U = int(nu.item())
    uniq, cnt = np.unique(rows, return_counts=True)
    assert U == uniq.size and np.array_equal(gr.cpu().numpy()[:U], uniq)
    rng = np.random.default_rng(1)
    pick = np.unique(np.concatenate([np.argsort(-cnt)[:20], rng.integers(0, U, 30)]))
    _, want = oracle.grad_table(rows, W, g, query=uniq[pick])
    assert np.array_equal(gv.cpu().numpy()[pick].view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("lengths,V,d,bad", [((40, 0, 57), 13, 64, ()), ((300, 7), 1024, 520, (3, 17)),
                                             ((5000,), 151936, 128, ()),
                                             ((3000,), 3, 520, (5,)),         # tokens of ~1000 items: long walk
                                             ((20000,), 151936, 2560, ()),    # prefill-like Zipf head
                                             ((400, 5), 64, 9216, (3,))])     # 18 whole slices, looped
def test_e1_grad(lengths, V, d, bad):
    say(f"grad e1 {lengths} V={V}")
    toks, rows, g, W = _inputs(lengths, 4096, V, d, seed=7, bad=bad)
    gt, gv, nu = ng.ngram_grad_e1(_dev(toks, np.int32), _dev(rows, np.int32), _dev(g.view(np.int16), np.int16), V)
    torch.cuda.synchronize()
    U = int(nu.item())
    q, want = oracle.grad_e1(toks, rows, g)
    assert U == q.size
    assert np.array_equal(gt.cpu().numpy()[:U], q)
    assert np.array_equal(gv.cpu().numpy()[:U].view(np.uint32), want.view(np.uint32))


def test_e1_grad_long_group_edges():
    """The e1 gradient's long-token walk at its edges: tokens of exactly 64
    items (walked with the short groups), 65 and 129 items (the long-group
    walk, a ragged last unit), spread over the batch, beside random short
    groups; d = 200 leaves a ragged 64-column slice."""
    n, V, d = 1200, 1024, 200
    rng = np.random.default_rng(21)
    toks = np.concatenate([np.full(65, 5), np.full(64, 9), np.full(129, 2),
                           rng.choice([v for v in range(V) if v not in (2, 5, 9)], n - 258)])
    toks = rng.permutation(toks).astype(np.int32)
    offs = synth.ragged_offsets((n,))
    rows = oracle.hash_rows(toks, offs, 4096)
    say("grad e1 long-group edges")
    g = synth.tensor(synth.KIND_BF16_WIDE, 22, synth.TAG_RESIDUAL, n * d).reshape(n, d)
    gt, gv, nu = ng.ngram_grad_e1(_dev(toks, np.int32), _dev(rows, np.int32), _dev(g.view(np.int16), np.int16), V)
    torch.cuda.synchronize()
    U = int(nu.item())
    q, want = oracle.grad_e1(toks, rows, g)
    assert U == q.size
    assert np.array_equal(gt.cpu().numpy()[:U], q)
    assert np.array_equal(gv.cpu().numpy()[:U].view(np.uint32), want.view(np.uint32))

@pytest.mark.parametrize("n,d", [(1, 8), (255, 64), (257, 64), (263, 520), (1000, 2560), (515, 1032)])
def test_gate_grad(n, d):
    say(f"grad gate n={n} d={d}")
    toks, rows, g, W = _inputs((n,), 4096, 1024, d, seed=9)
    rows[n // 2] = -1
    eN = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 11, synth.TAG_TABLE, n * d)).reshape(n, d) - 0.5
    eN = eN.astype(np.float32)
    eN[n // 2] = np.nan                      # an invalid token's sum is never read
    gw = ng.ngram_grad_gate(_dev(rows, np.int32), _dev(g.view(np.int16), np.int16), _dev(eN, np.float32))
    torch.cuda.synchronize()
    check_gate(gw.cpu().numpy(), rows, g, eN, f"dW_g n={n} d={d}")


def check_gate(got, rows, g, eN, what):
    _, want64 = oracle.grad_gate(rows, g, eN, with_f64=True)
    valid = rows.reshape(-1, 16)[:, 0] >= 0
    gf = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mag = (np.abs(gf[valid]) * np.abs(eN[valid].astype(np.float64))).sum(axis=0)
    near = assert_f32_rounded_once(got, want64, sum_bound(int(valid.sum()), mag), what)
    say(f"{what}: {got.size} values, {near} at an fp32 midpoint within the bound")


def test_grads_on_two_streams_equal_one_stream():
    """The e1 and gate gradients on a side stream with their own workspace,
    beside the table gradient on the main stream, give the same bits as the
    three calls in order on one stream."""
    say("grads on two streams")
    n, d, R, V = 3000, 520, 50_003, 151936
    toks, rows, g, W = _inputs((1000, 2000), R, V, d, seed=21)
    eN = (synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 22, synth.TAG_TABLE, n * d)).reshape(n, d) - 0.5)
    t, r, gg, w, e = (_dev(toks, np.int32), _dev(rows, np.int32), _dev(g.view(np.int16), np.int16),
                      _dev(W, np.float32), _dev(eN.astype(np.float32), np.float32))
    ws1, ws2 = ng.grad_workspace(n, d), ng.grad_workspace(n, d)
    serial = (ng.ngram_grad_table(r, w, gg, R, workspace=ws1), ng.ngram_grad_e1(t, r, gg, V, workspace=ws1),
              ng.ngram_grad_gate(r, gg, e, workspace=ws1))
    torch.cuda.synchronize()
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record(main)
    side.wait_event(ev)
    e1g = ng.ngram_grad_e1(t, r, gg, V, workspace=ws2, stream=side)
    gate = ng.ngram_grad_gate(r, gg, e, workspace=ws2, stream=side)
    tab = ng.ngram_grad_table(r, w, gg, R, workspace=ws1, stream=main)
    torch.cuda.synchronize()
    for a, b in ((serial[0], tab), (serial[1], e1g)):
        U = int(a[2].item())
        assert U == int(b[2].item())
        assert torch.equal(a[0][:U], b[0][:U]) and torch.equal(a[1][:U].view(torch.int32), b[1][:U].view(torch.int32))
    assert torch.equal(serial[2].view(torch.int32), gate.view(torch.int32))


def test_empty_grads():
    z = torch.zeros((0, 16), dtype=torch.int32, device="cuda:0")
    gr, gv, nu = ng.ngram_grad_table(z, torch.ones(8, device="cuda:0"), torch.zeros((0, 8), dtype=torch.int16,
                                                                                   device="cuda:0"), 10)
    torch.cuda.synchronize()
    assert int(nu.item()) == 0


def test_full_prefill_backward_sampled():
    """Prefill shape (8 x 4096 tokens, R = 20M, d = 2560): table, e1 and gate
    gradients of sampled rows / tokens / all columns, bit-exact."""
    from synth.workloads import CONFIGS, HostInputs
    sp = CONFIGS["prefill"]
    say("grad prefill shape")
    h = HostInputs(sp)
    rows = oracle.hash_rows(h.tokens, h.offsets, sp.R)
    n, d = sp.n, sp.d
    g = synth.tensor(synth.KIND_BF16_NORMAL6, 3, synth.TAG_RESIDUAL, n * d).reshape(n, d)
    W = h.W_g
    t_rows = _dev(rows, np.int32)
    t_g = _dev(g.view(np.int16), np.int16)
    gr, gv, nu = ng.ngram_grad_table(t_rows, _dev(W, np.float32), t_g, sp.R)
    gt, ge, nt = ng.ngram_grad_e1(_dev(h.tokens, np.int32), t_rows, t_g, sp.V)
    eN = (synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 4, synth.TAG_TABLE, n * d)).reshape(n, d) - 0.5).astype(np.float32)
    gw = ng.ngram_grad_gate(t_rows, t_g, _dev(eN, np.float32))
    torch.cuda.synchronize()
    uniq, cnt = np.unique(rows, return_counts=True)
    U = int(nu.item())
    assert U == uniq.size and np.array_equal(gr.cpu().numpy()[:U], uniq)
    rng = np.random.default_rng(2)
    # every row with 64 or more items (the long chains) and 1000 random rows
    pick = np.unique(np.concatenate([np.nonzero(cnt >= 64)[0], rng.integers(0, U, 1000)]))
    say(f"grad prefill: checking {pick.size} of {U} table rows ({int((cnt >= 64).sum())} with >= 64 items, "
        f"longest {cnt.max()})")
    _, want = oracle.grad_table(rows, W, g, query=uniq[pick])
    assert np.array_equal(gv[torch.from_numpy(pick).cuda()].cpu().numpy().view(np.uint32), want.view(np.uint32))
    ut, ct = np.unique(h.tokens, return_counts=True)
    assert int(nt.item()) == ut.size and np.array_equal(gt.cpu().numpy()[:ut.size], ut)
    tp = np.unique(np.concatenate([[0, 1, 2], np.nonzero(ct >= 64)[0], rng.integers(0, ut.size, 200)]))
    say(f"grad prefill: checking {tp.size} of {ut.size} e1 rows (longest {ct.max()} items)")
    _, want_e = oracle.grad_e1(h.tokens, rows, g, query=ut[tp])
    assert np.array_equal(ge[torch.from_numpy(tp).cuda()].cpu().numpy().view(np.uint32), want_e.view(np.uint32))
    check_gate(gw.cpu().numpy(), rows, g, eN, "dW_g prefill")
