"""HIP-graph capture: replays of a captured forward (decode steps with
history, and a prefill-sized batch) and of the captured backward give the
bits of the same calls run eagerly, on every replay, with eager work and
synchronisations between the replays."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_embedding_ngram_amd as ng  # noqa: E402
import synth  # noqa: E402
from synth.workloads import DeviceInputs, HostInputs, Spec  # noqa: E402
from tests.test_gpu_parity import say  # noqa: E402

pytestmark = pytest.mark.gpu


def _forward_calls(sp, batches):
    base = DeviceInputs(sp.replace(batch=0))
    T = base.table_obj()
    ins = []
    for b in range(batches):
        h = HostInputs(sp.replace(batch=b))
        di = DeviceInputs(sp.replace(batch=b), h, table=False, e1=False)
        out = torch.empty(sp.n * sp.d, dtype=torch.int16, device="cuda:0")
        ins.append((di, out))

    def run():
        for di, out in ins:
            ng.ngram_forward(di.tokens, di.offsets, T, base.W_g, out, e1=base.e1, residual=None,
                             history=di.history)
    return run, [o for _, o in ins]


@pytest.mark.parametrize("sp", [
    Spec("graph_decode", (1, 1, 1, 1), 151936, 100_003, 2560, history=True, table_kind=synth.KIND_BF16_WIDE,
         config_id=50),
    Spec("graph_prefill", (700, 500), 151936, 100_003, 2560, table_kind=synth.KIND_BF16_WIDE, config_id=51),
])
def test_forward_graph_replays_equal_eager(sp):
    say(f"graph replays {sp.name}")
    run, outs = _forward_calls(sp, 3)
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        run()                                   # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run()
    for rep in range(4):
        for o in outs:
            o.fill_(0x1234)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs"


def test_backward_graph_replays_equal_eager():
    say("graph replays backward")
    n, d, R, V = 3000, 520, 50_003, 151936
    offs = synth.ragged_offsets((1000, 2000))
    toks = synth.tokens(61, n, V, 1.1)
    import oracle
    rows = oracle.hash_rows(toks, offs, R)
    g = synth.tensor(synth.KIND_BF16_WIDE, 61, synth.TAG_RESIDUAL, n * d).reshape(n, d)
    W = synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 61, synth.TAG_WG, d))
    eN = (synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, 62, synth.TAG_TABLE, n * d)).reshape(n, d) - 0.5)
    dev = "cuda:0"
    t, r = torch.from_numpy(toks).to(dev), torch.from_numpy(rows).to(dev)
    gg = torch.from_numpy(g.view(np.int16)).to(dev)
    w, e = torch.from_numpy(W).to(dev), torch.from_numpy(eN.astype(np.float32)).to(dev)
    ws = ng.grad_workspace(n, d)
    gr = torch.empty(n * 16, dtype=torch.int32, device=dev)
    gt = torch.empty((n * 16, d), dtype=torch.float32, device=dev)
    nu = torch.empty(1, dtype=torch.int64, device=dev)
    et = torch.empty(n, dtype=torch.int32, device=dev)
    ge = torch.empty((n, d), dtype=torch.float32, device=dev)
    ne = torch.empty(1, dtype=torch.int64, device=dev)
    gw = torch.empty(d, dtype=torch.float32, device=dev)

    def run():
        ng.ngram_grad_table(r, w, gg, R, grad_rows_out=gr, grad_out=gt, n_unique_out=nu, workspace=ws)
        ng.ngram_grad_e1(t, r, gg, V, grad_tokens_out=et, grad_out=ge, n_unique_out=ne, workspace=ws)
        ng.ngram_grad_gate(r, gg, e, grad_Wg_out=gw, workspace=ws)

    run()
    torch.cuda.synchronize()
    U, Ue = int(nu.item()), int(ne.item())
    eager = (gr[:U].clone(), gt[:U].clone(), et[:Ue].clone(), ge[:Ue].clone(), gw.clone())
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        run()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            run()
    for rep in range(4):
        for x in (gr, gt, et, ge, gw, nu, ne):
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(nu.item()) == U and int(ne.item()) == Ue
        got = (gr[:U], gt[:U], et[:Ue], ge[:Ue], gw)
        for a, b in zip(got, eager):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), f"replay {rep} differs"
