"""The allocation-free gate gradient, ngram_grad_gate_noalloc, through the C
ABI: bit-identical to ngram_grad_gate (which takes a caller's workspace) on
the same inputs, on two calls in a row, the second with a smaller input (so
partials the first call left in the shared static scratch would show), and
a refusal, before anything is launched, of sizes beyond its scratch."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_embedding_ngram_amd as ng  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from tests.test_gpu_parity import say  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(n, d, seed):
    offs = synth.ragged_offsets([n])
    toks = synth.tokens(seed, n, 151936, 1.1)
    rows = oracle.hash_rows(toks, offs, 100_003)
    rows[n // 3] = -1                                   # an invalid token contributes nothing
    g = synth.tensor(synth.KIND_BF16_WIDE, seed, synth.TAG_RESIDUAL, n * d).reshape(n, d)
    eN = (synth.as_f32(synth.tensor(synth.KIND_F32_UNIT, seed, synth.TAG_TABLE, n * d)).reshape(n, d) - 0.5)
    eN = eN.astype(np.float32)
    eN[n // 3] = np.nan
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(DEV)
    return t(rows, np.int32), t(g, np.int16), t(eN, np.float32)


def test_noalloc_equals_the_workspace_call_on_two_calls_in_a_row():
    for n, d, seed in ((20_000, 2560, 1), (300, 520, 2)):
        say(f"gate gradient without allocation n={n} d={d}")
        rows, g, eN = _inputs(n, d, seed)
        want = ng.ngram_grad_gate(rows, g, eN)
        got = ng.ngram_grad_gate_noalloc(rows, g, eN)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32))
        assert bool(torch.isfinite(got).all())


def test_noalloc_refuses_sizes_beyond_its_scratch():
    L = ng.lib()
    cap = int(L.ngram_grad_gate_noalloc_max_elements())
    assert cap == (16 << 20) // 8
    d = 2560
    n_ok = (cap // d) * 128                              # ceil(n/128) * d <= cap
    n_bad = n_ok + 1
    rows, g, eN = _inputs(8, 64, 3)                      # buffers are not read: the call is refused first
    out = torch.empty(d, dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.ngram_grad_gate_noalloc(p(rows), p(g), p(eN), n_bad, d, p(out), s) == -3      # NGRAM_ERANGE
    assert b"static scratch" in L.ngram_last_error()
    assert L.ngram_grad_gate_noalloc(p(rows), p(g), p(eN), -1, d, p(out), s) == -1         # NGRAM_EINVAL
