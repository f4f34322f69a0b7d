"""Expected values from the oracle for a synthetic workload, on all tokens or
on a sample of them.  For big tables only the rows the sample touches are
generated on the host (a compact table plus remapped row ids); the oracle's
steps are then run on those, which gives the same values as on the full
table because each output depends only on its own rows."""
import numpy as np

import oracle


def _sampled(h, sample, rows_all):
    """The oracle's row ids for all tokens, and for the sampled tokens their
    sums eN, their e1 row indices into a compact e1 (or the token ids when
    the workload has no e1), that compact e1 and their residual rows."""
    sp = h.spec
    if rows_all is None:
        rows_all = oracle.hash_rows(h.tokens, h.offsets, sp.R, h.history)
    idx = np.arange(sp.n) if sample is None else np.asarray(sample, dtype=np.int64)
    rows_s = rows_all[idx]
    uniq, inv = np.unique(rows_s, return_inverse=True)
    remap = inv.reshape(rows_s.shape).astype(np.int32)
    Tc = h.table_rows(uniq)
    if sp.table == "int8":
        eN = oracle.embed_bag_int8(Tc, h.scale_rows(uniq), remap)
    elif sp.table == "mxfp4":
        eN = oracle.embed_bag_mxfp4(Tc, sp.d, remap)
    else:
        eN = oracle.embed_bag_bf16(Tc, remap)
    toks = h.tokens[idx]
    e1c = None
    if sp.e1:
        u1, inv1 = np.unique(toks, return_inverse=True)
        e1c, ids = h.e1_rows(u1), inv1.astype(np.int32)
    else:
        ids = toks
    res = h.residual_rows(idx) if sp.residual else None
    return rows_all, eN, ids, e1c, res


def expected(h, sample=None, rows_all=None):
    """(rows [n][16] for all tokens, eN [m][d], out [m][d] bf16 bits) for the
    m sampled tokens (all tokens when ``sample`` is None)."""
    rows_all, eN, ids, e1c, res = _sampled(h, sample, rows_all)
    out = oracle.gate_add(eN, ids, h.W_g, e1c, res)
    return rows_all, eN, out


def expected_gated(h, gp, sample=None, rows_all=None):
    """The normalised, gated fusion with parameters ``gp``: (rows [n][16],
    out [m][d] bf16 bits, stats [m][2] float64 = (r, logit), y [m][d]
    float64, bounds = (r [m], logit [m], y [m][d]): how far another float64
    evaluation may lie from the oracle's, see tests.tolerance)."""
    from tests.tolerance import gated_bounds
    rows_all, eN, ids, e1c, res = _sampled(h, sample, rows_all)
    out, stats, y = oracle.norm_gate_add(eN, ids, e1c, h.W_g, gp.gamma, gp.u, gp.v, gp.b, gp.eps, res)
    f = lambda b: (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    bounds = gated_bounds(eN, f(e1c[ids]), f(res) if res is not None else None, h.W_g, gp.gamma, gp.u, gp.v,
                          stats)
    return rows_all, out, stats, y, bounds


def sample_tokens(spec, m=64, seed=0):
    """Sequence starts and ends (positions 0, 1, 2, last) plus random tokens."""
    offs = np.concatenate([[0], np.cumsum(spec.lengths)])
    pick = []
    for s in range(len(spec.lengths)):
        a, b = int(offs[s]), int(offs[s + 1])
        pick += [i for i in (a, a + 1, a + 2, b - 1) if a <= i < b]
    rng = np.random.default_rng(seed)
    pick += list(rng.integers(0, spec.n, size=m))
    return np.unique(np.array(pick, dtype=np.int64))
