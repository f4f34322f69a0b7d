"""Expected values from the oracle for a synthetic workload, on all tokens or
on a sample of them.  For big tables only the rows the sample touches are
generated on the host (a compact table plus remapped row ids); the oracle's
steps are then run on those, which gives the same values as on the full
table because each output depends only on its own rows."""
import numpy as np

import oracle


def expected(h, sample=None, rows_all=None):
    """(rows [n][16] for all tokens, eN [m][d], out [m][d] bf16 bits) for the
    m sampled tokens (all tokens when ``sample`` is None)."""
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
    e1c = ids = None
    if sp.e1:
        u1, inv1 = np.unique(toks, return_inverse=True)
        e1c, ids = h.e1_rows(u1), inv1.astype(np.int32)
    else:
        ids = toks
    res = h.residual_rows(idx) if sp.residual else None
    out = oracle.gate_add(eN, ids, h.W_g, e1c, res)
    return rows_all, eN, out


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
