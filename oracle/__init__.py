"""Python access to the C oracle (``oracle/liboracle.so``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it; the product package never imports it.  Arguments are
numpy arrays on the host; the wrappers only marshal pointers.  ctypes releases
the GIL during each call, so independent calls may run on several threads.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB lets the mutation test load a deliberately broken copy.
LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
K = 16
PAD = (1 << 21) - 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I32 = ctypes.c_int32
        L.oracle_splitmix64.restype = ctypes.c_uint64
        L.oracle_splitmix64.argtypes = [ctypes.c_uint64]
        L.oracle_default_seeds.argtypes = [P]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_bf16_rne_array.argtypes = [P, I64, P]
        L.oracle_context.argtypes = [P, I64, P, I32, P, P]
        L.oracle_hash.argtypes = [P, I64, P, I32, P, P, I64, P]
        L.oracle_embed_bag_bf16.argtypes = [P, I64, I32, P, I64, P]
        L.oracle_embed_bag_int8.argtypes = [P, P, I64, I32, P, I64, P]
        L.oracle_gate_add.argtypes = [P, P, I64, I32, P, P, P, P]
        L.oracle_forward.argtypes = [P, I64, P, I32, P, P, I32, P, P, I64, I32,
                                     P, P, P, P, P, P]
        L.oracle_e2m1.restype = ctypes.c_float
        L.oracle_e2m1.argtypes = [ctypes.c_int]
        L.oracle_embed_bag_mxfp4.argtypes = [P, I64, I32, P, I64, P]
        L.oracle_grad_table_rows.argtypes = [P, I64, I32, P, P, P, I64, P]
        L.oracle_grad_e1_tokens.argtypes = [P, P, I64, I32, P, P, I64, P]
        L.oracle_grad_gate.argtypes = [P, P, P, I64, I32, P, P]
        F = ctypes.c_float
        L.oracle_bf16_rne_f64.restype = ctypes.c_uint16
        L.oracle_bf16_rne_f64.argtypes = [ctypes.c_double]
        L.oracle_norm_gate_add.argtypes = [P, P, I64, I32, P, P, P, P, P, F, F, P, P, P, P]
        L.oracle_project.argtypes = [P, I64, I32, P, I32, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def splitmix64(x: int) -> int:
    return int(lib().oracle_splitmix64(x & 0xFFFFFFFFFFFFFFFF))


def default_seeds() -> np.ndarray:
    s = np.zeros(K, dtype=np.uint64)
    lib().oracle_default_seeds(_p(s))
    return s


def bf16_rne(x) -> np.ndarray:
    x = _c(x, np.float32).reshape(-1)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_p(x), x.size, _p(out))
    return out


def context(tokens, seq_offsets, history=None) -> np.ndarray:
    t = _c(tokens, np.int32)
    so = _c(seq_offsets, np.int32)
    h = _c(history, np.int32)
    ctx = np.zeros((t.size, 3), dtype=np.int32)
    lib().oracle_context(_p(t), t.size, _p(so), so.size - 1, _p(h), _p(ctx))
    return ctx


def hash_rows(tokens, seq_offsets, R, history=None, seeds=None) -> np.ndarray:
    t = _c(tokens, np.int32)
    so = _c(seq_offsets, np.int32)
    h = _c(history, np.int32)
    sd = default_seeds() if seeds is None else _c(seeds, np.uint64)
    rows = np.zeros((t.size, K), dtype=np.int32)
    lib().oracle_hash(_p(t), t.size, _p(so), so.size - 1, _p(h), _p(sd), int(R), _p(rows))
    return rows


def embed_bag_bf16(T, rows) -> np.ndarray:
    T = _c(T, np.uint16)
    rows = _c(rows, np.int32)
    n = rows.shape[0]
    d = T.shape[1]
    eN = np.zeros((n, d), dtype=np.float32)
    lib().oracle_embed_bag_bf16(_p(T), T.shape[0], d, _p(rows), n, _p(eN))
    return eN


def embed_bag_int8(Q, scale, rows) -> np.ndarray:
    Q = _c(Q, np.int8)
    scale = _c(scale, np.float32)
    rows = _c(rows, np.int32)
    n = rows.shape[0]
    d = Q.shape[1]
    eN = np.zeros((n, d), dtype=np.float32)
    lib().oracle_embed_bag_int8(_p(Q), _p(scale), Q.shape[0], d, _p(rows), n, _p(eN))
    return eN


def e2m1(code: int) -> float:
    return float(lib().oracle_e2m1(int(code)))


def embed_bag_mxfp4(T, d, rows) -> np.ndarray:
    """``T``: uint8 [R][d/2 + d/32] MXFP4 rows."""
    T = _c(T, np.uint8)
    rows = _c(rows, np.int32)
    n = rows.shape[0]
    eN = np.zeros((n, d), dtype=np.float32)
    lib().oracle_embed_bag_mxfp4(_p(T), T.shape[0], d, _p(rows), n, _p(eN))
    return eN


def gate_add(eN, e1_rows, W_g, e1=None, residual=None) -> np.ndarray:
    eN = _c(eN, np.float32)
    n, d = eN.shape
    idx = _c(e1_rows, np.int32)
    e1 = _c(e1, np.uint16)
    W_g = _c(W_g, np.float32)
    res = _c(residual, np.uint16)
    out = np.zeros((n, d), dtype=np.uint16)
    lib().oracle_gate_add(_p(eN), _p(idx), n, d, _p(e1), _p(W_g), _p(res), _p(out))
    return out


def forward(tokens, seq_offsets, table, W_g, e1=None, residual=None, history=None,
            seeds=None, scale=None, mxfp4_d=None):
    """Whole path.  ``table`` is uint16 bf16 bits [R][d], int8 [R][d] with
    ``scale`` fp32 [R], or (``mxfp4_d`` = d) uint8 MXFP4 rows [R][d/2 + d/32].
    Returns (out bf16 bits [n][d], rows [n][16], eN fp32)."""
    t = _c(tokens, np.int32)
    so = _c(seq_offsets, np.int32)
    h = _c(history, np.int32)
    sd = default_seeds() if seeds is None else _c(seeds, np.uint64)
    is_int8 = np.asarray(table).dtype == np.int8
    if mxfp4_d is not None:
        tab = _c(table, np.uint8)
        R, d = tab.shape[0], int(mxfp4_d)
        dtype = 2
    else:
        tab = _c(table, np.int8 if is_int8 else np.uint16)
        R, d = tab.shape
        dtype = 1 if is_int8 else 0
    sc = _c(scale, np.float32)
    n = t.size
    out = np.zeros((n, d), dtype=np.uint16)
    rows = np.zeros((n, K), dtype=np.int32)
    eN = np.zeros((n, d), dtype=np.float32)
    lib().oracle_forward(_p(t), n, _p(so), so.size - 1, _p(h), _p(sd), dtype,
                         _p(tab), _p(sc), R, d, _p(_c(e1, np.uint16)), _p(_c(W_g, np.float32)),
                         _p(_c(residual, np.uint16)), _p(out), _p(rows), _p(eN))
    return out, rows, eN


def grad_table(rows, W_g, g, query=None):
    """(query rows, dT [nq][d] fp32).  ``g`` is bf16 bits [n][d]; ``query``
    defaults to every distinct valid row, ascending."""
    rows = _c(rows, np.int32)
    g = _c(g, np.uint16)
    n, d = g.shape
    if query is None:
        query = np.unique(rows[rows >= 0])
    query = _c(query, np.int32)
    out = np.zeros((query.size, d), dtype=np.float32)
    lib().oracle_grad_table_rows(_p(rows), n, d, _p(_c(W_g, np.float32)), _p(g), _p(query), query.size, _p(out))
    return query, out


def grad_e1(tokens, rows, g, query=None):
    """(query tokens, de1 [nq][d] fp32); ``query`` defaults to every distinct
    token of a valid position, ascending."""
    tokens = _c(tokens, np.int32)
    rows = _c(rows, np.int32).reshape(-1, K)
    g = _c(g, np.uint16)
    n, d = g.shape
    if query is None:
        query = np.unique(tokens[rows[:, 0] >= 0])
    query = _c(query, np.int32)
    out = np.zeros((query.size, d), dtype=np.float32)
    lib().oracle_grad_e1_tokens(_p(tokens), _p(rows), n, d, _p(g), _p(query), query.size, _p(out))
    return query, out


def grad_gate(rows, g, eN, with_f64=False):
    """dW_g fp32 [d] (the float64 sum rounded once); with ``with_f64`` also
    the float64 sum itself."""
    rows = _c(rows, np.int32)
    g = _c(g, np.uint16)
    eN = _c(eN, np.float32)
    n, d = g.shape
    out = np.zeros(d, dtype=np.float32)
    out64 = np.zeros(d, dtype=np.float64)
    lib().oracle_grad_gate(_p(rows), _p(g), _p(eN), n, d, _p(out), _p(out64))
    return (out, out64) if with_f64 else out


def bf16_rne_f64(x) -> np.ndarray:
    """float64 values rounded once to bf16 (bits), ties to even."""
    x = np.asarray(x, dtype=np.float64)
    L = lib()
    return np.array([L.oracle_bf16_rne_f64(float(v)) for v in x.reshape(-1)], dtype=np.uint16).reshape(x.shape)


def norm_gate_add(eN, e1_rows, e1, W_g, gamma, u, v, b, eps, residual=None):
    """Normalised, input-gated fusion of the sums eN [n][d], evaluated in
    float64.  Returns (out bf16 bits [n][d], stats float64 [n][2] = (r,
    logit), y float64 [n][d], the value rounded to out)."""
    eN = _c(eN, np.float32)
    n, d = eN.shape
    out = np.zeros((n, d), dtype=np.uint16)
    stats = np.zeros((n, 2), dtype=np.float64)
    y = np.zeros((n, d), dtype=np.float64)
    lib().oracle_norm_gate_add(_p(eN), _p(_c(e1_rows, np.int32)), n, d, _p(_c(e1, np.uint16)),
                               _p(_c(W_g, np.float32)), _p(_c(gamma, np.float32)), _p(_c(u, np.float32)),
                               _p(_c(v, np.float32)), float(np.float32(b)), float(np.float32(eps)),
                               _p(_c(residual, np.uint16)), _p(out), _p(stats), _p(y))
    return out, stats, y


def project(x, P):
    """Projection of the sums x [n][d_in] (fp32) by the bf16 weights P
    [d_out][d_in] (uint16 bits), x rounded to bf16 first; evaluated in
    float64.  Returns (y float64 [n][d_out], sum of |terms| float64
    [n][d_out])."""
    x = _c(x, np.float32)
    P = _c(P, np.uint16)
    n, d_in = x.shape
    d_out = P.shape[0]
    assert P.shape[1] == d_in
    y = np.zeros((n, d_out), dtype=np.float64)
    a = np.zeros((n, d_out), dtype=np.float64)
    lib().oracle_project(_p(x), n, d_in, _p(P), d_out, _p(y), _p(a))
    return y, a
