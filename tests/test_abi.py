"""The C ABI without a GPU: the library loads, exports every entry point that
include/ngram.h declares, and rejects bad arguments on the host (before any
HIP call) with the documented status codes."""
import ctypes
import os
import re

import numpy as np
import pytest

import hashed_gram_embedding_ngram_amd as ng
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ngram.h")
OK, EINVAL, EALIGN, ERANGE, EHIP, ENOTSUP = 0, -1, -2, -3, -4, -5
A = 0x10000          # a fake, 16-byte aligned device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ngram_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    L = ctypes.CDLL(ng.LIB_PATH)
    for name in names:
        assert hasattr(L, name), f"{name} declared in ngram.h but not exported"
    assert set(names) == set(ng._SIGNATURES), "binding and header disagree"


def test_status_strings_and_version():
    L = ng.lib()
    for s in (OK, EINVAL, EALIGN, ERANGE, EHIP, ENOTSUP):
        assert L.ngram_status_string(s)
    assert L.ngram_version() >= 1


def test_default_seeds_equal_the_oracle_seeds():
    # host code only: no GPU needed
    assert ng.default_seeds() == [int(s) for s in oracle.default_seeds()]


def _table(data=A, scale=None, R=1000, d=64, dtype=0, loc=0):
    return ng._Table(data, scale, R, d, dtype, loc, 0)


def _err():
    return ng.lib().ngram_last_error().decode()


def test_hash_argument_checks():
    L = ng.lib()
    seeds = None
    assert L.ngram_hash(A, -1, A, 1, None, seeds, 10, A, None) == EINVAL
    assert L.ngram_hash(None, 5, A, 1, None, seeds, 10, A, None) == EINVAL
    assert L.ngram_hash(A, 5, None, 1, None, seeds, 10, A, None) == EINVAL
    assert L.ngram_hash(A, 5, A, 0, None, seeds, 10, A, None) == EINVAL
    assert L.ngram_hash(A, 5, A, 1, None, seeds, 0, A, None) == ERANGE
    assert L.ngram_hash(A, 5, A, 1, None, seeds, 2**31, A, None) == ERANGE
    assert "R=" in _err()
    assert L.ngram_hash(A, 5, A, 1, None, seeds, 10, None, None) == EINVAL
    assert L.ngram_hash(A, 2**31, A, 1, None, seeds, 10, A, None) == ERANGE
    assert L.ngram_hash(None, 0, None, 0, None, seeds, 10, None, None) == OK   # empty: no launch


@pytest.mark.parametrize("kw,code", [
    (dict(data=None), EINVAL), (dict(R=0), ERANGE), (dict(R=2**31), ERANGE),
    (dict(d=12), EINVAL), (dict(d=0), EINVAL), (dict(d=-8), EINVAL), (dict(d=65544), ERANGE),
    (dict(data=A + 2), EALIGN), (dict(dtype=7), EINVAL), (dict(dtype=1), EINVAL),
    (dict(dtype=1, scale=A + 1), EALIGN), (dict(dtype=1, data=A + 4, scale=A), EALIGN),
    (dict(loc=5), EINVAL),
])
def test_table_checks(kw, code):
    L = ng.lib()
    t = _table(**kw)
    assert L.ngram_embed_bag(ctypes.byref(t), A, 4, A, None) == code, _err()
    assert L.ngram_forward(A, 4, A, 1, None, None, ctypes.byref(t), None, 0, A, None, A, None, None) == code


def test_embed_bag_checks():
    L = ng.lib()
    t = _table()
    assert L.ngram_embed_bag(None, A, 4, A, None) == EINVAL
    assert L.ngram_embed_bag(ctypes.byref(t), A, -1, A, None) == EINVAL
    assert L.ngram_embed_bag(ctypes.byref(t), None, 4, A, None) == EINVAL
    assert L.ngram_embed_bag(ctypes.byref(t), A, 4, None, None) == EINVAL
    assert L.ngram_embed_bag(ctypes.byref(t), A, 4, A + 4, None) == EALIGN
    assert L.ngram_embed_bag(ctypes.byref(t), None, 0, None, None) == OK
    t8 = _table(dtype=1, data=A + 8, scale=A + 4)            # int8: 8-byte data alignment
    assert L.ngram_embed_bag(ctypes.byref(t8), None, 0, None, None) == OK


def test_gate_add_checks():
    L = ng.lib()
    assert L.ngram_gate_add(A, A, 4, 12, None, 0, A, None, A, None) == EINVAL
    assert L.ngram_gate_add(A, A, 4, 65544, None, 0, A, None, A, None) == ERANGE
    assert L.ngram_gate_add(A, A, 4, 64, None, 0, None, None, A, None) == EINVAL
    assert L.ngram_gate_add(A, A, 4, 64, A, 0, A, None, A, None) == ERANGE
    assert L.ngram_gate_add(A, A, 4, 64, None, 0, A, None, None, None) == EINVAL
    assert L.ngram_gate_add(A, A, 4, 64, None, 0, A, None, A + 2, None) == EALIGN
    assert L.ngram_gate_add(A, A, 4, 64, None, 0, A + 4, None, A, None) == EALIGN
    assert L.ngram_gate_add(A, A, 4, 64, A, 10, A, A + 8, A, None) == EALIGN
    assert L.ngram_gate_add(A, A, -4, 64, None, 0, A, None, A, None) == EINVAL
    assert L.ngram_gate_add(None, None, 0, 64, None, 0, A, None, None, None) == OK


def test_forward_checks():
    L = ng.lib()
    t = ctypes.byref(_table())
    assert L.ngram_forward(A, 4, A, 1, None, None, t, None, 0, None, None, A, None, None) == EINVAL
    assert L.ngram_forward(A, 4, A, 1, None, None, t, A, 0, A, None, A, None, None) == ERANGE
    assert L.ngram_forward(A, 4, A, 1, None, None, t, None, 0, A, None, None, None, None) == EINVAL
    assert L.ngram_forward(A, 4, A, 1, None, None, t, None, 0, A, None, A + 2, None, None) == EALIGN
    assert L.ngram_forward(A, 4, A, 1, None, None, t, A + 2, 10, A, None, A, None, None) == EALIGN
    assert L.ngram_forward(A, 4, A, 0, None, None, t, None, 0, A, None, A, None, None) == EINVAL
    assert L.ngram_forward(A, 4, None, 1, None, None, t, None, 0, A, None, A, None, None) == EINVAL
    assert L.ngram_forward(None, 0, None, 0, None, None, t, None, 0, A, None, None, None, None) == OK


def test_gather_host_and_host_alloc_checks():
    L = ng.lib()
    dev_t = ctypes.byref(_table())
    ws = L.ngram_gather_host_workspace_bytes(4, 64)
    pb = L.ngram_gather_host_pinned_bytes(4)
    assert ws > 0 and pb == 16 + 4 * 64
    assert L.ngram_gather_host_workspace_bytes(-1, 64) == -1 and L.ngram_gather_host_pinned_bytes(-1) == -1
    G = L.ngram_gather_host
    assert G(dev_t, A, 4, A, ws, None, 0, A, None, A, A, 0, None) == ENOTSUP
    host_t = ctypes.byref(_table(loc=1))
    assert G(host_t, A, 4, A, ws, None, 0, A, None, A, A, 2, None) == EINVAL       # unknown mode
    assert G(host_t, None, 4, A, ws, None, 0, A, None, A, A, 0, None) == EINVAL
    assert G(host_t, A, 4, A, ws, None, 0, A, None, A, None, 0, None) == EINVAL    # n_staged_out
    assert G(host_t, A, 4, A, ws, None, 0, A + 8, None, A, A, 0, None) == EALIGN
    assert G(host_t, A, 2**28, A, ws, None, 0, A, None, A, A, 0, None) == ERANGE
    assert G(host_t, A, 4, None, ws, None, 0, A, None, A, A, 0, None) == EINVAL    # no workspace
    assert G(host_t, A, 4, A, ws - 1, None, 0, A, None, A, A, 0, None) == EINVAL   # workspace too small
    assert G(host_t, A, 4, A, ws, None, 0, A, None, A, A, 1, None) == EINVAL       # mode 1 without pinned
    assert G(host_t, A, 4, A, ws, A, pb - 1, A, None, A, A, 1, None) == EINVAL     # pinned too small
    h8 = ctypes.byref(_table(loc=1, dtype=1, scale=A))
    assert G(h8, A, 4, A, ws, None, 0, A, None, A, A, 0, None) == EINVAL           # int8 without scales
    assert G(host_t, None, 0, A, ws, None, 0, None, None, None, None, 0, None) == OK
    p = ctypes.c_void_p()
    assert L.ngram_host_alloc(0, ctypes.byref(p)) == EINVAL
    assert L.ngram_host_alloc(16, None) == EINVAL
    assert L.ngram_host_free(None) == OK


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(ng, "_lib", None)
    monkeypatch.setattr(ng, "LIB_PATH", "/nonexistent/libngram.so")
    with pytest.raises(ng.NgramError):
        ng.lib()


def test_product_package_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "hashed_gram_embedding_ngram_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.replace("oracle/", ""), f"{f} mentions the oracle"


def _pool(data=A, scale=None, slots=A, pool_rows=10_000, cached=0):
    return ng._Pool(data, scale, slots, pool_rows, cached)


def test_pool_workspace_sizes():
    L = ng.lib()
    assert L.ngram_pool_workspace_bytes(-1) == -1
    assert L.ngram_pool_workspace_bytes(0) >= 4 * (1024 + 4)
    n = 8192
    assert L.ngram_pool_workspace_bytes(n) >= 8 * (2 * 16 * n) + 4 * 16 * n


def test_pool_argument_checks():
    L = ng.lib()
    host_t = ctypes.byref(_table(loc=1))
    dev_t = ctypes.byref(_table())
    P = _pool()
    W = ctypes.c_int64(L.ngram_pool_workspace_bytes(4))
    assert L.ngram_pool_gather(dev_t, ctypes.byref(P), A, 4, A, None, A, W, None) == ENOTSUP
    assert L.ngram_pool_gather(host_t, None, A, 4, A, None, A, W, None) == EINVAL
    assert L.ngram_pool_gather(host_t, ctypes.byref(_pool(data=A + 8)), A, 4, A, None, A, W, None) == EALIGN
    assert L.ngram_pool_gather(host_t, ctypes.byref(_pool(pool_rows=63)), A, 4, A, None, A, W, None) == ERANGE
    assert L.ngram_pool_gather(host_t, ctypes.byref(_pool(pool_rows=100, cached=40)), A, 4, A, None, A, W,
                               None) == ERANGE
    assert L.ngram_pool_gather(host_t, ctypes.byref(P), A, 4, A, None, A, 16, None) == EINVAL
    assert L.ngram_pool_gather(host_t, ctypes.byref(P), A, 4, A, None, A + 8, W, None) == EINVAL
    assert L.ngram_pool_gather(host_t, ctypes.byref(P), None, 4, A, None, A, W, None) == EINVAL
    assert L.ngram_pool_gather(host_t, ctypes.byref(P), A, -1, A, None, A, W, None) == EINVAL
    assert L.ngram_pool_gather(host_t, ctypes.byref(P), None, 0, None, None, A, W, None) == OK
    h8 = ctypes.byref(_table(loc=1, dtype=1, scale=A))
    assert L.ngram_pool_gather(h8, ctypes.byref(P), A, 4, A, None, A, W, None) == EINVAL  # no pool scale
    assert L.ngram_pool_cache_rows(host_t, ctypes.byref(P), A, 10_001, None) == ERANGE
    assert L.ngram_pool_cache_rows(host_t, ctypes.byref(P), None, 5, None) == EINVAL
    assert L.ngram_pool_cache_rows(dev_t, ctypes.byref(P), A, 5, None) == ENOTSUP
    assert L.ngram_pool_reset(host_t, None, None) == EINVAL


def test_count_and_select_argument_checks():
    L = ng.lib()
    assert L.ngram_count_rows(A, -1, 100, A, 0, None) == EINVAL
    assert L.ngram_count_rows(A, 4, 0, A, 0, None) == ERANGE
    assert L.ngram_count_rows(A, 4, 100, None, 0, None) == EINVAL
    W = L.ngram_pool_workspace_bytes(0)
    sel = ctypes.c_int64(-1)
    assert L.ngram_select_hot_rows(A, 0, 10, A, ctypes.byref(sel), A, W, None) == ERANGE
    assert L.ngram_select_hot_rows(A, 100, -1, A, ctypes.byref(sel), A, W, None) == ERANGE
    assert L.ngram_select_hot_rows(A, 100, 10, A, None, A, W, None) == EINVAL
    assert L.ngram_select_hot_rows(A, 100, 10, A, ctypes.byref(sel), A, 64, None) == EINVAL
    assert L.ngram_select_hot_rows(A, 100, 0, None, ctypes.byref(sel), A, W, None) == OK and sel.value == 0


def test_grad_argument_checks():
    L = ng.lib()
    W = L.ngram_grad_workspace_bytes(4, 64)
    assert W > 0 and L.ngram_grad_workspace_bytes(-1, 64) == -1 and L.ngram_grad_workspace_bytes(4, 0) == -1
    AW = 0x100000                                          # 256-byte aligned
    assert L.ngram_grad_table(A, -1, 64, 100, A, A, A, A, A, AW, W, None) == EINVAL
    assert L.ngram_grad_table(A, 2**20 + 1, 64, 100, A, A, A, A, A, AW, W, None) == ERANGE
    assert L.ngram_grad_table(A, 4, 12, 100, A, A, A, A, A, AW, W, None) == EINVAL
    assert L.ngram_grad_table(A, 4, 64, 0, A, A, A, A, A, AW, W, None) == ERANGE
    assert L.ngram_grad_table(A, 4, 64, 100, A, A, A, A, A, AW + 16, W, None) == EINVAL
    assert L.ngram_grad_table(A, 4, 64, 100, A, A, A, A, A, AW, W - 1, None) == EINVAL
    assert L.ngram_grad_table(A, 4, 64, 100, None, A, A, A, A, AW, W, None) == EINVAL
    assert L.ngram_grad_table(A, 4, 64, 100, A, A + 2, A, A, A, AW, W, None) == EINVAL
    assert L.ngram_grad_e1(A, A, 4, 64, 0, A, A, A, A, AW, W, None) == ERANGE
    assert L.ngram_grad_e1(A, A, 4, 64, 2**21, A, A, A, A, AW, W, None) == ERANGE
    assert L.ngram_grad_e1(A, A, 4, 64, 100, A, A, A, None, AW, W, None) == EINVAL
    assert L.ngram_grad_gate(A, A, A, 4, 64, None, AW, W, None) == EINVAL
    assert L.ngram_grad_gate(A, A, A + 4, 4, 64, A, AW, W, None) == EINVAL


def test_gated_checks():
    L = ng.lib()

    def call(t=None, n=4, e1=A, W=A, gamma=A, u=A, v=A, b=0.0, eps=1e-6, res=None, out=A, stats=None, V=10):
        t = t or _table(d=64)
        return L.ngram_forward_gated(A, n, A, 1, None, None, ctypes.byref(t), e1, V, W, gamma, u, v, b, eps,
                                     res, out, None, stats, None)

    assert call(e1=None) == EINVAL
    assert call(gamma=None) == EINVAL and call(u=None) == EINVAL and call(v=None) == EINVAL
    assert call(W=None) == EINVAL
    assert call(eps=-1.0) == EINVAL and call(eps=float("nan")) == EINVAL and call(eps=float("inf")) == EINVAL
    assert call(b=float("inf")) == EINVAL and call(b=float("nan")) == EINVAL
    assert call(V=0) == ERANGE
    assert call(t=_table(d=8200)) == ERANGE and "gated" in _err()
    assert call(gamma=A + 4) == EALIGN and call(u=A + 8) == EALIGN and call(stats=A + 4) == EALIGN
    assert call(out=None) == EINVAL
    assert call(n=0, out=None) == OK                                  # empty: no launch
