"""Python binding of libngram.so, the hashed n-gram embedding gather-sum for
MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``csrc/ngram.hip`` behind the C ABI of ``include/ngram.h``; the functions here
check tensor dtypes and devices, pass raw pointers and the current HIP stream,
and raise on a non-zero status.  torch supplies device memory and streams.
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libngram.so")

K = 16
PAD_ID = (1 << 21) - 1
TABLE_BF16 = 0
TABLE_INT8_ROWSCALE = 1
TABLE_MXFP4 = 2
IN_DEVICE = 0
IN_HOST = 1


class NgramError(RuntimeError):
    pass


class _Table(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("row_scale", ctypes.c_void_p), ("R", ctypes.c_int64),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("location", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class _Launch(ctypes.Structure):
    _fields_ = [("tokens_per_workgroup", ctypes.c_int32), ("host_workgroups", ctypes.c_int32)]


class _Pool(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("row_scale", ctypes.c_void_p), ("slot_of_row", ctypes.c_void_p),
                ("pool_rows", ctypes.c_int64), ("cached", ctypes.c_int64)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIGNATURES = {
    "ngram_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ngram_last_error": (ctypes.c_char_p, []),
    "ngram_version": (ctypes.c_int, []),
    "ngram_default_seeds": (None, [_P]),
    "ngram_hash": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _P, _I64, _P, _P]),
    "ngram_embed_bag": (ctypes.c_int, [ctypes.POINTER(_Table), _P, _I64, _P, _P]),
    "ngram_embed_bag_ex": (ctypes.c_int, [ctypes.POINTER(_Table), _P, _I64, _P, ctypes.POINTER(_Launch), _P]),
    "ngram_gate_add": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _I64, _P, _P, _P, _P]),
    "ngram_forward": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _P, ctypes.POINTER(_Table), _P, _I64,
                                     _P, _P, _P, _P, _P]),
    "ngram_forward_ex": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _P, ctypes.POINTER(_Table), _P, _I64,
                                        _P, _P, _P, _P, ctypes.POINTER(_Launch), _P]),
    "ngram_forward_gated": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _P, ctypes.POINTER(_Table), _P, _I64,
                                           _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P, _P, _P, _P]),
    "ngram_forward_gated_ex": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _P, ctypes.POINTER(_Table), _P, _I64,
                                              _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P, _P, _P,
                                              ctypes.POINTER(_Launch), _P]),
    "ngram_norm_gate_add": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _I64, _P, _P, _P, _P, ctypes.c_float,
                                           ctypes.c_float, _P, _P, _P, _P]),
    "ngram_project": (ctypes.c_int, [_P, _I64, _I32, _P, _I32, _P, _P]),
    "ngram_embed_bag_bf16": (ctypes.c_int, [ctypes.POINTER(_Table), _P, _I64, _P, _P]),
    "ngram_host_alloc": (ctypes.c_int, [_I64, ctypes.POINTER(ctypes.c_void_p)]),
    "ngram_host_free": (ctypes.c_int, [_P]),
    "ngram_gather_host_workspace_bytes": (ctypes.c_int64, [_I64, _I32]),
    "ngram_gather_host_pinned_bytes": (ctypes.c_int64, [_I64]),
    "ngram_gather_host": (ctypes.c_int, [ctypes.POINTER(_Table), _P, _I64, _P, _I64, _P, _I64, _P, _P, _P, _P,
                                         _I32, _P]),
    "ngram_pool_workspace_bytes": (ctypes.c_int64, [_I64]),
    "ngram_pool_reset": (ctypes.c_int, [ctypes.POINTER(_Table), ctypes.POINTER(_Pool), _P]),
    "ngram_pool_cache_rows": (ctypes.c_int, [ctypes.POINTER(_Table), ctypes.POINTER(_Pool), _P, _I64, _P]),
    "ngram_pool_gather": (ctypes.c_int, [ctypes.POINTER(_Table), ctypes.POINTER(_Pool), _P, _I64, _P, _P, _P,
                                         _I64, _P]),
    "ngram_count_rows": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _P]),
    "ngram_grad_workspace_bytes": (ctypes.c_int64, [_I64, _I32]),
    "ngram_grad_table": (ctypes.c_int, [_P, _I64, _I32, _I64, _P, _P, _P, _P, _P, _P, _I64, _P]),
    "ngram_grad_e1": (ctypes.c_int, [_P, _P, _I64, _I32, _I64, _P, _P, _P, _P, _P, _I64, _P]),
    "ngram_grad_gate": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _P, _P, _I64, _P]),
    "ngram_grad_gate_noalloc_max_elements": (ctypes.c_int64, []),
    "ngram_grad_gate_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _P, _P]),
    "ngram_select_hot_rows": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.POINTER(ctypes.c_int64), _P, _I64, _P]),
}

_lib = None


def lib():
    """The loaded libngram.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NgramError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                             "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        L = lib()
        raise NgramError(f"{what}: {L.ngram_status_string(rc).decode()} "
                         f"({L.ngram_last_error().decode()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtypes, name, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise NgramError(f"{name} is required")
    if not t.is_cuda:
        raise NgramError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise NgramError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise NgramError(f"{name} must be contiguous")


def _need(t, count, name):
    """Refuse a buffer smaller than the call reads or writes."""
    if t is not None and t.numel() < count:
        raise NgramError(f"{name} holds {t.numel()} elements, the call needs {count}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32T = (torch.int32,)
_F32 = (torch.float32,)


def default_seeds():
    s = (ctypes.c_uint64 * K)()
    lib().ngram_default_seeds(s)
    return [int(x) for x in s]


def _launch_arg(launch):
    """``launch``: None, or (tokens_per_workgroup, host_workgroups), 0 for the
    library's choice of either."""
    if launch is None:
        return None
    tpw, hw = launch
    return ctypes.byref(_Launch(int(tpw), int(hw)))


def _seeds_arg(seeds):
    if seeds is None:
        return None
    if len(seeds) != K:
        raise NgramError("seeds must hold 16 values")
    return (ctypes.c_uint64 * K)(*[int(s) & 0xFFFFFFFFFFFFFFFF for s in seeds])


class Table:
    """An n-gram table: ``data`` [R][d] bf16 (or int8 with ``row_scale`` [R]
    fp32) in device memory, or a ``HostBuffer`` in pinned host memory."""

    def __init__(self, data, R: int, d: int, dtype: int = TABLE_BF16, row_scale=None):
        self.data = data
        self.row_scale = row_scale
        self.R, self.d, self.dtype = int(R), int(d), int(dtype)
        nbytes = self.R * row_bytes(self.d, self.dtype)
        if isinstance(data, HostBuffer):
            self.location = IN_HOST
            ptr = data.ptr
            if data.nbytes < nbytes:
                raise NgramError("host table buffer is smaller than R rows")
        else:
            dts = {TABLE_BF16: _BF16, TABLE_INT8_ROWSCALE: (torch.int8,), TABLE_MXFP4: (torch.uint8, torch.int8)}
            _dev(data, dts.get(self.dtype, _BF16), "table")
            if data.numel() * data.element_size() < nbytes:
                raise NgramError(f"table holds {data.numel() * data.element_size()} bytes, R rows need {nbytes}")
            self.location = IN_DEVICE
            ptr = data.data_ptr()
        if dtype == TABLE_INT8_ROWSCALE:
            _dev(row_scale, _F32, "row_scale")
            _need(row_scale, self.R, "row_scale")
        self._c = _Table(ptr, None if row_scale is None else row_scale.data_ptr(), self.R, self.d,
                         self.dtype, self.location, 0)

    @property
    def c(self):
        return ctypes.byref(self._c)


class HostBuffer:
    """Pinned, device-mapped host memory from ngram_host_alloc."""

    def __init__(self, nbytes: int):
        p = ctypes.c_void_p()
        _check(lib().ngram_host_alloc(int(nbytes), ctypes.byref(p)), "ngram_host_alloc")
        self.ptr = p.value
        self.nbytes = int(nbytes)

    def numpy(self, dtype, shape):
        import numpy as np
        buf = (ctypes.c_char * self.nbytes).from_address(self.ptr)
        return np.frombuffer(buf, dtype=dtype, count=int(np.prod(shape))).reshape(shape)

    def free(self):
        if self.ptr:
            _check(lib().ngram_host_free(ctypes.c_void_p(self.ptr)), "ngram_host_free")
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def row_bytes(d: int, dtype: int) -> int:
    """Bytes of one table row: 2d (bf16), d (int8) or d/2 + d/32 (MXFP4)."""
    if dtype == TABLE_BF16:
        return 2 * d
    if dtype == TABLE_MXFP4:
        return d // 2 + d // 32
    return d


def _vocab(e1, d):
    """Rows of the [V][d] e1 table (any shape with V*d elements)."""
    if e1 is None:
        return 0
    if e1.numel() % d:
        raise NgramError(f"e1 has {e1.numel()} elements, not a multiple of d={d}")
    return e1.numel() // d


def ngram_hash(tokens, seq_offsets, R, rows_out=None, history=None, seeds=None, stream=None):
    _dev(tokens, _I32T, "tokens")
    _dev(seq_offsets, _I32T, "seq_offsets")
    _dev(history, _I32T, "history", allow_none=True)
    n = tokens.numel()
    if rows_out is None:
        rows_out = torch.empty((n, K), dtype=torch.int32, device=tokens.device)
    _dev(rows_out, _I32T, "rows_out")
    _need(rows_out, n * K, "rows_out")
    _need(history, 2 * (seq_offsets.numel() - 1), "history")
    _check(lib().ngram_hash(_ptr(tokens), n, _ptr(seq_offsets), seq_offsets.numel() - 1,
                            _ptr(history), _seeds_arg(seeds), int(R), _ptr(rows_out), _stream(stream)),
           "ngram_hash")
    return rows_out


def ngram_embed_bag(table: Table, rows, eN_out=None, launch=None, stream=None):
    _dev(rows, _I32T, "rows")
    n = rows.shape[0] if rows.dim() == 2 else rows.numel() // K
    if eN_out is None:
        eN_out = torch.empty((n, table.d), dtype=torch.float32, device=rows.device)
    _dev(eN_out, _F32, "eN_out")
    _need(rows, n * K, "rows")
    _need(eN_out, n * table.d, "eN_out")
    if launch is None:
        rc = lib().ngram_embed_bag(table.c, _ptr(rows), n, _ptr(eN_out), _stream(stream))
    else:
        rc = lib().ngram_embed_bag_ex(table.c, _ptr(rows), n, _ptr(eN_out), _launch_arg(launch), _stream(stream))
    _check(rc, "ngram_embed_bag")
    return eN_out


def ngram_gate_add(eN, tokens, W_g, out, e1=None, residual=None, stream=None):
    _dev(eN, _F32, "eN")
    _dev(tokens, _I32T, "tokens")
    _dev(W_g, _F32, "W_g")
    _dev(out, _BF16, "out")
    _dev(e1, _BF16, "e1", allow_none=True)
    _dev(residual, _BF16, "residual", allow_none=True)
    n, d = eN.shape
    V = _vocab(e1, d)
    _need(tokens, n, "tokens")
    _need(W_g, d, "W_g")
    _need(out, n * d, "out")
    _need(residual, n * d, "residual")
    _check(lib().ngram_gate_add(_ptr(eN), _ptr(tokens), n, d, _ptr(e1), V, _ptr(W_g),
                                _ptr(residual), _ptr(out), _stream(stream)), "ngram_gate_add")
    return out


def ngram_forward(tokens, seq_offsets, table: Table, W_g, out, e1=None, residual=None,
                  history=None, seeds=None, rows_out=None, launch=None, stream=None):
    _dev(tokens, _I32T, "tokens")
    _dev(seq_offsets, _I32T, "seq_offsets")
    _dev(history, _I32T, "history", allow_none=True)
    _dev(W_g, _F32, "W_g")
    _dev(out, _BF16, "out")
    _dev(e1, _BF16, "e1", allow_none=True)
    _dev(residual, _BF16, "residual", allow_none=True)
    _dev(rows_out, _I32T, "rows_out", allow_none=True)
    V = _vocab(e1, table.d)
    n, d = tokens.numel(), table.d
    _need(W_g, d, "W_g")
    _need(out, n * d, "out")
    _need(residual, n * d, "residual")
    _need(rows_out, n * K, "rows_out")
    _need(history, 2 * (seq_offsets.numel() - 1), "history")
    args = (_ptr(tokens), tokens.numel(), _ptr(seq_offsets), seq_offsets.numel() - 1, _ptr(history),
            _seeds_arg(seeds), table.c, _ptr(e1), V, _ptr(W_g), _ptr(residual), _ptr(out), _ptr(rows_out))
    if launch is None:
        rc = lib().ngram_forward(*args, _stream(stream))
    else:
        rc = lib().ngram_forward_ex(*args, _launch_arg(launch), _stream(stream))
    _check(rc, "ngram_forward")
    return out


def ngram_forward_gated(tokens, seq_offsets, table: Table, W_g, gamma, u, v, b, eps, out, e1,
                        residual=None, history=None, seeds=None, rows_out=None, stats_out=None, launch=None,
                        stream=None):
    """Normalised, input-gated forward (see ngram_forward_gated in ngram.h);
    ``stats_out`` [n][2] float64 receives (r, logit) per token."""
    _dev(tokens, _I32T, "tokens")
    _dev(seq_offsets, _I32T, "seq_offsets")
    _dev(history, _I32T, "history", allow_none=True)
    for t, name in ((W_g, "W_g"), (gamma, "gamma"), (u, "u"), (v, "v")):
        _dev(t, _F32, name)
    _dev(out, _BF16, "out")
    _dev(e1, _BF16, "e1")
    _dev(residual, _BF16, "residual", allow_none=True)
    _dev(rows_out, _I32T, "rows_out", allow_none=True)
    _dev(stats_out, (torch.float64,), "stats_out", allow_none=True)
    V = _vocab(e1, table.d)
    n, d = tokens.numel(), table.d
    for t, name in ((W_g, "W_g"), (gamma, "gamma"), (u, "u"), (v, "v")):
        _need(t, d, name)
    _need(out, n * d, "out")
    _need(residual, n * d, "residual")
    _need(rows_out, n * K, "rows_out")
    _need(stats_out, 2 * n, "stats_out")
    _need(history, 2 * (seq_offsets.numel() - 1), "history")
    args = (_ptr(tokens), n, _ptr(seq_offsets), seq_offsets.numel() - 1, _ptr(history), _seeds_arg(seeds),
            table.c, _ptr(e1), V, _ptr(W_g), _ptr(gamma), _ptr(u), _ptr(v), float(b), float(eps), _ptr(residual),
            _ptr(out), _ptr(rows_out), _ptr(stats_out))
    if launch is None:
        rc = lib().ngram_forward_gated(*args, _stream(stream))
    else:
        rc = lib().ngram_forward_gated_ex(*args, _launch_arg(launch), _stream(stream))
    _check(rc, "ngram_forward_gated")
    return out


def ngram_norm_gate_add(eN, tokens, e1, W_g, gamma, u, v, b, eps, out, residual=None, stats_out=None,
                        stream=None):
    """The normalised, input-gated epilogue on given fp32 sums eN [n][d]
    (see ngram_norm_gate_add in ngram.h)."""
    _dev(eN, _F32, "eN")
    _dev(tokens, _I32T, "tokens")
    for t, name in ((W_g, "W_g"), (gamma, "gamma"), (u, "u"), (v, "v")):
        _dev(t, _F32, name)
    _dev(out, _BF16, "out")
    _dev(e1, _BF16, "e1")
    _dev(residual, _BF16, "residual", allow_none=True)
    _dev(stats_out, (torch.float64,), "stats_out", allow_none=True)
    n, d = eN.shape
    V = _vocab(e1, d)
    _need(tokens, n, "tokens")
    for t, name in ((W_g, "W_g"), (gamma, "gamma"), (u, "u"), (v, "v")):
        _need(t, d, name)
    _need(out, n * d, "out")
    _need(residual, n * d, "residual")
    _need(stats_out, 2 * n, "stats_out")
    _check(lib().ngram_norm_gate_add(_ptr(eN), _ptr(tokens), n, d, _ptr(e1), V, _ptr(W_g), _ptr(gamma), _ptr(u),
                                     _ptr(v), float(b), float(eps), _ptr(residual), _ptr(out), _ptr(stats_out),
                                     _stream(stream)), "ngram_norm_gate_add")
    return out


def ngram_embed_bag_bf16(table: Table, rows, out=None, stream=None):
    """The sums of ngram_embed_bag rounded to bf16: out [n][d] (bf16 bits)."""
    _dev(rows, _I32T, "rows")
    n = rows.shape[0]
    if out is None:
        out = torch.empty((n, table.d), dtype=torch.int16, device=rows.device)
    _dev(out, _BF16, "out")
    _need(out, n * table.d, "out")
    _check(lib().ngram_embed_bag_bf16(table.c, _ptr(rows), n, _ptr(out), _stream(stream)), "ngram_embed_bag_bf16")
    return out


def ngram_project(x, P, y=None, stream=None):
    """y [n][d_out] fp32 = P x for x [n][d_in] and P [d_out][d_in], both bf16
    bits (int16 tensors); see ngram_project in ngram.h."""
    _dev(x, _BF16, "x")
    _dev(P, _BF16, "P")
    n, d_in = x.shape
    d_out = P.shape[0]
    if P.dim() != 2 or P.shape[1] != d_in:
        raise NgramError(f"P must be [d_out][{d_in}], got {tuple(P.shape)}")
    if y is None:
        y = torch.empty((n, d_out), dtype=torch.float32, device=x.device)
    _dev(y, _F32, "y")
    _need(y, n * d_out, "y")
    _check(lib().ngram_project(_ptr(x), n, d_in, _ptr(P), d_out, _ptr(y), _stream(stream)), "ngram_project")
    return y


GATHER_ZERO_COPY = 0
GATHER_ASYNC_COPY = 1


def gather_host_workspace(n: int, d: int, device="cuda:0"):
    nbytes = int(lib().ngram_gather_host_workspace_bytes(int(n), int(d)))
    return torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)


def gather_host_pinned(n: int) -> "HostBuffer":
    """Pinned host memory for ngram_gather_host's async-copy mode."""
    return HostBuffer(max(16, int(lib().ngram_gather_host_pinned_bytes(int(n)))))


def ngram_gather_host(table: Table, rows, stage_out, remap_out, stage_scale_out=None, n_staged_out=None,
                      mode=GATHER_ZERO_COPY, workspace=None, pinned=None, stream=None):
    """Stage the batch's distinct rows of a pinned-host table in device
    memory.  Returns (stage_out, remap_out, n_staged_out [1] int64)."""
    _dev(rows, _I32T, "rows")
    _dev(remap_out, _I32T, "remap_out")
    _dev(stage_scale_out, _F32, "stage_scale_out", allow_none=True)
    if not stage_out.is_cuda or not stage_out.is_contiguous():
        raise NgramError("stage_out must be a contiguous device tensor")
    n = rows.shape[0] if rows.dim() == 2 else rows.numel() // K
    _need(rows, n * K, "rows")
    _need(remap_out, n * K, "remap_out")
    rb = row_bytes(table.d, table.dtype)
    if stage_out.numel() * stage_out.element_size() < n * K * rb:
        raise NgramError("stage_out is smaller than n * 16 rows")
    if table.dtype == TABLE_INT8_ROWSCALE:
        _need(stage_scale_out, n * K, "stage_scale_out")
    if n_staged_out is None:
        n_staged_out = torch.empty(1, dtype=torch.int64, device=rows.device)
    _dev(n_staged_out, (torch.int64,), "n_staged_out")
    if workspace is None:
        workspace = gather_host_workspace(n, table.d, rows.device)
    own_pinned = None
    if mode == GATHER_ASYNC_COPY and pinned is None:
        own_pinned = pinned = gather_host_pinned(n)
    p_ptr = None if pinned is None else ctypes.c_void_p(pinned.ptr)
    p_bytes = 0 if pinned is None else pinned.nbytes
    _check(lib().ngram_gather_host(table.c, _ptr(rows), n, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   p_ptr, p_bytes, _ptr(stage_out), _ptr(stage_scale_out), _ptr(remap_out),
                                   _ptr(n_staged_out), int(mode), _stream(stream)), "ngram_gather_host")
    if own_pinned is not None:
        # the copies read only the table, but the row list they were built
        # from sits in this buffer: let the stream pass them before freeing it
        (stream or torch.cuda.current_stream()).synchronize()
        own_pinned.free()
    return stage_out, remap_out, n_staged_out


class RowPool:
    """Device-memory row pool in front of a pinned-host table: ``pool_rows``
    rows of the table's dtype (a hot-row cache in the first ``cached`` rows,
    staged misses after them), per-row scales for int8, and the [R] map
    ``slot_of_row``.  The buffers are torch device tensors."""

    def __init__(self, table: Table, pool_rows: int, device="cuda:0", stream=None):
        if table.location != IN_HOST:
            raise NgramError("a row pool fronts a table in host memory")
        self.table = table
        self.pool_rows = int(pool_rows)
        if table.dtype == TABLE_MXFP4:
            self.data = torch.empty(self.pool_rows * row_bytes(table.d, table.dtype), dtype=torch.uint8,
                                    device=device)
        else:
            dt = torch.int16 if table.dtype == TABLE_BF16 else torch.int8
            self.data = torch.empty(self.pool_rows * table.d, dtype=dt, device=device)
        self.row_scale = (torch.empty(self.pool_rows, dtype=torch.float32, device=device)
                          if table.dtype == TABLE_INT8_ROWSCALE else None)
        self.slot_of_row = torch.empty(table.R, dtype=torch.int32, device=device)
        self._c = _Pool(self.data.data_ptr(), None if self.row_scale is None else self.row_scale.data_ptr(),
                        self.slot_of_row.data_ptr(), self.pool_rows, 0)
        _check(lib().ngram_pool_reset(table.c, ctypes.byref(self._c), _stream(stream)), "ngram_pool_reset")

    @property
    def cached(self):
        return int(self._c.cached)

    def device_table(self) -> Table:
        """The pool as a device table of ``pool_rows`` rows."""
        return Table(self.data, self.pool_rows, self.table.d, self.table.dtype, row_scale=self.row_scale)


def ngram_pool_workspace_bytes(n: int) -> int:
    return int(lib().ngram_pool_workspace_bytes(int(n)))


def pool_workspace(n: int, device="cuda:0"):
    nbytes = ngram_pool_workspace_bytes(n)
    return torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)


def ngram_pool_reset(pool: RowPool, stream=None):
    _check(lib().ngram_pool_reset(pool.table.c, ctypes.byref(pool._c), _stream(stream)), "ngram_pool_reset")


def ngram_pool_cache_rows(pool: RowPool, hot_rows, C=None, stream=None):
    _dev(hot_rows, _I32T, "hot_rows")
    C = hot_rows.numel() if C is None else int(C)
    _need(hot_rows, C, "hot_rows")
    _check(lib().ngram_pool_cache_rows(pool.table.c, ctypes.byref(pool._c), _ptr(hot_rows), C, _stream(stream)),
           "ngram_pool_cache_rows")


def ngram_pool_gather(pool: RowPool, rows, pool_rows_out=None, fetched_out=None, workspace=None, stream=None):
    _dev(rows, _I32T, "rows")
    n = rows.shape[0] if rows.dim() == 2 else rows.numel() // K
    _need(rows, n * K, "rows")
    if pool_rows_out is None:
        pool_rows_out = torch.empty((n, K), dtype=torch.int32, device=rows.device)
    _dev(pool_rows_out, _I32T, "pool_rows_out")
    _need(pool_rows_out, n * K, "pool_rows_out")
    if fetched_out is not None:
        _dev(fetched_out, (torch.int64,), "fetched_out")
    if workspace is None:
        workspace = pool_workspace(n, rows.device)
    _check(lib().ngram_pool_gather(pool.table.c, ctypes.byref(pool._c), _ptr(rows), n, _ptr(pool_rows_out),
                                   _ptr(fetched_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "ngram_pool_gather")
    return pool_rows_out


def ngram_count_rows(rows, R, counts=None, accumulate=False, stream=None):
    _dev(rows, _I32T, "rows")
    n = rows.shape[0] if rows.dim() == 2 else rows.numel() // K
    if counts is None:
        counts = torch.empty(int(R), dtype=torch.int32, device=rows.device)
        accumulate = False
    _dev(counts, _I32T, "counts")
    _need(counts, int(R), "counts")
    _check(lib().ngram_count_rows(_ptr(rows), n, int(R), _ptr(counts), 1 if accumulate else 0, _stream(stream)),
           "ngram_count_rows")
    return counts


def ngram_select_hot_rows(counts, C, hot_rows_out=None, workspace=None, stream=None):
    """Returns (hot_rows_out, selected); synchronizes the stream."""
    _dev(counts, _I32T, "counts")
    if hot_rows_out is None:
        hot_rows_out = torch.empty(max(int(C), 1), dtype=torch.int32, device=counts.device)
    _dev(hot_rows_out, _I32T, "hot_rows_out")
    _need(hot_rows_out, int(C), "hot_rows_out")
    if workspace is None:
        workspace = pool_workspace(0, counts.device)
    sel = ctypes.c_int64(0)
    _check(lib().ngram_select_hot_rows(_ptr(counts), counts.numel(), int(C), _ptr(hot_rows_out), ctypes.byref(sel),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)), "ngram_select_hot_rows")
    return hot_rows_out, int(sel.value)


def grad_workspace(n: int, d: int, device="cuda:0"):
    nbytes = int(lib().ngram_grad_workspace_bytes(int(n), int(d)))
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws_args(workspace):
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def ngram_grad_table(rows, W_g, dout, R, grad_rows_out=None, grad_out=None, n_unique_out=None,
                     workspace=None, stream=None):
    """Sparse table gradient: (grad_rows_out [16n], grad_out [16n][d], n_unique_out [1] int64);
    the first n_unique_out rows are valid."""
    _dev(rows, _I32T, "rows")
    _dev(W_g, _F32, "W_g")
    _dev(dout, _BF16, "dout")
    n = rows.shape[0] if rows.dim() == 2 else rows.numel() // K
    d = dout.numel() // max(n, 1) if n else W_g.numel()
    _need(rows, n * K, "rows")
    _need(W_g, d, "W_g")
    dev = rows.device
    grad_rows_out = torch.empty(n * K, dtype=torch.int32, device=dev) if grad_rows_out is None else grad_rows_out
    grad_out = torch.empty((n * K, d), dtype=torch.float32, device=dev) if grad_out is None else grad_out
    n_unique_out = torch.empty(1, dtype=torch.int64, device=dev) if n_unique_out is None else n_unique_out
    _dev(grad_rows_out, _I32T, "grad_rows_out")
    _dev(grad_out, _F32, "grad_out")
    _dev(n_unique_out, (torch.int64,), "n_unique_out")
    _need(grad_rows_out, n * K, "grad_rows_out")
    _need(grad_out, n * K * d, "grad_out")
    workspace = grad_workspace(n, d, dev) if workspace is None else workspace
    _check(lib().ngram_grad_table(_ptr(rows), n, d, int(R), _ptr(W_g), _ptr(dout), _ptr(grad_rows_out),
                                  _ptr(grad_out), _ptr(n_unique_out), *_ws_args(workspace), _stream(stream)),
           "ngram_grad_table")
    return grad_rows_out, grad_out, n_unique_out


def ngram_grad_e1(tokens, rows, dout, V, grad_tokens_out=None, grad_out=None, n_unique_out=None,
                  workspace=None, stream=None):
    _dev(tokens, _I32T, "tokens")
    _dev(rows, _I32T, "rows")
    _dev(dout, _BF16, "dout")
    n = tokens.numel()
    d = dout.numel() // max(n, 1)
    _need(rows, n * K, "rows")
    dev = tokens.device
    grad_tokens_out = torch.empty(n, dtype=torch.int32, device=dev) if grad_tokens_out is None else grad_tokens_out
    grad_out = torch.empty((n, d), dtype=torch.float32, device=dev) if grad_out is None else grad_out
    n_unique_out = torch.empty(1, dtype=torch.int64, device=dev) if n_unique_out is None else n_unique_out
    _need(grad_tokens_out, n, "grad_tokens_out")
    _need(grad_out, n * d, "grad_out")
    workspace = grad_workspace(n, d, dev) if workspace is None else workspace
    _check(lib().ngram_grad_e1(_ptr(tokens), _ptr(rows), n, d, int(V), _ptr(dout), _ptr(grad_tokens_out),
                               _ptr(grad_out), _ptr(n_unique_out), *_ws_args(workspace), _stream(stream)),
           "ngram_grad_e1")
    return grad_tokens_out, grad_out, n_unique_out


def ngram_grad_gate(rows, dout, eN, grad_Wg_out=None, workspace=None, stream=None):
    _dev(rows, _I32T, "rows")
    _dev(dout, _BF16, "dout")
    _dev(eN, _F32, "eN")
    n, d = eN.shape
    _need(rows, n * K, "rows")
    _need(dout, n * d, "dout")
    grad_Wg_out = torch.empty(d, dtype=torch.float32, device=eN.device) if grad_Wg_out is None else grad_Wg_out
    _need(grad_Wg_out, d, "grad_Wg_out")
    workspace = grad_workspace(n, d, eN.device) if workspace is None else workspace
    _check(lib().ngram_grad_gate(_ptr(rows), _ptr(dout), _ptr(eN), n, d, _ptr(grad_Wg_out), *_ws_args(workspace),
                                 _stream(stream)), "ngram_grad_gate")
    return grad_Wg_out


def ngram_grad_gate_noalloc(rows, dout, eN, grad_Wg_out=None, stream=None):
    """The gate gradient without a workspace (the library's static scratch;
    calls that overlap on one GPU race)."""
    _dev(rows, _I32T, "rows")
    _dev(dout, _BF16, "dout")
    _dev(eN, _F32, "eN")
    n, d = eN.shape
    _need(rows, n * K, "rows")
    _need(dout, n * d, "dout")
    grad_Wg_out = torch.empty(d, dtype=torch.float32, device=eN.device) if grad_Wg_out is None else grad_Wg_out
    _dev(grad_Wg_out, _F32, "grad_Wg_out")
    _need(grad_Wg_out, d, "grad_Wg_out")
    _check(lib().ngram_grad_gate_noalloc(_ptr(rows), _ptr(dout), _ptr(eN), n, d, _ptr(grad_Wg_out), _stream(stream)),
           "ngram_grad_gate_noalloc")
    return grad_Wg_out
