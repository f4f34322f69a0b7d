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
IN_DEVICE = 0
IN_HOST = 1


class NgramError(RuntimeError):
    pass


class _Table(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("row_scale", ctypes.c_void_p), ("R", ctypes.c_int64),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("location", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


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
    "ngram_gate_add": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _I64, _P, _P, _P, _P]),
    "ngram_forward": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _P, ctypes.POINTER(_Table), _P, _I64,
                                     _P, _P, _P, _P, _P]),
    "ngram_host_alloc": (ctypes.c_int, [_I64, ctypes.POINTER(ctypes.c_void_p)]),
    "ngram_host_free": (ctypes.c_int, [_P]),
    "ngram_gather_host": (ctypes.c_int, [ctypes.POINTER(_Table), _P, _I64, _P, _P, _P, _P]),
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
        if isinstance(data, HostBuffer):
            self.location = IN_HOST
            ptr = data.ptr
        else:
            _dev(data, _BF16 if dtype == TABLE_BF16 else (torch.int8,), "table")
            _need(data, self.R * self.d, "table")
            self.location = IN_DEVICE
            ptr = data.data_ptr()
        if isinstance(data, HostBuffer) and data.nbytes < self.R * self.d * (2 if dtype == TABLE_BF16 else 1):
            raise NgramError("host table buffer is smaller than R * d elements")
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


def ngram_embed_bag(table: Table, rows, eN_out=None, stream=None):
    _dev(rows, _I32T, "rows")
    n = rows.shape[0] if rows.dim() == 2 else rows.numel() // K
    if eN_out is None:
        eN_out = torch.empty((n, table.d), dtype=torch.float32, device=rows.device)
    _dev(eN_out, _F32, "eN_out")
    _need(rows, n * K, "rows")
    _need(eN_out, n * table.d, "eN_out")
    _check(lib().ngram_embed_bag(table.c, _ptr(rows), n, _ptr(eN_out), _stream(stream)),
           "ngram_embed_bag")
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
                  history=None, seeds=None, rows_out=None, stream=None):
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
    _check(lib().ngram_forward(_ptr(tokens), tokens.numel(), _ptr(seq_offsets), seq_offsets.numel() - 1,
                               _ptr(history), _seeds_arg(seeds), table.c, _ptr(e1), V, _ptr(W_g),
                               _ptr(residual), _ptr(out), _ptr(rows_out), _stream(stream)),
           "ngram_forward")
    return out


def ngram_gather_host(table: Table, rows, stage_out, remap_out, stage_scale_out=None, stream=None):
    _dev(rows, _I32T, "rows")
    _dev(remap_out, _I32T, "remap_out")
    _dev(stage_scale_out, _F32, "stage_scale_out", allow_none=True)
    if not stage_out.is_cuda or not stage_out.is_contiguous():
        raise NgramError("stage_out must be a contiguous device tensor")
    n = rows.shape[0] if rows.dim() == 2 else rows.numel() // K
    _need(rows, n * K, "rows")
    _need(remap_out, n * K, "remap_out")
    row_bytes = table.d * (2 if table.dtype == TABLE_BF16 else 1)
    if stage_out.numel() * stage_out.element_size() < n * K * row_bytes:
        raise NgramError("stage_out is smaller than n * 16 rows")
    if table.dtype == TABLE_INT8_ROWSCALE:
        _need(stage_scale_out, n * K, "stage_scale_out")
    _check(lib().ngram_gather_host(table.c, _ptr(rows), n, _ptr(stage_out), _ptr(stage_scale_out),
                                   _ptr(remap_out), _stream(stream)), "ngram_gather_host")
    return stage_out, remap_out
