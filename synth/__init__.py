"""Seeded synthetic inputs for the hashed n-gram embedding workloads.

This module is shared by the oracle side and the GPU side of every test and
benchmark, and by nothing else.  It holds no step of the n-gram method: no
context extraction, no hashing, no gather, no sum, no gate and no rounding.
Every value is built from the bits of a counter-based generator by exact
integer operations and exact power-of-two scalings, so that the numpy code
here and the HIP fill kernels in ``synth/fill.hip`` produce identical bits.

Generator: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011).  Element ``e`` of a tensor with tag
``tag`` under seed ``seed`` takes word ``e % 4`` of the block with counter
``(g_lo, g_hi, tag, 0)``, ``g = e // 4``, key ``(seed_lo, seed_hi)``.

Value recipes (``x`` is the element's 32-bit word):

* ``bf16_normal(E)``: ``S = sum of the four 7-bit fields of x - 254`` in
  [-254, 254] (Irwin-Hall of four uniforms, sigma 73.9), value ``S * 2^-E``.
  ``|S| < 256`` makes the value exactly representable in bf16, so the bits
  are those of the exact fp32 product, upper half.  ``E = 12`` gives sigma
  0.018 (stand-in for N(0, 0.02)); ``E = 6`` gives sigma 1.15 (for N(0, 1)).
* ``bf16_wide``: sign bit, exponent field in [100, 131], 7 random mantissa
  bits; magnitudes span 2^-27 .. 2^5, so fp32 sums of such rows round and the
  order of the sum becomes observable.
* ``f32_unit``: ``(x >> 8) * 2^-24``, uniform on [0, 1) (gate vector).
* ``i8_normal``: sum of four 6-bit fields minus 126, in [-126, 126], sigma 37.
* ``f32_scale``: ``(2^23 + (x & 0x7FFFFF)) * 2^-34``, in [2^-11, 2^-10)
  (per-row int8 scale; 37 * 7.3e-4 gives values of about 0.027).
* tokens: Zipf(s) over ranks 1..V, ``P(r) ~ r^-s``, id = r - 1, drawn by the
  inverse CDF on a float64 cumulative sum with a 53-bit uniform built from
  two words of the token's block; ``uniform`` tokens use floor(u * V).
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)

# Tensor tags: the third counter word.  A workload seed plus a tag names
# one tensor.
TAG_TOKENS = 1
TAG_TABLE = 2
TAG_E1 = 3
TAG_WG = 4
TAG_RESIDUAL = 5
TAG_SCALE = 6
TAG_HISTORY = 7
TAG_GAMMA = 8
TAG_GATE_U = 9
TAG_GATE_V = 10

KIND_BF16_NORMAL12 = 0   # sigma 0.018
KIND_BF16_NORMAL6 = 1    # sigma 1.15
KIND_BF16_WIDE = 2
KIND_F32_UNIT = 3
KIND_I8_NORMAL = 4
KIND_F32_SCALE = 5
KIND_MXFP4 = 6          # 4-bit rows: random codes, scales 2^-8 .. 2^-5
KIND_MXFP4_WIDE = 7     # 4-bit rows: random codes, scales 2^-27 .. 2^4


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of uint32 counters (vectorised)."""
    c = [np.asarray(v, dtype=np.uint64) & _MASK32 for v in (c0, c1, c2, c3)]
    k0 = np.uint64(k0) & _MASK32
    k1 = np.uint64(k1) & _MASK32
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * c[0]
        p1 = m1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return [v.astype(np.uint32) for v in c]


def words(seed: int, tag: int, elem) -> np.ndarray:
    """The 32-bit generator word of each element index in ``elem``."""
    e = np.asarray(elem, dtype=np.uint64)
    g = e >> np.uint64(2)
    w = (e & np.uint64(3)).astype(np.int64)
    out = philox4x32_10(g & _MASK32, g >> np.uint64(32), np.full_like(g, tag),
                        np.zeros_like(g), seed & 0xFFFFFFFF, seed >> 32)
    stacked = np.stack(out, axis=-1)
    return np.take_along_axis(stacked, w[..., None], axis=-1)[..., 0]


def block_words(seed: int, tag: int, blocks) -> np.ndarray:
    """All four words of each block index in ``blocks``; shape [..., 4]."""
    g = np.asarray(blocks, dtype=np.uint64)
    out = philox4x32_10(g & _MASK32, g >> np.uint64(32), np.full_like(g, tag),
                        np.zeros_like(g), seed & 0xFFFFFFFF, seed >> 32)
    return np.stack(out, axis=-1)


def value_bits(kind: int, x: np.ndarray) -> np.ndarray:
    """Map generator words to element bits (uint16 for bf16, uint32 for fp32,
    int8 for int8) by the recipes in the module docstring."""
    x = x.astype(np.uint32)
    if kind in (KIND_BF16_NORMAL12, KIND_BF16_NORMAL6):
        s = ((x & 127) + ((x >> 7) & 127) + ((x >> 14) & 127)
             + ((x >> 21) & 127)).astype(np.int32) - 254
        e = 12 if kind == KIND_BF16_NORMAL12 else 6
        f = s.astype(np.float32) * np.float32(2.0 ** -e)   # exact
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    if kind == KIND_BF16_WIDE:
        sign = x & 1
        expo = 100 + ((x >> 1) & 31)
        mant = (x >> 6) & 127
        return ((sign << 15) | (expo << 7) | mant).astype(np.uint16)
    if kind == KIND_F32_UNIT:
        return ((x >> 8).astype(np.float32) * np.float32(2.0 ** -24)).view(np.uint32)
    if kind == KIND_I8_NORMAL:
        s = ((x & 63) + ((x >> 6) & 63) + ((x >> 12) & 63)
             + ((x >> 18) & 63)).astype(np.int32) - 126
        return s.astype(np.int8)
    if kind == KIND_F32_SCALE:
        m = (np.uint32(1 << 23) + (x & 0x7FFFFF)).astype(np.float32)  # exact
        return (m * np.float32(2.0 ** -34)).view(np.uint32)
    raise ValueError(f"unknown kind {kind}")


def mxfp4_bytes(kind: int, x: np.ndarray, b: np.ndarray, d: int) -> np.ndarray:
    """Bytes of 4-bit MXFP4 rows from generator words: the code bytes (two
    4-bit codes each) are the word's low byte; the scale bytes are E8M0
    exponents, 119 + (x & 3) or, for the wide kind, 100 + ((x >> 8) & 31)."""
    x = x.astype(np.uint32)
    scale = (119 + (x & 3)) if kind == KIND_MXFP4 else (100 + ((x >> 8) & 31))
    return np.where(np.asarray(b) < d // 2, x & 0xFF, scale).astype(np.uint8)


def mxfp4_row_bytes(d: int) -> int:
    return d // 2 + d // 32


def mxfp4_rows(kind: int, seed: int, tag: int, d: int, row_ids) -> np.ndarray:
    """Rows ``row_ids`` of a generated MXFP4 table: uint8 [len][d/2 + d/32]."""
    rb = mxfp4_row_bytes(d)
    r = np.asarray(row_ids, dtype=np.uint64).reshape(-1, 1)
    b = np.arange(rb, dtype=np.uint64)[None, :]
    return mxfp4_bytes(kind, words(seed, tag, r * np.uint64(rb) + b), b, d)


def tensor(kind: int, seed: int, tag: int, numel: int, offset: int = 0) -> np.ndarray:
    """Elements ``offset .. offset+numel-1`` of a generated tensor (flat)."""
    return value_bits(kind, words(seed, tag, np.arange(offset, offset + numel, dtype=np.uint64)))


def rows(kind: int, seed: int, tag: int, d: int, row_ids) -> np.ndarray:
    """Rows ``row_ids`` of a generated ``[R][d]`` tensor, on demand: shape
    ``[len(row_ids), d]``.  Needs no copy of the whole tensor."""
    r = np.asarray(row_ids, dtype=np.uint64).reshape(-1, 1)
    e = r * np.uint64(d) + np.arange(d, dtype=np.uint64)[None, :]
    return value_bits(kind, words(seed, tag, e))


def as_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def zipf_cdf(V: int, s: float) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-float(s))
    c = np.cumsum(w)
    return c / c[-1]


def _unit53(seed: int, tag: int, n: int, offset: int = 0) -> np.ndarray:
    b = block_words(seed, tag, np.arange(offset, offset + n, dtype=np.uint64))
    a = (b[:, 0] >> 5).astype(np.float64)      # 27 bits
    c = (b[:, 1] >> 6).astype(np.float64)      # 26 bits
    return (a * 67108864.0 + c) * (1.0 / 9007199254740992.0)


def tokens(seed: int, n: int, V: int, s: float = 1.1, dist: str = "zipf",
           tag: int = TAG_TOKENS, offset: int = 0) -> np.ndarray:
    """``n`` token ids in [0, V): Zipf(s) over ranks, or ``dist='uniform'``."""
    u = _unit53(seed, tag, n, offset)
    if dist == "uniform":
        ids = np.floor(u * V).astype(np.int64)
    elif dist == "zipf":
        ids = np.searchsorted(zipf_cdf(V, s), u, side="right")
    else:
        raise ValueError(dist)
    return np.minimum(ids, V - 1).astype(np.int32)


def workload_seed(config: int, batch: int = 0) -> int:
    """Seed of one synthetic batch of one workload (plain integer packing)."""
    return ((config & 0xFF) << 56) | ((batch & 0xFFFFFF) << 32) | 0x5EED


def seq_offsets(n_seqs: int, seq_len: int) -> np.ndarray:
    return (np.arange(n_seqs + 1, dtype=np.int64) * seq_len).astype(np.int32)


def ragged_offsets(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


# ------------------------------ GPU fill ------------------------------------
_gpu_lib = None


def _gpu():
    global _gpu_lib
    if _gpu_lib is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError("synth/libsynth.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(path)
        L.synth_fill.restype = ctypes.c_int
        L.synth_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        _gpu_lib = L
    return _gpu_lib


def fill_gpu(kind: int, seed: int, tag: int, t, offset: int = 0, stream=None):
    """Fill the CUDA tensor ``t`` (flat view) with elements ``offset ..`` of the
    generated tensor, on ``stream`` (default: the current stream)."""
    import torch
    assert t.is_cuda and t.is_contiguous()
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = _gpu().synth_fill(int(kind), seed & 0xFFFFFFFFFFFFFFFF, int(tag), t.data_ptr(),
                           t.numel(), int(offset), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill failed: {rc}")
    return t


def fill_gpu_mxfp4(kind: int, seed: int, tag: int, t, d: int, offset: int = 0, stream=None):
    """Fill the uint8 CUDA tensor ``t`` with bytes ``offset ..`` of a
    generated MXFP4 table of row width ``d``."""
    import ctypes

    import torch
    assert t.is_cuda and t.is_contiguous() and t.element_size() == 1
    if stream is None:
        stream = torch.cuda.current_stream()
    L = _gpu()
    L.synth_fill_mxfp4.restype = ctypes.c_int
    L.synth_fill_mxfp4.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    rc = L.synth_fill_mxfp4(int(kind), seed & 0xFFFFFFFFFFFFFFFF, int(tag), t.data_ptr(), t.numel(), int(offset),
                            int(d), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_mxfp4 failed: {rc}")
    return t
