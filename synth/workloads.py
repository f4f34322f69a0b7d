"""The synthetic workloads: shapes, distributions and seeds, and builders of
the same inputs on the host (numpy, rows on demand) and on the GPU (torch
tensors filled by the fill kernels).  Input generation only.

Workload shapes (the model the pages describe: 20M-row, 2560-wide table,
16 rows per token, vocab ~150K):

* tiny:     1 sequence x 256 tokens, V 1024, Zipf(1.1); table 4096 x 64 bf16;
            e1 1024 x 64; W_g[64]; no residual.
* decodeB:  B in {1, 2, 4} sequences x 1 token with a 2-token history, V 151936,
            Zipf(1.1); table 20,000,000 x 2560 bf16; e1 151936 x 2560; no residual.
* prefill:  8 x 4096 tokens (context reset at each sequence start), V 151936,
            Zipf(1.1); same table and e1; residual [32768][2560] bf16 ~N(0,1),
            updated in place.
* host:     1 x 8192 tokens, Zipf(1.1); table 5,000,000 x 2560 bf16 in pinned
            host memory; e1, W_g, residual as prefill.
* int8:     16 x 4096 tokens, Zipf(1.2); table 20,000,000 x 2560 int8 with a
            per-row fp32 scale; e1, W_g, residual as prefill.
* fp4:      the prefill batch over a 20,000,000 x 2560 MXFP4 table.
* gated:    the prefill batch and bf16 table through the normalised, gated
            fusion, with its parameters from gate_params().
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import (KIND_BF16_NORMAL6, KIND_BF16_NORMAL12, KIND_F32_SCALE, KIND_F32_UNIT,
               KIND_I8_NORMAL, KIND_MXFP4, mxfp4_row_bytes, mxfp4_rows, TAG_E1, TAG_GAMMA, TAG_GATE_U,
               TAG_GATE_V, TAG_HISTORY, TAG_RESIDUAL, TAG_SCALE, TAG_TABLE,
               TAG_TOKENS, TAG_WG, as_f32, ragged_offsets, rows, tensor, tokens, value_bits,
               words, workload_seed)


@dataclasses.dataclass
class Spec:
    name: str
    lengths: tuple
    V: int
    R: int
    d: int
    zipf_s: float = 1.1
    dist: str = "zipf"
    table: str = "bf16"                 # "bf16" | "int8" | "mxfp4"
    table_kind: int = KIND_BF16_NORMAL12
    e1: bool = True
    residual: bool = False
    history: bool = False
    config_id: int = 0
    batch: int = 0

    @property
    def n(self) -> int:
        return int(sum(self.lengths))

    @property
    def seed(self) -> int:
        return workload_seed(self.config_id, self.batch)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


BIG_R = 20_000_000
HOST_R = 5_000_000
VOCAB = 151936
D = 2560

CONFIGS = {
    "tiny": Spec("tiny", (256,), 1024, 4096, 64, config_id=1),
    "decode1": Spec("decode1", (1,), VOCAB, BIG_R, D, history=True, config_id=2),
    "decode2": Spec("decode2", (1, 1), VOCAB, BIG_R, D, history=True, config_id=2),
    "decode4": Spec("decode4", (1, 1, 1, 1), VOCAB, BIG_R, D, history=True, config_id=2),
    "prefill": Spec("prefill", (4096,) * 8, VOCAB, BIG_R, D, residual=True, config_id=3),
    "host": Spec("host", (8192,), VOCAB, HOST_R, D, residual=True, config_id=4),
    "int8": Spec("int8", (4096,) * 16, VOCAB, BIG_R, D, zipf_s=1.2, table="int8",
                 table_kind=KIND_I8_NORMAL, residual=True, config_id=5),
    # the prefill batch over a 4-bit table: 20M x (1280 + 80) bytes = 27.2 GB
    "fp4": Spec("fp4", (4096,) * 8, VOCAB, BIG_R, D, table="mxfp4", table_kind=KIND_MXFP4, residual=True,
                config_id=6),
    "gated": Spec("gated", (4096,) * 8, VOCAB, BIG_R, D, residual=True, config_id=7),
}


@dataclasses.dataclass
class GateParams:
    gamma: np.ndarray     # [d] fp32 in [0.5, 1.5)
    u: np.ndarray         # [d] fp32 in [-0.5, 0.5)
    v: np.ndarray         # [d] fp32 in [-2^-5, 2^-5)
    b: float
    eps: float


def gate_params(spec: Spec, b: float = 0.25, eps: float = 1e-6) -> GateParams:
    """Parameters of the normalised, gated fusion: exact fp32 shifts and
    power-of-two scalings of unit uniforms (Philox, tags 8..10)."""
    s, d = spec.seed, spec.d
    unit = lambda tag: as_f32(tensor(KIND_F32_UNIT, s, tag, d))
    gamma = (unit(TAG_GAMMA) + np.float32(0.5)).astype(np.float32)
    u = (unit(TAG_GATE_U) - np.float32(0.5)).astype(np.float32)
    v = ((unit(TAG_GATE_V) - np.float32(0.5)) * np.float32(2.0 ** -4)).astype(np.float32)
    return GateParams(gamma, u, v, float(np.float32(b)), float(np.float32(eps)))


class HostInputs:
    """The workload on the host: small tensors whole, big ones row by row."""

    def __init__(self, spec: Spec):
        self.spec = spec
        s = spec.seed
        self.tokens = tokens(s, spec.n, spec.V, spec.zipf_s, spec.dist)
        self.offsets = ragged_offsets(spec.lengths)
        self.history = (tokens(s, 2 * len(spec.lengths), spec.V, spec.zipf_s, spec.dist,
                               tag=TAG_HISTORY).reshape(-1, 2) if spec.history else None)
        self.W_g = as_f32(tensor(KIND_F32_UNIT, s, TAG_WG, spec.d))

    def table_rows(self, ids):
        s = self.spec
        if s.table == "mxfp4":
            return mxfp4_rows(s.table_kind, s.seed, TAG_TABLE, s.d, ids)
        return rows(s.table_kind, s.seed, TAG_TABLE, s.d, ids)

    def scale_rows(self, ids):
        s = self.spec
        ids = np.asarray(ids, dtype=np.uint64)
        return as_f32(value_bits(KIND_F32_SCALE, words(s.seed, TAG_SCALE, ids)))

    def e1_rows(self, ids):
        s = self.spec
        return rows(KIND_BF16_NORMAL12, s.seed, TAG_E1, s.d, ids)

    def residual_rows(self, token_idx):
        s = self.spec
        return rows(KIND_BF16_NORMAL6, s.seed, TAG_RESIDUAL, s.d, token_idx)

    def full_table(self):
        s = self.spec
        if s.table == "mxfp4":
            return self.table_rows(np.arange(s.R))
        return tensor(s.table_kind, s.seed, TAG_TABLE, s.R * s.d).reshape(s.R, s.d)

    def full_scale(self):
        s = self.spec
        return as_f32(tensor(KIND_F32_SCALE, s.seed, TAG_SCALE, s.R))

    def full_e1(self):
        s = self.spec
        return tensor(KIND_BF16_NORMAL12, s.seed, TAG_E1, s.V * s.d).reshape(s.V, s.d)

    def full_residual(self):
        s = self.spec
        return tensor(KIND_BF16_NORMAL6, s.seed, TAG_RESIDUAL, s.n * s.d).reshape(s.n, s.d)


class DeviceInputs:
    """The workload on the GPU (torch tensors, filled on the device)."""

    def __init__(self, spec: Spec, host: HostInputs | None = None, device="cuda:0",
                 table=True, e1=True, residual=True):
        import torch

        from . import fill_gpu, fill_gpu_mxfp4
        self.spec = spec
        h = host or HostInputs(spec)
        dev = torch.device(device)
        s = spec.seed
        self.tokens = torch.from_numpy(h.tokens).to(dev)
        self.offsets = torch.from_numpy(h.offsets).to(dev)
        self.history = None if h.history is None else torch.from_numpy(np.ascontiguousarray(h.history)).to(dev)
        self.W_g = torch.from_numpy(h.W_g).to(dev)
        self.table = self.scale = self.e1 = self.residual = None
        if table:
            if spec.table == "mxfp4":
                self.table = fill_gpu_mxfp4(spec.table_kind, s, TAG_TABLE,
                                            torch.empty(spec.R * mxfp4_row_bytes(spec.d), dtype=torch.uint8,
                                                        device=dev), spec.d)
            elif spec.table == "int8":
                self.table = fill_gpu(spec.table_kind, s, TAG_TABLE,
                                      torch.empty(spec.R * spec.d, dtype=torch.int8, device=dev))
                self.scale = fill_gpu(KIND_F32_SCALE, s, TAG_SCALE,
                                      torch.empty(spec.R, dtype=torch.float32, device=dev))
            else:
                self.table = fill_gpu(spec.table_kind, s, TAG_TABLE,
                                      torch.empty(spec.R * spec.d, dtype=torch.int16, device=dev))
        if e1 and spec.e1:
            self.e1 = fill_gpu(KIND_BF16_NORMAL12, s, TAG_E1,
                               torch.empty(spec.V * spec.d, dtype=torch.int16, device=dev))
        if residual and spec.residual:
            self.residual = fill_gpu(KIND_BF16_NORMAL6, s, TAG_RESIDUAL,
                                     torch.empty(spec.n * spec.d, dtype=torch.int16, device=dev))

    def table_obj(self):
        import hashed_gram_embedding_ngram_amd as ng
        sp = self.spec
        if sp.table == "int8":
            return ng.Table(self.table, sp.R, sp.d, ng.TABLE_INT8_ROWSCALE, row_scale=self.scale)
        if sp.table == "mxfp4":
            return ng.Table(self.table, sp.R, sp.d, ng.TABLE_MXFP4)
        return ng.Table(self.table, sp.R, sp.d)


def fill_host_table(spec: Spec, buf_np: np.ndarray, device="cuda:0", chunk_rows=1 << 16):
    """Fill a host array [R][d] (e.g. pinned memory) with the workload's table,
    generated on the GPU chunk by chunk and copied down."""
    import torch

    from . import fill_gpu, fill_gpu_mxfp4
    dev = torch.device(device)
    d = spec.d
    if spec.table == "mxfp4":
        per_row, dt = mxfp4_row_bytes(d), torch.uint8
    else:
        per_row, dt = d, (torch.int8 if spec.table == "int8" else torch.int16)
    tmp = torch.empty(chunk_rows * per_row, dtype=dt, device=dev)
    host = torch.from_numpy(buf_np.reshape(-1))
    for r0 in range(0, spec.R, chunk_rows):
        nr = min(chunk_rows, spec.R - r0)
        view = tmp[: nr * per_row]
        if spec.table == "mxfp4":
            fill_gpu_mxfp4(spec.table_kind, spec.seed, TAG_TABLE, view, d, offset=r0 * per_row)
        else:
            fill_gpu(spec.table_kind, spec.seed, TAG_TABLE, view, offset=r0 * per_row)
        host[r0 * per_row:(r0 + nr) * per_row].copy_(view, non_blocking=False)
    torch.cuda.synchronize()
