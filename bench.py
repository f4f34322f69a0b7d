"""Benchmark of the hashed n-gram embedding gather-sum on one MI355X.

A step is one pass of the whole path over one batch: ngram_forward (context,
hash, gather of 16 rows per token, fp32 sum, gate with e1 and W_g, residual
add, bf16 rounding) on the workload's batch, inputs resident in HBM.  The
default workload is prefill: 8 sequences x 4096 tokens (Zipf(1.1) over a
151936-token vocabulary), a 20,000,000 x 2560 bf16 table (95.4 GiB), e1
151936 x 2560 bf16, W_g[2560] fp32, residual [32768][2560] bf16 updated in
place.  Consecutive steps rotate over 4 distinct batches (tokens + residual,
672 MB of residual) so that no step finds the previous step's residual in
the 256 MB Infinity Cache.

Prints one JSON line: tokens/s over the timed steps, the roofline of the
fused kernel (algorithmic HBM bytes per launch / mean launch time from HIP
events on the launch stream, against 8 TB/s), and the CPU oracle's rate on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "n-gram gather-sum tokens/s; achieved GB/s as % of HBM (or PCIe) peak"
HBM_PEAK_GBPS = 8000.0
PCIE_PEAK_GBPS = 64.0          # PCIe Gen5 x16, one direction
K_ROWS = 16


def nominal_bytes_per_token(d: int, table: str = "bf16", e1: bool = True, residual: bool = True) -> int:
    """Algorithmic HBM bytes one token moves through the fused kernel: its 16
    table rows (bf16: 2 B per element; int8: 1 B per element plus a 4-byte row
    scale; MXFP4: half a byte per element plus one scale byte per 32), its e1 row, its residual row read and its output row written (2 B
    per element each), and its token id (4 B).  W_g (d x 4 B) is read once per
    launch and counted per launch, not per token."""
    row = {"bf16": d * 2, "int8": d + 4, "mxfp4": d // 2 + d // 32}[table]
    b = K_ROWS * row + 4
    if e1:
        b += 2 * d
    if residual:
        b += 2 * d
    b += 2 * d                 # output row
    return b


def dma_time_estimate_us(K: int, d: int, elem_bytes: int, bandwidth_gbps: float) -> float:
    """Closed-form PCIe time of one token's rows: K * d * S / bandwidth
    ("Qwen3.8-Flash-Next: A 51B N-gram Embedding Table with Heterogeneous
    Memory Prefetch", Key point 3, the T_DMA equation)."""
    return K * d * elem_bytes / (bandwidth_gbps * 1e9) * 1e6


def table_bytes(R: int, d: int, table: str = "bf16") -> int:
    return R * {"bf16": 2 * d, "int8": d + 4, "mxfp4": d // 2 + d // 32}[table]


def source_sha256() -> str:
    p = os.path.join(ROOT, "hashed_gram_embedding_ngram_amd", "csrc", "ngram.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_sha256():
        return None
    return t.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "int8", "fp4", "gated", "projected", "decode1", "decode2", "decode4", "host",
                             "backward", "unfused"])
    ap.add_argument("--host-mode", default="zero_copy", choices=["zero_copy", "staged", "async", "pool"],
                    help="host workload: sum straight from pinned memory; stage the distinct rows in HBM first, "
                         "read by GPU workgroups (staged) or copied by the DMA engines (async); or go through an "
                         "HBM row pool (hot-row cache + per-batch dedup)")
    ap.add_argument("--host-wgs", type=int, default=0,
                    help="host workload, zero copy: workgroups of the capped grid that reads the host table "
                         "(0: the library's choice)")
    ap.add_argument("--cu-split", type=int, default=0,
                    help="host workload: run the gather on a stream confined to the first N compute units and "
                         "the GEMM stand-in on a stream confined to the others (0: no confinement)")
    ap.add_argument("--interference", action="store_true",
                    help="host workload: also time the GEMM stand-in beside other PCIe readers (the same gather "
                         "kernel over consecutive rows, a DMA copy of the same bytes) to separate the causes of "
                         "its slowdown")
    ap.add_argument("--cache-rows", type=int, default=1 << 22, help="pool mode: rows of the hot-row cache")
    ap.add_argument("--cache-history", type=int, default=32, help="pool mode: earlier batches counted")
    ap.add_argument("--dist", default="zipf", choices=["zipf", "uniform"],
                    help="token distribution (uniform: the no-reuse control)")
    ap.add_argument("--batches", type=int, default=4, help="distinct batches rotated over")
    ap.add_argument("--graph", action="store_true",
                    help="capture one launch per batch in a HIP graph and time graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tpw", type=int, default=0,
                    help="tokens per workgroup of the gather kernels (0: the library's choice)")
    ap.add_argument("--serial", action="store_true",
                    help="backward: the three gradient calls in order on one stream")
    ap.add_argument("--cpu-rows", type=int, default=1_000_000,
                    help="table rows of the host copy the CPU oracle reads")
    ap.add_argument("--gather-probe", action="store_true",
                    help="run only a bare random-row gather (16 rows per token of the prefill batch, reads only) "
                         "at several row sizes and load widths: what the memory system delivers for each")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy kernel (for scaling HBM counters)")
    return ap.parse_args()


def cpu_baseline(host_inputs, table_np, scale_np, e1_np, res_np, R_cpu, prep_s, table_note, mxfp4_d=None,
                 gate=None, repeats=5, chunk=512):
    """The oracle timed on the host cores on a bounded sample of the
    workload: the whole batch, hashed into a host copy of the first ``R_cpu``
    table rows when the full table does not fit in host memory (a random-row
    gather far beyond the last-level cache is DRAM-bound either way).  The
    batch is cut into ``chunk``-token pieces, each carrying its 2-token
    history, so that every core has work and the results are those of the
    whole batch; one oracle_forward call per piece (or the oracle's hash,
    sum and normalised gated fusion) on a pool of threads.  Reported: the
    median of ``repeats`` passes on all cores the process may use (at most
    16), and the median of ``repeats`` passes over the first sequence on 1
    core."""
    import concurrent.futures as cf
    import statistics

    import numpy as np

    import oracle

    toks, offs, hist = host_inputs.tokens, host_inputs.offsets, host_inputs.history
    pieces = []
    for sq in range(len(offs) - 1):
        a0, b0 = int(offs[sq]), int(offs[sq + 1])
        for a in range(a0, b0, chunk):
            b = min(b0, a + chunk)
            if a == a0:
                h = None if hist is None else np.ascontiguousarray(hist[sq:sq + 1])
            else:
                h = np.array([[toks[a - 2], toks[a - 1]]], np.int32)
            pieces.append((sq, a, b, h))

    def one(piece):
        sq, a, b, h = piece
        so = np.array([0, b - a], np.int32)
        res = None if res_np is None else res_np[a:b]
        if gate is None:
            oracle.forward(toks[a:b], so, table_np, host_inputs.W_g, e1=e1_np, residual=res,
                           history=h, scale=scale_np, mxfp4_d=mxfp4_d)
        else:
            rows = oracle.hash_rows(toks[a:b], so, R_cpu, h)
            eN = oracle.embed_bag_bf16(table_np, rows)
            oracle.norm_gate_add(eN, toks[a:b], e1_np, host_inputs.W_g, gate.gamma, gate.u, gate.v,
                                 gate.b, gate.eps, res)
        return b - a

    def timed_pass(work, threads):
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            done = sum(ex.map(one, work))
        return done, time.perf_counter() - t0

    threads = max(1, min(len(os.sched_getaffinity(0)), 16, len(pieces)))
    all_passes = [timed_pass(pieces, threads) for _ in range(repeats)]
    first_seq = [pc for pc in pieces if pc[0] == 0]
    one_passes = [timed_pass(first_seq, 1) for _ in range(repeats)]
    n_all, n_one = all_passes[0][0], one_passes[0][0]
    rate_all = [n_all / w for _, w in all_passes]
    rate_one = [n_one / w for _, w in one_passes]
    what = ("the oracle hash, sum and normalised gated fusion" if gate is not None
            else "one oracle_forward call")
    return {
        "value": statistics.median(rate_all),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"the {n_all}-token batch in {len(pieces)} pieces of up to {chunk} tokens ({what} per piece, "
                   f"each with its 2-token history), median of {repeats} passes on {threads} threads; {table_note}; "
                   f"prep {prep_s:.1f} s, not timed"),
        "single_core": {"value": statistics.median(rate_one), "unit": "tokens/s", "cores": 1,
                        "sample": f"the first sequence ({n_one} tokens), median of {repeats} passes"},
        "passes_s": [round(w, 4) for _, w in all_passes],
        "cpu_model": _cpu_model(),
        "wall_s": sum(w for _, w in all_passes) + sum(w for _, w in one_passes),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path is built and measured on a single MI355X; it has no multi-GPU mode)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        # A plain elementwise copy of known size: reads 1 GiB, writes 1 GiB per
        # launch.  HBM counters of this kernel give the scale of the counters.
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            torch.mul(src, 3, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 4,
                          "calibrate_copy_bytes_written": dst.numel() * 4, "launches": args.steps}))
        return

    import hashed_gram_embedding_ngram_amd as ng
    import synth
    from synth.workloads import CONFIGS, HostInputs

    if args.gather_probe:
        run_gather_probe(args)
        return
    if args.workload == "host":
        run_host(args)
        return
    if args.workload == "backward":
        run_backward(args)
        return
    if args.workload == "projected":
        run_projected(args)
        return
    if args.workload == "unfused":
        run_unfused(args)
        return

    dev = torch.device("cuda:0")
    spec = CONFIGS[args.workload].replace(dist=args.dist)
    n, d = spec.n, spec.d
    t_setup = time.time()

    # Shared tensors: table, e1, W_g (batch 0's seed).
    h0 = HostInputs(spec)
    s0 = spec.seed
    if spec.table == "int8":
        table = synth.fill_gpu(spec.table_kind, s0, synth.TAG_TABLE,
                               torch.empty(spec.R * d, dtype=torch.int8, device=dev))
        scale = synth.fill_gpu(synth.KIND_F32_SCALE, s0, synth.TAG_SCALE,
                               torch.empty(spec.R, dtype=torch.float32, device=dev))
        T = ng.Table(table, spec.R, d, ng.TABLE_INT8_ROWSCALE, row_scale=scale)
    elif spec.table == "mxfp4":
        table = synth.fill_gpu_mxfp4(spec.table_kind, s0, synth.TAG_TABLE,
                                     torch.empty(spec.R * synth.mxfp4_row_bytes(d), dtype=torch.uint8, device=dev), d)
        scale = None
        T = ng.Table(table, spec.R, d, ng.TABLE_MXFP4)
    else:
        table = synth.fill_gpu(spec.table_kind, s0, synth.TAG_TABLE,
                               torch.empty(spec.R * d, dtype=torch.int16, device=dev))
        scale = None
        T = ng.Table(table, spec.R, d)
    e1 = synth.fill_gpu(synth.KIND_BF16_NORMAL12, s0, synth.TAG_E1,
                        torch.empty(spec.V * d, dtype=torch.int16, device=dev)) if spec.e1 else None
    W_g = torch.from_numpy(h0.W_g).to(dev)

    # Rotating batches: tokens, offsets, history, residual (in place), out.
    nb = max(1, args.batches)
    batches = []
    for b in range(nb):
        hb = h0 if b == 0 else HostInputs(spec.replace(batch=b))
        tok = torch.from_numpy(hb.tokens).to(dev)
        off = torch.from_numpy(hb.offsets).to(dev)
        hist = None if hb.history is None else torch.from_numpy(np.ascontiguousarray(hb.history)).to(dev)
        if spec.residual:
            res = synth.fill_gpu(synth.KIND_BF16_NORMAL6, spec.replace(batch=b).seed, synth.TAG_RESIDUAL,
                                 torch.empty(n * d, dtype=torch.int16, device=dev))
            out = res
        else:
            res = None
            out = torch.empty(n * d, dtype=torch.int16, device=dev)
        batches.append((tok, off, hist, res, out))
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    stream = torch.cuda.current_stream()
    gated = args.workload == "gated"
    if gated:
        from synth.workloads import gate_params
        gp = gate_params(spec)
        g_gamma, g_u, g_v = (torch.from_numpy(a).to(dev) for a in (gp.gamma, gp.u, gp.v))

    shape = (args.tpw, 0) if args.tpw else None

    def launch(tok, off, hist, res, out, stream=None):
        if gated:
            ng.ngram_forward_gated(tok, off, T, W_g, g_gamma, g_u, g_v, gp.b, gp.eps, out, e1,
                                   residual=res, history=hist, launch=shape, stream=stream)
        else:
            ng.ngram_forward(tok, off, T, W_g, out, e1=e1, residual=res, history=hist, launch=shape,
                             stream=stream)

    def step(i):
        tok, off, hist, res, out = batches[i % nb]
        launch(tok, off, hist, res, out, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    if args.graph:
        # One graph holds one launch per batch; each replay runs nb steps.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nb):
                launch(*batches[i])
        reps = max(1, args.steps // nb)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s_ev.record()
        for _ in range(reps):
            g.replay()
        e_ev.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        args.steps = reps * nb
        mean_launch_s = s_ev.elapsed_time(e_ev) / 1e3 / args.steps
        latency_floor = graph_floor(batches, e1, d, nb, reps)
    else:
        latency_floor = None
        # one event pair around the back-to-back launches on the launch
        # stream: the mean interval per launch (kernel + dispatch gap), which
        # per-launch pairs would inflate by each event's own processing
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        s_ev.record(stream)
        for i in range(args.steps):
            step(args.warmup + i)
        e_ev.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mean_launch_s = s_ev.elapsed_time(e_ev) / 1e3 / args.steps

    bpt = nominal_bytes_per_token(d, spec.table, spec.e1, spec.residual)
    bytes_per_launch = bpt * n + 4 * d * (4 if gated else 1)          # W_g (+ gamma, u, v) once per launch
    achieved = bytes_per_launch / mean_launch_s / 1e9
    traffic = measured_traffic(args.workload if args.dist == "zipf" else f"{args.workload}_{args.dist}")

    result = {
        "metric": METRIC,
        "value": n * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": spec.name,
            "tokens": n,
            "sequences": len(spec.lengths),
            "seq_len": spec.lengths[0],
            "R": spec.R,
            "d": d,
            "K": K_ROWS,
            "table_dtype": spec.table,
            "vocab": spec.V,
            "token_dist": f"zipf({spec.zipf_s})" if args.dist == "zipf" else "uniform",
            "residual_in_place": spec.residual,
            "rotating_batches": nb,
            "hip_graph": bool(args.graph),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel": "ngram_gated_kernel" if gated else "ngram_fwd_kernel",
            "algorithmic_bytes_per_token": bpt,
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "mean_launch_us": mean_launch_s * 1e6,
        },
        "setup_s": setup_s,
    }
    if latency_floor is not None:
        result["latency_floor"] = latency_floor

    if not args.no_cpu_baseline:
        R_cpu = min(args.cpu_rows, spec.R)
        tp = time.time()
        if spec.table == "int8":
            table_np = table[: R_cpu * d].cpu().numpy().reshape(R_cpu, d)
            scale_np = scale[:R_cpu].cpu().numpy()
        elif spec.table == "mxfp4":
            rb = synth.mxfp4_row_bytes(d)
            table_np = table[: R_cpu * rb].cpu().numpy().reshape(R_cpu, rb)
            scale_np = None
        else:
            table_np = table[: R_cpu * d].cpu().numpy().view(np.uint16).reshape(R_cpu, d)
            scale_np = None
        e1_np = None if e1 is None else e1.cpu().numpy().view(np.uint16).reshape(spec.V, d)
        res_np = None if batches[0][3] is None else batches[0][3].cpu().numpy().view(np.uint16).reshape(n, d)
        note = (f"rows hashed mod {R_cpu} into a {table_np.nbytes / 2**30:.2f} GiB host copy of the first "
                f"{R_cpu} of the {spec.R} table rows (the full table does not fit in host memory)")
        result["cpu_baseline"] = cpu_baseline(HostInputs(spec.replace(R=R_cpu)), table_np, scale_np,
                                              e1_np, res_np, R_cpu, time.time() - tp, note,
                                              mxfp4_d=d if spec.table == "mxfp4" else None,
                                              gate=gp if gated else None)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def graph_floor(batches, e1, d, nb, reps):
    """What a graph-replayed step costs at least, measured the same way as the
    step (one graph holding nb launches, replayed reps times): an empty
    kernel (torch.cuda._sleep(0)), and one kernel that loads the batch's
    token ids and then, dependent on them, their e1 rows (torch.index_select:
    launch + a dependent pair of memory round trips, which is the shape of a
    decode step's critical path: token ids, then the rows they select)."""
    import torch

    def replay_us(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nb):
                body(i)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        for _ in range(reps):
            g.replay()
        e_ev.record()
        torch.cuda.synchronize()
        return s_ev.elapsed_time(e_ev) * 1e3 / (reps * nb)

    floor = {"empty_kernel_us": replay_us(lambda i: torch.cuda._sleep(0))}
    if e1 is not None:
        table = e1.view(-1, d)
        outs = [torch.empty((batches[i][0].numel(), d), dtype=table.dtype, device=table.device) for i in range(nb)]
        floor["token_then_row_load_us"] = replay_us(
            lambda i: torch.index_select(table, 0, batches[i][0], out=outs[i]))
    return floor


def backward_bytes_per_token(d: int, rows_per_token_unique: float, tokens_unique: float) -> float:
    """Algorithmic HBM bytes of one backward step per token: the 16 reads of
    its dL/dout row by the table's segmented reduce (16 x 2d), its share of
    the fp32 table-gradient rows written (unique rows per token x 4d), the
    e1 reduce's read of dL/dout (2d) and write of unique-token rows
    (x 4d), and the gate gradient's read of dL/dout and eN (2d + 4d)."""
    return 16 * 2 * d + rows_per_token_unique * 4 * d + 2 * d + tokens_unique * 4 * d + 6 * d


def run_gather_probe(args):
    """A bare gather of the prefill batch's 16 rows per token (the same
    hashed row ids, R = 20M) from a table of R rows of S bytes, L bytes per
    lane, reads only (synth/libprobe.so): the rate the memory system gives
    random rows of each size, against which the fused kernels' rates are
    read.  S: 1360 (an MXFP4 row at d = 2560), 2560 (int8), 5120 (bf16)."""
    import ctypes

    import torch

    import hashed_gram_embedding_ngram_amd as ng
    from synth.workloads import CONFIGS, HostInputs

    dev = torch.device("cuda:0")
    spec = CONFIGS["prefill"]
    n, R = spec.n, spec.R
    h = HostInputs(spec)
    rows = ng.ngram_hash(torch.from_numpy(h.tokens).to(dev), torch.from_numpy(h.offsets).to(dev), R)
    tab = torch.empty(R * 5120, dtype=torch.uint8, device=dev)       # contents do not matter
    out = torch.empty(n, dtype=torch.int32, device=dev)
    probe = ctypes.CDLL(os.path.join(ROOT, "synth", "libprobe.so"))
    stream = torch.cuda.current_stream()
    res = []
    for S, L in ((1360, 4), (1360, 8), (1360, 16), (2560, 4), (2560, 8), (2560, 16), (5120, 8), (5120, 16)):
        def go():
            rc = probe.probe_gather(ctypes.c_void_p(tab.data_ptr()), ctypes.c_int64(S), ctypes.c_void_p(rows.data_ptr()),
                                    ctypes.c_int64(n), ctypes.c_int32(L), ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"probe_gather({S}, {L}) failed: {rc}")
        for _ in range(args.warmup):
            go()
        torch.cuda.synchronize()
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record(stream)
        for _ in range(args.steps):
            go()
        e_ev.record(stream)
        torch.cuda.synchronize()
        t = s_ev.elapsed_time(e_ev) / 1e3 / args.steps
        gbps = n * 16 * S / t / 1e9
        res.append({"row_bytes": S, "lane_bytes": L, "us_per_launch": t * 1e6, "GBps": gbps, "frac": gbps / HBM_PEAK_GBPS})
    # the fused forward's byte mix without its arithmetic: the same gather
    # plus an e1 row (by token id, V x 5120 B), a residual row read and an
    # output row written per token (5120 B each, d = 2560 bf16)
    side = 2 * spec.d
    tokens = torch.from_numpy(h.tokens).to(dev)
    e1 = torch.empty(spec.V * side, dtype=torch.uint8, device=dev)
    resid = torch.empty(n * side, dtype=torch.uint8, device=dev)
    outb = torch.empty(n * side, dtype=torch.uint8, device=dev)
    mix = []
    for S, L in ((1360, 4), (1360, 16), (2560, 8), (5120, 16)):
        def go():
            rc = probe.probe_gather_mix(ctypes.c_void_p(tab.data_ptr()), ctypes.c_int64(S),
                                        ctypes.c_void_p(rows.data_ptr()), ctypes.c_int64(n), ctypes.c_int32(L),
                                        ctypes.c_void_p(tokens.data_ptr()), ctypes.c_void_p(e1.data_ptr()),
                                        ctypes.c_void_p(resid.data_ptr()), ctypes.c_int64(side),
                                        ctypes.c_void_p(outb.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"probe_gather_mix({S}, {L}) failed: {rc}")
        for _ in range(args.warmup):
            go()
        torch.cuda.synchronize()
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record(stream)
        for _ in range(args.steps):
            go()
        e_ev.record(stream)
        torch.cuda.synchronize()
        t = s_ev.elapsed_time(e_ev) / 1e3 / args.steps
        gbps = n * (16 * S + 3 * side) / t / 1e9
        mix.append({"row_bytes": S, "lane_bytes": L, "side_bytes": side, "us_per_launch": t * 1e6, "GBps": gbps,
                    "frac": gbps / HBM_PEAK_GBPS})
    print(json.dumps({"gather_probe": res, "gather_mix_probe": mix, "tokens": n, "R": R, "rows_per_token": 16}),
          flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak


def run_projected(args):
    """The projected path at the prefill shape: hash and gather-sum (the fp32
    sums rounded to bf16), projection by a 2560 x 2560 bf16 weight (bf16
    MFMA, fp32 accumulation), then the normalised, input-gated epilogue with
    the residual in place.  The sums come from the fused forward with W_g = 1
    and neither e1 nor residual: its output is then bf16(fmaf(1, s, +0)) =
    bf16(s) for every sum s (a sum that starts from +0 is never -0), the
    same bits as ngram_hash + ngram_embed_bag_bf16 in one launch.  A step is
    the three launches on one stream; each launch is timed with HIP events.
    The roofline object is the projection's (matrix-core bound: 2 n d_in
    d_out flops per launch against the dense bf16 peak)."""
    import statistics

    import numpy as np
    import torch

    import hashed_gram_embedding_ngram_amd as ng
    import synth
    from synth.workloads import CONFIGS, HostInputs, gate_params

    dev = torch.device("cuda:0")
    spec = CONFIGS["prefill"].replace(dist=args.dist)
    n, d = spec.n, spec.d
    t_setup = time.time()
    h = HostInputs(spec)
    s0 = spec.seed
    table = synth.fill_gpu(spec.table_kind, s0, synth.TAG_TABLE, torch.empty(spec.R * d, dtype=torch.int16, device=dev))
    T = ng.Table(table, spec.R, d)
    e1 = synth.fill_gpu(synth.KIND_BF16_NORMAL12, s0, synth.TAG_E1, torch.empty(spec.V * d, dtype=torch.int16, device=dev))
    W_g = torch.from_numpy(h.W_g).to(dev)
    gp = gate_params(spec)
    g_gamma, g_u, g_v = (torch.from_numpy(a).to(dev) for a in (gp.gamma, gp.u, gp.v))
    w = (np.random.default_rng(s0).standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)
    P = torch.from_numpy((w.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)).to(dev)
    tok = torch.from_numpy(h.tokens).to(dev)
    off = torch.from_numpy(h.offsets).to(dev)
    res = synth.fill_gpu(synth.KIND_BF16_NORMAL6, s0, synth.TAG_RESIDUAL, torch.empty(n * d, dtype=torch.int16, device=dev))
    ones = torch.ones(d, dtype=torch.float32, device=dev)
    xb = torch.empty((n, d), dtype=torch.int16, device=dev)
    p = torch.empty((n, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    stream = torch.cuda.current_stream()
    names = ["hash_sum_bf16", "project", "norm_gate_add"]

    def stages():
        return [lambda: ng.ngram_forward(tok, off, T, ones, xb, stream=stream),
                lambda: ng.ngram_project(xb, P, y=p, stream=stream),
                lambda: ng.ngram_norm_gate_add(p, tok, e1, W_g, g_gamma, g_u, g_v, gp.b, gp.eps, res, residual=res,
                                               stream=stream)]

    fns = stages()
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for k, f in enumerate(fns):
            f()
            ev[i][k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {nm: statistics.mean(ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps)) * 1e3
           for k, nm in enumerate(names)}
    proj_s = per["project"] / 1e6
    flops = 2.0 * n * d * d
    achieved = flops / proj_s / 1e12
    result = {
        "metric": METRIC,
        "value": n * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x bf16 -> f32 (projection), f32/f64 elsewhere",
        "data": "synthetic",
        "config": {"workload": "projected", "tokens": n, "sequences": len(spec.lengths), "R": spec.R, "d": d,
                   "d_out": d, "K": K_ROWS, "table_dtype": spec.table, "vocab": spec.V,
                   "token_dist": f"zipf({spec.zipf_s})" if args.dist == "zipf" else "uniform",
                   "residual_in_place": True},
        "stage_us": per,
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "kernel": "project_kernel",
            "algorithmic_flops_per_launch": flops,
            "mean_launch_us": per["project"],
        },
        "setup_s": setup_s,
        "cpu_baseline": None if args.no_cpu_baseline else projected_cpu_baseline(h, table, e1, res, P, gp, spec),
    }
    print(json.dumps(result), flush=True)


def run_unfused(args):
    """The prefill batch through the three separate calls: ngram_hash (row ids
    to HBM), ngram_embed_bag (the fp32 sums to HBM) and ngram_gate_add (gate
    with e1 and W_g, residual added in place, bf16 out); the same outputs as
    the fused forward, with the row ids and the sums written and read back.
    A step is the three launches on one stream, each timed with HIP events;
    the roofline object is the sum kernel's (16 rows and 64 B of row ids read
    and 4 d bytes of sums written per token)."""
    import statistics

    import torch

    import hashed_gram_embedding_ngram_amd as ng
    import synth
    from synth.workloads import CONFIGS, HostInputs

    dev = torch.device("cuda:0")
    spec = CONFIGS["prefill"].replace(dist=args.dist)
    n, d = spec.n, spec.d
    t_setup = time.time()
    h = HostInputs(spec)
    s0 = spec.seed
    table = synth.fill_gpu(spec.table_kind, s0, synth.TAG_TABLE, torch.empty(spec.R * d, dtype=torch.int16, device=dev))
    T = ng.Table(table, spec.R, d)
    e1 = synth.fill_gpu(synth.KIND_BF16_NORMAL12, s0, synth.TAG_E1, torch.empty(spec.V * d, dtype=torch.int16, device=dev))
    W_g = torch.from_numpy(h.W_g).to(dev)
    tok = torch.from_numpy(h.tokens).to(dev)
    off = torch.from_numpy(h.offsets).to(dev)
    res = synth.fill_gpu(synth.KIND_BF16_NORMAL6, s0, synth.TAG_RESIDUAL, torch.empty(n * d, dtype=torch.int16, device=dev))
    rows = torch.empty((n, K_ROWS), dtype=torch.int32, device=dev)
    eN = torch.empty((n, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    stream = torch.cuda.current_stream()
    names = ["hash", "embed_bag", "gate_add"]
    fns = [lambda: ng.ngram_hash(tok, off, spec.R, rows_out=rows, stream=stream),
           lambda: ng.ngram_embed_bag(T, rows, eN_out=eN, stream=stream),
           lambda: ng.ngram_gate_add(eN, tok, W_g, res, e1=e1, residual=res, stream=stream)]
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for k, f in enumerate(fns):
            f()
            ev[i][k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {nm: statistics.mean(ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps)) * 1e3
           for k, nm in enumerate(names)}
    bag_bytes = n * (K_ROWS * 2 * d + K_ROWS * 4 + 4 * d)
    achieved = bag_bytes / (per["embed_bag"] / 1e6) / 1e9
    print(json.dumps({
        "metric": METRIC, "value": n * args.steps / wall, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "unfused", "tokens": n, "sequences": len(spec.lengths), "R": spec.R, "d": d,
                   "K": K_ROWS, "table_dtype": spec.table, "vocab": spec.V,
                   "token_dist": f"zipf({spec.zipf_s})" if args.dist == "zipf" else "uniform",
                   "residual_in_place": True},
        "stage_us": per,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "kernel": "ngram_bag_kernel",
                     "algorithmic_bytes_per_launch": bag_bytes, "mean_launch_us": per["embed_bag"],
                     "gate_add_bytes_per_launch": n * 10 * d,
                     "gate_add_frac": n * 10 * d / (per["gate_add"] / 1e6) / 1e9 / HBM_PEAK_GBPS},
        "setup_s": setup_s, "cpu_baseline": None}), flush=True)


def projected_cpu_baseline(h, table, e1, res, P, gp, spec, m=256, repeats=5):
    """The oracle's projected path (hash, sum, float64 projection, normalised
    gated fusion) on the first m tokens of the batch, rows hashed into a host
    copy of the first 1,000,000 table rows, one piece of m / 16 tokens per
    thread; median of ``repeats`` passes, and of ``repeats`` passes on 1 core."""
    import concurrent.futures as cf
    import statistics

    import numpy as np

    import oracle

    d = spec.d
    R_cpu = 1_000_000
    tp = time.time()
    table_np = table[: R_cpu * d].cpu().numpy().view(np.uint16).reshape(R_cpu, d)
    e1_np = e1.cpu().numpy().view(np.uint16).reshape(spec.V, d)
    res_np = res[: m * d].cpu().numpy().view(np.uint16).reshape(m, d)
    P_np = P.cpu().numpy().view(np.uint16)
    prep = time.time() - tp
    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    step = (m + threads - 1) // threads
    toks = h.tokens[:m]
    pieces = [(a, min(m, a + step)) for a in range(0, m, step)]

    def one(piece):
        a, b = piece
        hist = None if a == 0 else np.array([[toks[a - 2] if a >= 2 else (1 << 21) - 1, toks[a - 1]]], np.int32)
        rows = oracle.hash_rows(toks[a:b], np.array([0, b - a], np.int32), R_cpu, hist)
        eN = oracle.embed_bag_bf16(table_np, rows)
        y, _ = oracle.project(eN, P_np)
        oracle.norm_gate_add(y.astype(np.float32), toks[a:b], e1_np, h.W_g, gp.gamma, gp.u, gp.v, gp.b, gp.eps,
                             res_np[a:b])
        return b - a

    def timed(work, nthreads):
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(nthreads) as ex:
            done = sum(ex.map(one, work))
        return done / (time.perf_counter() - t0)

    rate_all = [timed(pieces, threads) for _ in range(repeats)]
    rate_one = [timed(pieces[:1], 1) for _ in range(repeats)]
    return {"value": statistics.median(rate_all), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"the first {m} tokens of the batch in {len(pieces)} pieces (oracle hash, sum, float64 "
                       f"projection by the {d} x {d} weight, normalised gated fusion), rows hashed mod {R_cpu} into "
                       f"a host copy of the first {R_cpu} table rows; median of {repeats} passes; prep {prep:.1f} s"),
            "single_core": {"value": statistics.median(rate_one), "unit": "tokens/s", "cores": 1,
                            "sample": f"the first piece ({pieces[0][1]} tokens), median of {repeats} passes"},
            "cpu_model": _cpu_model()}


def cu_masked_streams(n_side: int):
    """Two streams of default priority on disjoint compute units: the first
    ``n_side`` CUs for the side stream, the rest for the main stream
    (hipExtStreamCreateWithCUMask of the HIP runtime torch has loaded)."""
    import ctypes

    import torch

    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    total = torch.cuda.get_device_properties(0).multi_processor_count
    words = (total + 31) // 32

    def make(cus):
        mask = (ctypes.c_uint32 * words)()
        for c in cus:
            mask[c // 32] |= 1 << (c % 32)
        h = ctypes.c_void_p()
        rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), mask)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({rc})")
        return torch.cuda.ExternalStream(h.value)

    return make(range(n_side)), make(range(n_side, total)), total


def run_backward(args):
    """Gradients of one prefill batch (8 x 4096 tokens, R = 20M, d = 2560):
    ngram_grad_table + ngram_grad_e1 + ngram_grad_gate, from the forward's
    row ids and sums and a synthetic bf16 dL/dout."""
    import numpy as np
    import torch

    import hashed_gram_embedding_ngram_amd as ng
    import synth
    from synth.workloads import CONFIGS, HostInputs

    dev = torch.device("cuda:0")
    spec = CONFIGS["prefill"].replace(dist=args.dist)
    n, d, R = spec.n, spec.d, spec.R
    h = HostInputs(spec)
    tok = torch.from_numpy(h.tokens).to(dev)
    off = torch.from_numpy(h.offsets).to(dev)
    W = torch.from_numpy(h.W_g).to(dev)
    table = synth.fill_gpu(spec.table_kind, spec.seed, synth.TAG_TABLE, torch.empty(R * d, dtype=torch.int16, device=dev))
    rows = ng.ngram_hash(tok, off, R)
    eN = ng.ngram_embed_bag(ng.Table(table, R, d), rows)
    del table
    g = synth.fill_gpu(synth.KIND_BF16_NORMAL6, 77, synth.TAG_RESIDUAL, torch.empty(n * d, dtype=torch.int16, device=dev))
    ws = ng.grad_workspace(n, d, dev)
    gr = torch.empty(n * 16, dtype=torch.int32, device=dev)
    gt = torch.empty((n * 16, d), dtype=torch.float32, device=dev)
    nu = torch.empty(1, dtype=torch.int64, device=dev)
    et = torch.empty(n, dtype=torch.int32, device=dev)
    ge = torch.empty((n, d), dtype=torch.float32, device=dev)
    ne = torch.empty(1, dtype=torch.int64, device=dev)
    gw = torch.empty(d, dtype=torch.float32, device=dev)

    # The table gradient (HBM-bound) on the main stream; the gate and e1
    # gradients on a side stream with their own workspace, joined at the end
    # of the step.  --serial runs all three in order on one stream.
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ws2 = ng.grad_workspace(n, d, dev)
    ev_in, ev_side = torch.cuda.Event(), torch.cuda.Event()

    def step():
        if args.serial:
            ng.ngram_grad_table(rows, W, g, R, grad_rows_out=gr, grad_out=gt, n_unique_out=nu, workspace=ws)
            ng.ngram_grad_e1(tok, rows, g, spec.V, grad_tokens_out=et, grad_out=ge, n_unique_out=ne, workspace=ws)
            ng.ngram_grad_gate(rows, g, eN, grad_Wg_out=gw, workspace=ws)
            return
        ev_in.record(main)
        side.wait_event(ev_in)
        # the gate gradient (bandwidth-bound) first, while the main stream
        # sorts the row ids (little traffic); then the e1 gradient
        ng.ngram_grad_gate(rows, g, eN, grad_Wg_out=gw, workspace=ws2, stream=side)
        ng.ngram_grad_e1(tok, rows, g, spec.V, grad_tokens_out=et, grad_out=ge, n_unique_out=ne, workspace=ws2,
                         stream=side)
        ng.ngram_grad_table(rows, W, g, R, grad_rows_out=gr, grad_out=gt, n_unique_out=nu, workspace=ws,
                            stream=main)
        ev_side.record(side)
        main.wait_event(ev_side)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s_ev.record()
    for _ in range(args.steps):
        step()
    e_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = s_ev.elapsed_time(e_ev) / 1e3 / args.steps
    U, Ut = int(nu.item()), int(ne.item())
    bpt = backward_bytes_per_token(d, U / n, Ut / n)
    achieved = bpt * n / step_s / 1e9
    print(json.dumps({
        "metric": "n-gram backward (table + e1 + gate gradients) tokens/s",
        "value": n * args.steps / wall, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "backward", "tokens": n, "R": R, "d": d, "K": K_ROWS,
                   "unique_rows": U, "unique_tokens": Ut, "streams": 1 if args.serial else 2},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "kernel": "backward step",
                     "algorithmic_bytes_per_token": bpt, "step_us": step_s * 1e6},
        "cpu_baseline": None}), flush=True)


def run_host(args):
    """The pinned-host-table workload: 8192 tokens, a 5,000,000 x 2560 bf16
    table in pinned host memory.  Side stream: hash, then the 16 rows of each
    token read by the GPU over PCIe and summed into an fp32 [n][2560] HBM
    buffer (zero copy), or first staged into HBM and summed there.  Main
    stream: a [32768 x 2560] @ [2560 x 2560] bf16 GEMM stand-in for the first
    decoder block, repeated; it then waits on the side stream's event and
    runs the gate and residual add.  Reports the gather's PCIe rate alone, the
    GEMMs alone, both overlapped, and the exposed time (overlapped - GEMMs)."""
    import numpy as np
    import torch

    import hashed_gram_embedding_ngram_amd as ng
    import synth
    from synth.workloads import CONFIGS, DeviceInputs, HostInputs, fill_host_table

    dev = torch.device("cuda:0")
    spec = CONFIGS["host"].replace(dist=args.dist)
    n, d, R = spec.n, spec.d, spec.R
    t0 = time.time()
    hb = ng.HostBuffer(R * d * 2)
    fill_host_table(spec, hb.numpy(np.int16, (R, d)))
    T_host = ng.Table(hb, R, d)
    h = HostInputs(spec)
    di = DeviceInputs(spec, h, table=False)
    eN = torch.empty((n, d), dtype=torch.float32, device=dev)
    rows = torch.empty((n, 16), dtype=torch.int32, device=dev)
    out = torch.empty(n * d, dtype=torch.int16, device=dev)
    stage = remap = pool = None
    if args.host_mode in ("staged", "async"):
        stage = torch.empty((n * 16, d), dtype=torch.int16, device=dev)
        remap = torch.empty((n, 16), dtype=torch.int32, device=dev)
        n_staged = torch.zeros(1, dtype=torch.int64, device=dev)
        gws = ng.gather_host_workspace(n, d, dev)
        pinned = ng.gather_host_pinned(n) if args.host_mode == "async" else None
        gmode = ng.GATHER_ASYNC_COPY if args.host_mode == "async" else ng.GATHER_ZERO_COPY
    cache_info = None
    if args.host_mode == "pool":
        # Row frequencies of earlier batches choose the cached rows.
        counts = None
        for b in range(1, args.cache_history + 1):
            hb_in = HostInputs(spec.replace(batch=b))
            r_b = ng.ngram_hash(torch.from_numpy(hb_in.tokens).to(dev), torch.from_numpy(hb_in.offsets).to(dev), R)
            counts = ng.ngram_count_rows(r_b, R, counts=counts, accumulate=counts is not None)
        pool = ng.RowPool(T_host, args.cache_rows + 16 * n)
        hot, selected = ng.ngram_select_hot_rows(counts, args.cache_rows)
        tc = time.time()
        ng.ngram_pool_cache_rows(pool, hot, selected)
        torch.cuda.synchronize()
        cache_info = {"cache_rows": selected, "cache_gib": selected * d * 2 / 2**30,
                      "history_batches": args.cache_history, "fill_s": time.time() - tc}
        pool_T = pool.device_table()
        prow = torch.empty((n, 16), dtype=torch.int32, device=dev)
        fetched = torch.zeros(1, dtype=torch.int64, device=dev)
        pws = ng.pool_workspace(n, dev)
    A = torch.randn((32768, d), dtype=torch.bfloat16, device=dev)
    B = torch.randn((d, d), dtype=torch.bfloat16, device=dev).contiguous()
    C = torch.empty((32768, d), dtype=torch.bfloat16, device=dev)
    cu_total = None
    if args.cu_split > 0:
        side, main, cu_total = cu_masked_streams(args.cu_split)
        torch.cuda.set_stream(main)
    else:
        side = torch.cuda.Stream(device=dev)        # default priority
        main = torch.cuda.current_stream()
    setup_s = time.time() - t0

    def gather(stream):
        ng.ngram_hash(di.tokens, di.offsets, R, rows_out=rows, stream=stream)
        if args.host_mode in ("staged", "async"):
            ng.ngram_gather_host(T_host, rows, stage, remap, n_staged_out=n_staged, mode=gmode, workspace=gws,
                                 pinned=pinned, stream=stream)
            ng.ngram_embed_bag(ng.Table(stage, n * 16, d), remap, eN_out=eN, stream=stream)
        elif args.host_mode == "pool":
            ng.ngram_pool_gather(pool, rows, pool_rows_out=prow, fetched_out=fetched, workspace=pws, stream=stream)
            ng.ngram_embed_bag(pool_T, prow, eN_out=eN, stream=stream)
        else:
            ng.ngram_embed_bag(T_host, rows, eN_out=eN, stream=stream,
                               launch=(0, args.host_wgs) if args.host_wgs else None)

    def gemms(k):
        for _ in range(k):
            torch.matmul(A, B, out=C)

    def timed(fn, reps):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps

    # the gather alone (side stream), with events on that stream
    gather(side)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s_, e_ in ev:
        s_.record(side)
        gather(side)
        e_.record(side)
    torch.cuda.synchronize()
    gather_s = sum(a.elapsed_time(b) for a, b in ev) / len(ev) / 1e3
    # PCIe reference: one pinned H2D copy of 1 GiB
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    h2d_s = timed(lambda: dst.copy_(src, non_blocking=True), 3)
    del src, dst
    # GEMMs alone; enough of them to outlast the gather (after a warm-up call
    # that absorbs the GEMM library's first-call setup)
    gemms(3)
    torch.cuda.synchronize()
    gemm1 = timed(lambda: gemms(1), 5)
    k = max(1, int(np.ceil(1.25 * gather_s / gemm1)))
    gemm_s = timed(lambda: gemms(k), 3)

    def overlapped():
        # the GEMMs are enqueued first: the async-copy mode waits on the host
        # for the side stream's dedup before it enqueues its copies
        side.wait_stream(main)
        gemms(k)
        gather(side)
        ev_done = torch.cuda.Event()
        ev_done.record(side)
        main.wait_event(ev_done)
        ng.ngram_gate_add(eN, di.tokens, di.W_g, out, e1=di.e1, residual=di.residual, stream=main)
    both_s = timed(overlapped, 3)
    gate_s = timed(lambda: ng.ngram_gate_add(eN, di.tokens, di.W_g, out, e1=di.e1,
                                             residual=di.residual, stream=main), 5)

    interference = None
    if args.interference:
        # The GEMM stand-in's time per call beside each reader of pinned host
        # memory running on the side stream for the whole GEMM loop: the
        # random-row gather (the path), the same kernel over consecutive rows
        # (the same bytes and grid, sequential addresses), and a DMA copy of
        # the same bytes (no compute units, PCIe traffic only).
        seq_rows = torch.arange(n * 16, dtype=torch.int32, device=dev).reshape(n, 16)
        eN2 = torch.empty_like(eN)
        pinned_src = torch.empty(n * 16 * d * 2, dtype=torch.uint8, pin_memory=True)
        dma_dst = torch.empty(n * 16 * d * 2, dtype=torch.uint8, device=dev)
        readers = {
            "random_row_gather": lambda st: ng.ngram_embed_bag(T_host, rows, eN_out=eN, stream=st),
            "consecutive_row_gather": lambda st: ng.ngram_embed_bag(T_host, seq_rows, eN_out=eN2, stream=st),
            "dma_copy": lambda st: dma_dst.copy_(pinned_src, non_blocking=True),
        }
        ng.ngram_hash(di.tokens, di.offsets, R, rows_out=rows, stream=side)
        interference = {"gemm_alone_ms_per_call": gemm1 * 1e3, "bytes_per_reader_call": n * 16 * d * 2}
        for name, fn in readers.items():
            with torch.cuda.stream(side):
                fn(side)                                            # warm-up
            torch.cuda.synchronize()
            ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev0[0].record(side)
            with torch.cuda.stream(side):
                fn(side)
            ev0[1].record(side)
            torch.cuda.synchronize()
            reader_s = ev0[0].elapsed_time(ev0[1]) / 1e3
            reps = max(1, int(np.ceil(1.5 * k * gemm1 / reader_s)))
            side.wait_stream(main)
            with torch.cuda.stream(side):
                for _ in range(reps):
                    fn(side)
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(main)
            gemms(k)
            g1.record(main)
            torch.cuda.synchronize()
            interference[name] = {"reader_alone_ms": reader_s * 1e3,
                                  "reader_GBps": n * 16 * d * 2 / reader_s / 1e9,
                                  "gemm_beside_ms_per_call": g0.elapsed_time(g1) / k}
        del pinned_src, dma_dst

    # The bytes that cross PCIe: all 16 rows per token (zero copy), the
    # distinct rows (staged, async), or the distinct uncached rows (pool).
    pcie_bytes = nominal_pcie = n * 16 * d * 2
    staged_info = None
    if stage is not None:
        torch.cuda.synchronize()
        U = int(n_staged.item())
        pcie_bytes = U * d * 2
        staged_info = {"distinct_rows": U, "pcie_bytes_per_batch": pcie_bytes,
                       "nominal_GBps": nominal_pcie / gather_s / 1e9,
                       "engine": "DMA (one copy per distinct row)" if args.host_mode == "async"
                       else "GPU workgroups (zero copy, capped grid)"}
    if cache_info is not None:
        torch.cuda.synchronize()
        cache_info["rows_fetched_per_batch"] = int(fetched.item())
        cache_info["pcie_bytes_per_batch"] = int(fetched.item()) * d * 2
        cache_info["nominal_GBps"] = nominal_pcie / gather_s / 1e9
        pcie_bytes = cache_info["pcie_bytes_per_batch"]
    achieved = pcie_bytes / gather_s / 1e9
    result = {
        "metric": METRIC,
        "value": n / gather_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 1,
        "ms_per_step": gather_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "host", "tokens": n, "R": R, "d": d, "K": K_ROWS, "table_dtype": "bf16",
                   "table_location": "pinned host memory", "mode": args.host_mode,
                   "cu_split": None if not args.cu_split else f"gather {args.cu_split} CUs, GEMM {cu_total - args.cu_split}",
                   "host_workgroups": args.host_wgs or 8,
                   "token_dist": f"zipf({spec.zipf_s})" if args.dist == "zipf" else "uniform"},
        "roofline": {"bound": "pcie", "achieved": achieved, "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / PCIE_PEAK_GBPS, "traffic": None,
                     "kernel": {"zero_copy": "ngram_bag_kernel (host table)", "staged": "pool_fetch_kernel (staging)",
                                "async": "host-to-device copies", "pool": "pool_fetch_kernel"}[args.host_mode],
                     "algorithmic_bytes_per_launch": pcie_bytes,
                     "h2d_copy_GBps": (1 << 30) / h2d_s / 1e9},
        "overlap": {"gemm_stand_in": "[32768 x 2560] @ [2560 x 2560] bf16", "gemm_count": k,
                    "gemm_alone_ms": gemm_s * 1e3, "gather_alone_ms": gather_s * 1e3,
                    "overlapped_ms": both_s * 1e3, "exposed_ms": (both_s - gemm_s) * 1e3,
                    "gate_add_ms": gate_s * 1e3,
                    "dma_estimate_ms": dma_time_estimate_us(K_ROWS, d, 2, PCIE_PEAK_GBPS) * n / 1e3},
        "row_pool": cache_info,
        "staged": staged_info,
        "interference": interference,
        "setup_s": setup_s,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res_np = di.residual.cpu().numpy().view(np.uint16).reshape(n, d)
        e1_np = di.e1.cpu().numpy().view(np.uint16).reshape(spec.V, d)
        result["cpu_baseline"] = cpu_baseline(h, hb.numpy(np.uint16, (R, d)), None, e1_np, res_np, R, 0.0,
                                              f"the full {R * d * 2 / 2**30:.2f} GiB table, read in place in "
                                              "pinned host memory")
    print(json.dumps(result), flush=True)
    hb.free()


if __name__ == "__main__":
    main()
