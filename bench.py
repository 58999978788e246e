"""Benchmark of the per-layer GNN message-passing hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

Default workload (config 3): one GAT layer forward + backward, binary32,
4 heads x 64, input width 256, on an R-MAT graph (a=0.57, b=c=0.19) with
2^21 nodes, average degree 20, directed, with self-loops: H' = XW, the
per-head scores, SDDMM-add + LeakyReLU(0.2) + edge softmax, the weighted
aggregation, and the backward (SDDMM dot, softmax backward, edge sums, the
transposed aggregation, dW, dX) for a seeded upstream gradient, with every
input resident in HBM.

Printed value: GEdge·feat/s = (edge x feature products of the step's
aggregation-shaped passes) / step time; for the GAT layer the weighted
aggregation, the SDDMM dot and the transposed aggregation (3 nnz h d_head).
Beside it:
  * roofline: the dominant kernel of the step (GAT: the backward's pass over
    the out-edges; GCN and the quantised exchange: the 256-wide aggregation),
    algorithmic bytes per launch / its average duration, timed with HIP events
    on its own stream over the timed steps; `traffic` from the committed
    rocprofv3 counter summary of the same kernel, when that summary was taken
    on the current sources;
  * kernels_measured: every instrumented kernel of a few further steps, with
    its byte (or flop) model and fraction of the HBM (or matrix-core) peak;
  * cpu_baseline: the CPU oracle on a bounded sample of the same workload.

Other configs (--config): 2 = 3-layer GCN, binary32, R-MAT 2^20 (128 -> 256
-> 256 -> 41, softmax cross-entropy); 4 = the 3-layer GCN with bf16 feature
storage on a 2.45M-node Chung-Lu graph (100 -> 256 -> 256 -> 47); 5 = one
partition's quantised exchange (30% marginal rows of a 2^20-node R-MAT graph,
256 wide) followed by the aggregation.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0


def source_digest():
    """sha1 over every library source and the build script (compiler flags):
    a counter summary taken on other sources no longer describes the kernel."""
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "sparse_message_passing_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    files += [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))]
    files.append(os.path.join(ROOT, "sparse_message_passing_amd", "build.py"))
    for p in files:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, key):
    """HBM bytes per launch of kernel `key` on `workload`, read from the
    committed rocprofv3 counter summary profiles/<workload>_hbm_counters.md;
    None when there is none or it was taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.md")
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    sha = re.search(r"^- source sha1: ([0-9a-f]{40})$", text, re.M)
    hit = re.search(r"^- traffic bytes per launch \[" + re.escape(key) + r"\]: (\d+)$", text, re.M)
    if sha is None or hit is None or sha.group(1) != source_digest():
        return None
    return int(hit.group(1))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--cpu-sample-edges", type=int, default=2_000_000)
    ap.add_argument("--calibrate", action="store_true",
                    help="run only the reference kernels of known traffic and flops and print their rates")
    return ap.parse_args()


def calibrate(reps=5):
    """Achievable peaks of this GPU from reference kernels of known bytes and
    flops (sparse_message_passing_amd/calib/calib.hip): a streaming read and
    a copy of 1 GiB, random row gathers from tables that fit the L2 of one
    XCD (2 MiB), the memory-side cache (32-128 MiB) or neither (1-2 GiB), and
    matrix-core loops in f32, bf16 and i8.  Under rocprofv3 --pmc the same
    launches give the counter reading per byte moved."""
    import ctypes as C
    import torch
    from sparse_message_passing_amd import build as hb
    L = C.CDLL(hb.CALIB_LIB)
    P, I64 = C.c_void_p, C.c_int64
    L.gnn_calib_read.argtypes = [P, I64, P, I64, P]
    L.gnn_calib_copy.argtypes = [P, P, I64, P]
    L.gnn_calib_gather.argtypes = [P, I64, P, I64, P, I64, P]
    L.gnn_calib_mfma.argtypes = [C.c_int, I64, C.c_int, P, P, P]
    for f in (L.gnn_calib_read, L.gnn_calib_copy, L.gnn_calib_gather, L.gnn_calib_mfma):
        f.restype = C.c_int
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    sp = stream.cuda_stream

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"calibration launch failed ({rc})")

    out = {}
    GiB = 1 << 30
    with torch.cuda.stream(stream):
        src = torch.ones(GiB // 4, device=dev)
        dst = torch.empty_like(src)
        red = torch.empty(4096, device=dev)
        t = event_time(lambda: ok(L.gnn_calib_read(src.data_ptr(), GiB, red.data_ptr(), 4096, sp)), reps, stream)
        out["read_1GiB"] = {"ms": round(t, 4), "GBs": round(GiB / (t * 1e-3) / 1e9, 1), "bytes_read": GiB}
        t = event_time(lambda: ok(L.gnn_calib_copy(src.data_ptr(), dst.data_ptr(), GiB, sp)), reps, stream)
        out["copy_1GiB"] = {"ms": round(t, 4), "GBs": round(2 * GiB / (t * 1e-3) / 1e9, 1), "bytes_read": GiB,
                            "bytes_written": GiB}
        del dst
        blocks = 256 * 16
        gout = torch.empty(blocks * 256, device=dev)
        n_idx = 1 << 23
        r = np.random.default_rng(12345)
        gath = {}
        for tab in (2 << 20, 32 << 20, 128 << 20, GiB, 2 * GiB):
            table = src if tab <= GiB else torch.ones(tab // 4, device=dev)
            for rb in (128, 256, 1024):
                rows = tab // rb
                idx = torch.from_numpy(r.integers(0, rows, n_idx, dtype=np.int32)).to(dev)
                t = event_time(lambda: ok(L.gnn_calib_gather(table.data_ptr(), rb, idx.data_ptr(), n_idx,
                                                             gout.data_ptr(), blocks, sp)), reps, stream)
                gath[f"table{tab >> 20}MiB_row{rb}B"] = {"ms": round(t, 4),
                                                          "gathered_GBs": round(n_idx * rb / (t * 1e-3) / 1e9, 1)}
            del table
        out["gather_uniform_8M_rows"] = gath
        mf = torch.empty(256 * 8 * 256, device=dev)
        work = C.c_double()
        for kind, name, iters in ((0, "mfma_f32_16x16x4", 4000), (1, "mfma_bf16_16x16x32", 2000),
                                  (2, "mfma_i8_16x16x64", 2000)):
            t = event_time(lambda: ok(L.gnn_calib_mfma(kind, 256 * 8, iters, mf.data_ptr(), C.byref(work), sp)),
                           reps, stream)
            out[name] = {"ms": round(t, 4), "TFLOPs": round(work.value / (t * 1e-3) / 1e12, 1)}
    torch.cuda.synchronize()
    return out


def event_time(fn, reps, stream):
    """Average duration (ms) of fn() over reps launches, HIP events on `stream`."""
    import torch
    with torch.cuda.stream(stream):
        fn()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(reps):
            fn()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


# ---------------------------------------------------------------------------
# algorithmic work per launch of each instrumented kernel (bytes each array
# must move at least once, or flops); n nodes, nnz edges incl. self-loops
# ---------------------------------------------------------------------------
def spmm_compulsory_bytes(n, nnz, d, s_in=4, s_out=4, edge_weights=True, heads=1):
    """row_ptr (int64) + col (int32) + the edge weights (one f32 per edge and
    head as stored, else dinv, one f32 per node) + each input row once + each
    output row once + the degree order (int32 per row)."""
    w = 4 * nnz * heads if edge_weights else 4 * n
    return 8 * (n + 1) + 4 * nnz + w + s_in * n * d + s_out * n * d + 4 * n


def gat_bwd_csc_bytes(n, nnz, h, dh):
    """Per head slab: col_ptr, destination ids, the order, the H' and dY
    slices read once, dH' slice written once, dS written (S is formed from
    the H' row), the 12-byte per-destination records, the dE plane written."""
    return h * (8 * (n + 1) + 8 * nnz + 12 * n * dh + 20 * n)


def gat_fwd_bytes(n, nnz, h, dh):
    """Per head slab: row_ptr, source ids, the order, the H' slice read once,
    D, the Y slice written once, the softmax maximum and 1/sum written."""
    return h * (8 * (n + 1) + 4 * nnz + 8 * n * dh + 20 * n)


def kernel_model(key, n, nnz, ctx):
    """(kind, amount) for an instrumented key: ("bytes", B) or ("flops", F, bytes);
    None when the key has no model here."""
    kv = dict(re.findall(r"(\w+)=(\S+)", key))
    name = key.split()[0]
    size = lambda t: 2 if t == "bf16" else 4
    if name == "spmm_kernel":
        m = re.search(r"(\w+)->(\w+)", key)
        d, h = int(kv["d"]), int(kv["h"])
        return ("bytes", spmm_compulsory_bytes(n, nnz, d, size(m.group(1)), size(m.group(2)), heads=h))
    if name == "gat_fwd_kernel":
        return ("bytes", gat_fwd_bytes(n, nnz, int(kv["h"]), int(kv["dh"])))
    if name == "gat_bwd_csc_kernel":
        return ("bytes", gat_bwd_csc_bytes(n, nnz, int(kv["h"]), int(kv["dh"])))
    if name == "gat_in_sum_kernel":
        h, dh = int(kv["h"]), int(kv["dh"])
        return ("bytes", 8 * (n + 1) + 4 * nnz + 4 * nnz * h + 4 * n * h + 4 * n)
    if name == "sddmm_dot_kernel":
        h, dh = int(kv["h"]), int(kv["dh"])
        s = size(key.split()[-1])
        return ("bytes", 8 * (n + 1) + 4 * nnz + 2 * s * n * h * dh + 4 * nnz * h)
    if name == "softmax_fwd_kernel":
        return ("bytes", 8 * (n + 1) + 8 * nnz * int(kv["h"]))
    if name in ("quantize_kernel", "dequantize_kernel"):
        b, d = int(kv["b"]), int(kv["d"])
        m = ctx.get("quant_rows", {}).get(b)
        if m is None:
            return None
        return ("bytes", 4 * m * d + m * d * b // 8 + 8 * m + 4 * m)
    if name == "gemm":
        M, N, K = int(kv["M"]), int(kv["N"]), int(kv["K"])
        ab = re.search(r"(\w+),(\w+)->(\w+)", key)
        sa, sb, sc = (size(ab.group(i)) for i in (1, 2, 3))
        return ("flops", 2 * M * N * K, sa * M * K + sb * K * N + sc * M * N, ab.group(1), ab.group(2))
    return None


def kernel_table(gnnmp, keys, n, nnz, ctx):
    out = {}
    for key in keys:
        cnt, tot = gnnmp.gnn_timer_result(key)
        if cnt == 0:
            continue
        ms = tot / cnt
        rec = {"launches": cnt, "ms_per_launch": round(ms, 4)}
        m = kernel_model(key, n, nnz, ctx)
        if m and m[0] == "bytes":
            gbs = m[1] / (ms * 1e-3) / 1e9
            rec.update(bound="hbm", bytes_per_launch=m[1], achieved_GBs=round(gbs, 1),
                       frac=round(gbs / HBM_PEAK_GBS, 4))
        elif m and m[0] == "flops":
            flops, byts, ta, tb = m[1], m[2], m[3], m[4]
            peak = BF16_MFMA_PEAK_TFLOPS if (ta == "bf16" and tb == "bf16") else FP32_MFMA_PEAK_TFLOPS
            tf = flops / (ms * 1e-3) / 1e12
            ceiling = min(peak, flops / byts * HBM_PEAK_GBS / 1e3)  # TFLOP/s the HBM roofline allows
            rec.update(bound="mfma" if ceiling >= peak else "hbm", tflops=round(tf, 2), peak_tflops=peak,
                       frac_of_peak=round(tf / peak, 4), ceiling_tflops=round(ceiling, 1),
                       frac_of_ceiling=round(tf / ceiling, 4))
        out[key] = rec
    return out


# ---------------------------------------------------------------------------
# CPU oracle baselines
# ---------------------------------------------------------------------------
def oracle_graph(k):
    from oracle.graph import build_graph
    from sparse_message_passing_amd import synth
    inp = synth.workload_inputs(k)
    return build_graph(inp["src"], inp["dst"], int(inp["n"]), synth.WORKLOADS[k]["symmetric"]), inp


def oracle_threads():
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline_gcn_full(og, inp, work_per_pass, min_seconds=10.0, max_passes=3):
    """The oracle's 3-layer forward+backward on the whole workload, repeated
    until at least `min_seconds` of CPU work (at most `max_passes` passes)."""
    import oracle
    Ws = [inp["W0"], inp["W1"], inp["W2"]]
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        oracle.gcn_forward_backward(og, inp["X"], Ws, inp["labels"])
        dt += time.perf_counter() - t0
        passes += 1
    return dict(value=round(passes * work_per_pass / dt / 1e9, 4), unit="GEdge·feat/s", cores=oracle_threads(),
                kind="oracle", sample=f"{passes} full 3-layer forward+backward pass(es) of the same workload "
                                      f"({og.n} nodes, nnz {og.nnz}), {dt:.2f} s")


def sample_graph(og, edges):
    """A bounded sample of the workload's graph: the destination rows from
    0.7071 n on (R-MAT gives ids with few one bits its hubs, so that start has
    a typical mix) holding about `edges` in-edges, with every source of those
    edges, relabelled compactly (ascending ids keep every row's order); the
    sources outside the rows get their self-loop, so every node has a row.
    Returns (oracle graph, original ids of its nodes)."""
    import oracle
    r0 = int(og.n * 0.7071)
    e0 = int(og.row_ptr[r0])
    r1 = int(np.searchsorted(og.row_ptr, e0 + edges))
    r1 = max(r0 + 1, min(r1, og.n))
    e1 = int(og.row_ptr[r1])
    col, dst = og.col[e0:e1].astype(np.int64), og.dst[e0:e1].astype(np.int64)
    T = np.unique(np.concatenate([np.arange(r0, r1), col]))
    extra = np.setdiff1d(T, np.arange(r0, r1))
    col = np.concatenate([col, extra])
    dst = np.concatenate([dst, extra])
    key = np.searchsorted(T, dst) * T.size + np.searchsorted(T, col)
    key.sort()
    nd, nc = (key // T.size).astype(np.int32), (key % T.size).astype(np.int32)
    rp = np.zeros(T.size + 1, np.int64)
    rp[1:] = np.cumsum(np.bincount(nd, minlength=T.size))
    return oracle.OracleGraph(int(T.size), rp, nc, nd), T


EDGE_OPS = ("spmm", "sddmm_add", "sddmm_dot", "edge_softmax", "edge_softmax_bwd", "edge_reduce")


def cpu_baseline_sampled(k, og, inp, work, edges):
    """The oracle's own step (the same functions the parity tests check) run on
    a bounded sample of the workload (sample_graph), with the time of its
    per-edge calls (aggregations, SDDMM, edge softmax and its backward, edge
    sums) and of the rest (dense products, scores, quantisation, loss, store
    rounding: per-node work) kept apart; each part is scaled to the whole
    workload (edges: nnz / sample nnz; the rest: n / sample nodes) and the
    step work is divided by the scaled time."""
    import oracle
    from sparse_message_passing_amd import synth
    cfg = synth.WORKLOADS[k]
    sg, T = sample_graph(og, edges)
    spent = {"edge": 0.0}
    saved = {name: getattr(oracle, name) for name in EDGE_OPS}

    def timed(fn):
        def w(*a, **kw):
            t0 = time.perf_counter()
            try:
                return fn(*a, **kw)
            finally:
                spent["edge"] += time.perf_counter() - t0
        return w

    for name, fn in saved.items():
        setattr(oracle, name, timed(fn))
    try:
        t0 = time.perf_counter()
        if cfg["kind"] == "gat":
            X = inp["X"][T]
            fw = oracle.gat_layer_fwd(sg, X, inp["W"], inp["a_src"], inp["a_dst"], cfg["heads"], cfg["slope"])
            oracle.gat_layer_bwd(sg, fw, X, inp["W"], inp["a_src"], inp["a_dst"], inp["dY"][T], cfg["heads"],
                                 cfg["slope"])
        elif cfg["kind"] == "gcn":
            Ws = [inp[f"W{i}"] for i in range(len(cfg["widths"]) - 1)]
            oracle.gcn_forward_backward(sg, inp["X"][T], Ws, inp["labels"][T], dt=cfg.get("dtype", "f32"))
        else:
            sel = np.isin(T, inp["rows"])
            rows = np.nonzero(sel)[0].astype(np.int32)
            bits = inp["mixed_bits"][np.searchsorted(inp["rows"], T[sel])]
            Hmix, _, _ = oracle.quantized_aggregate(sg, inp["H"][T], rows, bits, int(inp["philox_seed"]))
        total = time.perf_counter() - t0
    finally:
        for name, fn in saved.items():
            setattr(oracle, name, fn)
    t_edge = spent["edge"]
    t_node = total - t_edge
    est = t_edge * og.nnz / sg.nnz + t_node * og.n / sg.n
    return dict(value=round(work / est / 1e9, 4), unit="GEdge·feat/s", cores=oracle_threads(), kind="oracle",
                sample=f"the oracle's whole step on {sg.n} of {og.n} nodes and {sg.nnz} of {og.nnz} edges "
                       f"(the in-edges of destinations {int(og.n * 0.7071)}.. with their sources, relabelled): "
                       f"{t_edge:.2f} s in per-edge calls scaled by {og.nnz / sg.nnz:.1f}, {t_node:.2f} s in "
                       f"per-node work scaled by {og.n / sg.n:.2f}: {est:.1f} s estimated for the whole step")


def cpu_oracle_kernels(k, og, inp, edges=1_000_000):
    """The oracle's own steps timed on one host thread and on all of them, on
    a bounded row sample: the 256-wide aggregation (GCN workloads), the SDDMM
    dot and the edge softmax (GAT), the quantiser over the marginal rows
    (quantised exchange).  Rates in the bench's units."""
    import oracle
    from sparse_message_passing_amd import synth
    allt = oracle_threads()
    cfg = synth.WORKLOADS[k]
    out = {"threads_all": allt}
    jobs = []
    sub, T = sample_graph(og, edges)
    if cfg["kind"] in ("gcn", "quant"):
        X = np.random.default_rng(77).standard_normal((sub.n, 256))
        w = sub.gcn_norm()[1].astype(np.float64)
        jobs.append(("spmm_d256_gedge_feat_s", lambda: oracle.spmm(sub, X, w), sub.nnz * 256,
                     f"{sub.n} nodes, {sub.nnz} edges"))
    if cfg["kind"] == "gat":
        A = np.random.default_rng(78).standard_normal((sub.n, 256))
        B = np.random.default_rng(79).standard_normal((sub.n, 256))
        E = np.random.default_rng(80).standard_normal((sub.nnz, 4))
        jobs.append(("sddmm_dot_gedge_feat_s", lambda: oracle.sddmm_dot(sub, A, B, 4), sub.nnz * 256,
                     f"{sub.n} nodes, {sub.nnz} edges, 4 heads x 64"))
        jobs.append(("edge_softmax_gedge_s", lambda: oracle.edge_softmax(sub, E), sub.nnz, f"{sub.nnz} edges, 4 heads"))
        Hq = np.random.default_rng(81).standard_normal((60_000, 256)).astype(np.float32)
        rq = np.arange(60_000, dtype=np.int32)
        jobs.append(("quantize_8bit_rows_per_s", lambda: oracle.quantize(Hq, rq, 8, 1), rq.size,
                     f"{rq.size} rows x 256 at 8 bits"))
    if cfg["kind"] == "quant":
        H = inp["H"]
        rows = inp["rows"].astype(np.int32)
        jobs.append(("quantize_8bit_rows_per_s", lambda: oracle.quantize(H, rows, 8, 1), rows.size,
                     f"{rows.size} rows x 256 at 8 bits"))
    for name, fn, work, what in jobs:
        rec = {"sample": what}
        for label, th in (("one_thread", 1), ("all_threads", allt)):
            prev = oracle.set_threads(th)
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
            oracle.set_threads(prev)
            rec[label] = round(work / dt / 1e9, 4) if "gedge" in name else round(work / dt, 1)
        out[name] = rec
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported (sharding is a design note, "
              "not a measured path)", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_message_passing_amd import gnnmp, synth
    from sparse_message_passing_amd.step import GatLayer, GcnStack, OverlapExchange, QuantExchange

    if a.calibrate:
        print(json.dumps({"calibration": calibrate()}), flush=True)
        return

    if not os.path.exists(gnnmp.LIB_PATH):
        from sparse_message_passing_amd import build as hb
        hb.build(verbose=False)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()
    cfg = synth.WORKLOADS[a.config]
    t0 = time.time()
    inp = synth.workload_inputs(a.config)
    n = int(inp["n"])
    print(f"# inputs ready ({time.time() - t0:.1f} s)", file=sys.stderr, flush=True)
    t0 = time.time()
    g = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=cfg["symmetric"], csc=cfg["kind"] == "gat")
    print(f"# graph built: n={g.n} nnz={g.nnz} max_in_degree={g.max_in_degree} ({time.time() - t0:.1f} s)",
          file=sys.stderr, flush=True)
    T = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    extra = {}
    ctx = {}
    with torch.cuda.stream(stream):
        if cfg["kind"] == "gcn":
            Ws = [T(inp[f"W{i}"]) for i in range(3)]
            runner = GcnStack(g, T(inp["X"]), Ws, T(inp["labels"]), dtype=cfg.get("dtype", "f32"))
            metric_work = runner.spmm_edge_feats()
            sdt = "bf16" if cfg.get("dtype") == "bf16" else "f32"
            dom_key = f"spmm_kernel d=256 h=1 {sdt}->{sdt} csr"
            es = 2 if sdt == "bf16" else 4
            dom_bytes = spmm_compulsory_bytes(g.n, g.nnz, 256, es, es)
        elif cfg["kind"] == "gat":
            h, dh = cfg["heads"], cfg["d_head"]
            runner = GatLayer(g, T(inp["X"]), T(inp["W"]), T(inp["a_src"]), T(inp["a_dst"]), h, dh, cfg["slope"],
                              T(inp["dY"]))
            metric_work = g.nnz * h * dh * 3  # weighted SpMM, SDDMM dot, transposed SpMM
            dom_key = f"gat_bwd_csc_kernel h={h} dh={dh}"
            dom_bytes = gat_bwd_csc_bytes(g.n, g.nnz, h, dh)
        else:
            runner = QuantExchange(g, T(inp["H"]), inp["rows"], inp["mixed_bits"], int(inp["philox_seed"]))
            metric_work = g.nnz * cfg["d"]
            dom_key = "spmm_kernel d=256 h=1 f32->f32 csr"
            dom_bytes = spmm_compulsory_bytes(g.n, g.nnz, 256)
            ctx["quant_rows"] = {bb: int(r.numel()) for bb, r, _, _, _ in runner.groups}
    # a plain 1 GiB device copy: the reference that scales the HBM byte
    # counters (FETCH_SIZE / WRITE_SIZE) when this command runs under rocprofv3
    with torch.cuda.stream(stream):
        cal_src = torch.empty(256 << 20, dtype=torch.float32, device=dev)
        cal_dst = torch.empty_like(cal_src)
        cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst
    for _ in range(a.warmup):
        with torch.cuda.stream(stream):
            runner.step()
    torch.cuda.synchronize()

    # ---- timed region: the steps, with the dominant kernel's launches
    # bracketed by HIP events on the stream they run on -------------------
    gnnmp.gnn_timer_start(dom_key, capacity=max(64, 8 * a.steps))
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(a.steps):
            runner.step()
        end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    gnnmp.gnn_timer_stop()
    ms = start.elapsed_time(end) / a.steps
    print(f"# timed {a.steps} steps: {ms:.3f} ms/step (wall {wall:.2f} s)", file=sys.stderr, flush=True)
    value = metric_work / (ms * 1e-3) / 1e9
    launches, dom_total = gnnmp.gnn_timer_result(dom_key)
    if launches == 0:
        raise RuntimeError(f"the dominant kernel {dom_key!r} was not launched in the timed steps")
    dom_ms = dom_total / launches
    ach = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg["name"], dom_key)
    roofline = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic)
    extra["dominant_kernel"] = {"key": dom_key, "launches_timed": launches, "ms_per_launch": round(dom_ms, 4),
                                "algorithmic_bytes_per_launch": dom_bytes,
                                "edge_feat_per_s": None}
    if traffic:
        extra["dominant_kernel"]["counter_GBs"] = round(traffic / (dom_ms * 1e-3) / 1e9, 1)
        extra["dominant_kernel"]["traffic_amplification"] = round(traffic / dom_bytes, 2)
    hd = 256 if cfg["kind"] != "gat" else cfg["heads"] * cfg["d_head"]
    extra["dominant_kernel"]["edge_feat_per_s"] = round(g.nnz * hd / (dom_ms * 1e-3) / 1e9, 2)

    # ---- every instrumented kernel over a few more steps ---------------------
    gnnmp.gnn_timer_start(None, capacity=4096)
    with torch.cuda.stream(stream):
        for _ in range(3):
            runner.step()
    torch.cuda.synchronize()
    gnnmp.gnn_timer_stop()
    extra["kernels_measured"] = kernel_table(gnnmp, gnnmp.gnn_timer_keys(), g.n, g.nnz, ctx)
    gnnmp.gnn_timer_release()

    # ---- primitives of the path timed alone ----------------------------------
    if cfg["kind"] == "gcn":
        d = 256
        X = runner.H[1]                       # a 256-wide activation
        Y = torch.empty_like(X)
        ws = torch.empty(max(gnnmp.lib().gnn_spmm_workspace_size(g.h, 0, d), 1), dtype=torch.uint8, device=dev)
        extra["spmm_d256_alone_ms"] = round(event_time(lambda: gnnmp.gnn_spmm(g, X, Y, ws=ws), a.kernel_reps,
                                                       stream), 4)
        es = X.element_size()
        extra["spmm_d256_gather_model_bytes"] = 8 * (g.n + 1) + 8 * g.nnz + es * g.nnz * d + es * g.n * d
        Wt = runner.Ws[1]
        Z = torch.empty_like(X)
        # Tango's quantisation-aware variant of the 256 x 256 update (maxima,
        # stochastic 8-bit quantisation of both operands, int8 matrix cores)
        if X.dtype == torch.float32:
            qws = torch.empty(gnnmp.lib().gnn_gemm_q8_workspace_size(g.n, d, d), dtype=torch.uint8, device=dev)
            q8_ms = event_time(lambda: gnnmp.gnn_gemm_q8(X, Wt, Z, seed=5, ws=qws), a.kernel_reps, stream)
            extra["gemm_q8_256x256_ms"] = round(q8_ms, 4)
            extra["gemm_q8_256x256_tops_incl_quantise"] = round(2.0 * g.n * d * d / (q8_ms * 1e-3) / 1e12, 2)
        if a.config == 2:
            # GraphSAGE's mean aggregator on the same edges: the aggregation
            # alone and a 256 -> 256 layer forward + backward (the backward
            # runs the transposed mean operator over the CSC view)
            gs = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=True, csc=True)
            extra["sage_mean_spmm_d256_ms"] = round(event_time(
                lambda: gnnmp.gnn_spmm(gs, X, Y, weights="mean", ws=ws), a.kernel_reps, stream), 4)
            Ys = torch.empty_like(X)
            with torch.cuda.stream(stream):
                dYs = torch.randn_like(X)
            dXs = torch.empty_like(X)
            dWs = torch.empty((d, d), device=dev)
            extra["sage_layer_fwd_ms"] = round(event_time(
                lambda: gnnmp.gnn_sage_layer_fwd(gs, X, Wt, Ys, True), a.kernel_reps, stream), 4)
            extra["sage_layer_bwd_ms"] = round(event_time(
                lambda: gnnmp.gnn_sage_layer_bwd(gs, X, Wt, Ys, dYs, True, dWs, dX=dXs), a.kernel_reps, stream), 4)
            del Ys, dYs, dXs, gs
    if cfg["kind"] == "gat":
        # the SDDMM dot (f32) as a primitive, Tango's variant on 8-bit codes
        # (maxima + quantisation of both operands + the gather of 1-byte
        # codes), and the SDDMM add + edge softmax primitives, on the layer's
        # own H', S, D and dY
        h, dh = cfg["heads"], cfg["d_head"]
        Hp, S, D = gnnmp.gat_saved_views(g, runner.saved, h, dh)[:3]
        dYs = runner.dY
        dal = torch.empty((g.nnz, h), device=dev)
        E = torch.empty((g.nnz, h), device=dev)
        extra["sddmm_dot_f32_ms"] = round(event_time(
            lambda: gnnmp.gnn_sddmm(g, "dot", Hp, dYs, h, dh, dal), a.kernel_reps, stream), 4)
        extra["sddmm_dot_f32_GBs"] = round(kernel_model(f"sddmm_dot_kernel h={h} dh={dh} f32", g.n, g.nnz, ctx)[1]
                                           / (extra["sddmm_dot_f32_ms"] * 1e-3) / 1e9, 1)
        sws = torch.empty(gnnmp.lib().gnn_sddmm_q8_workspace_size(g.h, h * dh), dtype=torch.uint8, device=dev)
        extra["sddmm_q8_ms"] = round(event_time(
            lambda: gnnmp.gnn_sddmm_q8(g, Hp, dYs, h, dh, dal, seed=5, ws=sws), a.kernel_reps, stream), 4)
        extra["sddmm_add_lrelu_ms"] = round(event_time(
            lambda: gnnmp.gnn_sddmm(g, "add", S, D, h, 1, E, slope=cfg["slope"]), a.kernel_reps, stream), 4)
        extra["edge_softmax_ms"] = round(event_time(
            lambda: gnnmp.gnn_edge_softmax(g, E, dal), a.kernel_reps, stream), 4)
        sm_bytes = kernel_model(f"softmax_fwd_kernel h={h}", g.n, g.nnz, ctx)[1]
        extra["edge_softmax_GBs"] = round(sm_bytes / (extra["edge_softmax_ms"] * 1e-3) / 1e9, 1)
        # the 8-bit stochastic quantiser (the exchange's message compression)
        # on every third row of the layer's H'
        qrows = torch.arange(0, g.n, 3, dtype=torch.int32, device=dev)
        m, dq = qrows.numel(), h * dh
        qp = torch.empty(m * dq, dtype=torch.uint8, device=dev)
        qs, qz = torch.empty(m, device=dev), torch.empty(m, device=dev)
        extra["quantize_8bit_ms"] = round(event_time(
            lambda: gnnmp.gnn_quantize(Hp, qrows, 8, 5, qp, qs, qz), a.kernel_reps, stream), 4)
        q_bytes = 4 * m * dq + m * dq + 8 * m + 4 * m
        extra["quantize_8bit_rows"] = m
        extra["quantize_8bit_GBs"] = round(q_bytes / (extra["quantize_8bit_ms"] * 1e-3) / 1e9, 1)
        extra["quantize_8bit_frac"] = round(q_bytes / (extra["quantize_8bit_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        extra["sddmm_dot_f32_frac"] = round(extra["sddmm_dot_f32_GBs"] / HBM_PEAK_GBS, 4)
        extra["edge_softmax_frac"] = round(extra["edge_softmax_GBs"] / HBM_PEAK_GBS, 4)
    if cfg["kind"] == "quant":
        # the same exchange with the dequantisation inside the gather, and the
        # backward exchange of the embedding gradients (also fused)
        with torch.cuda.stream(stream):
            fused = QuantExchange(g, T(inp["H"]), inp["rows"], inp["mixed_bits"], int(inp["philox_seed"]), fused=True)
            dY = torch.randn_like(fused.H)
        fused_ms = event_time(fused.step, a.kernel_reps, stream)
        bwd_ms = event_time(lambda: fused.backward(dY), a.kernel_reps, stream)
        extra["fused_step_ms"] = round(fused_ms, 4)
        extra["fused_step_gedge_feat_s"] = round(metric_work / (fused_ms * 1e-3) / 1e9, 2)
        extra["backward_exchange_ms"] = round(bwd_ms, 4)
        # adaptive bit-widths: statistics on the GPU, greedy assignment on the
        # host, at the average width of the uniform {2, 4, 8} draw
        from sparse_message_passing_amd.step import adaptive_bits
        rows_d = T(inp["rows"].astype(np.int32))
        beta_d = torch.empty(rows_d.numel(), device=dev)
        rng_d = torch.empty_like(beta_d)
        extra["quant_stats_ms"] = round(event_time(lambda: gnnmp.gnn_quant_stats(g, runner.H, rows_d, beta_d, rng_d),
                                                   a.kernel_reps, stream), 4)
        avg = float(inp["mixed_bits"].mean())
        t0 = time.perf_counter()
        bits_a, beta_h = adaptive_bits(g, runner.H, inp["rows"], avg)
        extra["assign_total_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
        var = lambda b: float(np.sum(beta_h.astype(np.float64) / (2.0 ** b - 1.0) ** 2))
        extra["variance_adaptive_over_uniform"] = round(var(bits_a) / var(inp["mixed_bits"]), 4)
        extra["adaptive_bits_histogram"] = {int(b): int((bits_a == b).sum()) for b in (2, 4, 8)}
        # the exchange split by message origin (local / remote in-edges) under
        # three schedules of the same kernels, and the stage timeline of each
        with torch.cuda.stream(stream):
            ov = OverlapExchange(g, T(inp["H"]), inp["rows"], inp["mixed_bits"], int(inp["philox_seed"]))
        for name, fn in (("sequential", ov.step_sequential), ("free", ov.step_free), ("staged", ov.step_staged)):
            extra[f"split_{name}_ms"] = round(event_time(fn, a.kernel_reps, stream), 4)
            torch.cuda.synchronize()
            extra[f"split_{name}_timeline_ms"] = ov.timeline()
    cpu = None
    if not a.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        og, oinp = oracle_graph(a.config)
        if a.config == 2:
            cpu = cpu_baseline_gcn_full(og, oinp, metric_work)
        else:
            cpu = cpu_baseline_sampled(a.config, og, oinp, metric_work, a.cpu_sample_edges)
        extra["cpu_oracle"] = cpu_oracle_kernels(a.config, og, oinp)
        print("# CPU oracle timed", file=sys.stderr, flush=True)
    out = {
        "metric": "GNN layer fwd+bwd GEdge·feat/s; SpMM/SDDMM HBM GB/s as % of peak",
        "value": round(value, 3),
        "unit": "GEdge·feat/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-storage/f32-accumulate" if cfg.get("dtype") == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "nodes": g.n, "nnz": g.nnz, "max_in_degree": g.max_in_degree,
                   "widths": cfg.get("widths"), "edge_feat_per_step": metric_work},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
