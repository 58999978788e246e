"""Benchmark of the per-layer GNN message-passing hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

Default workload (config 2): 3-layer GCN forward + backward, binary32,
R-MAT (a=0.57, b=c=0.19) with 2^20 nodes and average degree 16,
symmetrised with self-loops and GCN normalisation; widths 128 -> 256 -> 256
-> 41; mean softmax cross-entropy against random labels.  A step is one
forward pass, the loss, and the backward pass down to the first layer's
weight gradient, with every input resident in HBM.

Printed value: GEdge*feat/s = (sum over the step's aggregations of
nnz * width) / step time.  Beside it: the roofline of the dominant kernel
(the aggregation of the 256-wide layers, HBM-bound), timed with HIP events
on its own stream, and the CPU oracle timed on a bounded sample of the same
workload.

Other configs (timed the same way, for the record): 3 = one GAT layer
(4 heads x 64, R-MAT 2^21, directed) forward + backward; 4 = the 3-layer
GCN with bf16 feature storage on a 2.45M-node Chung-Lu graph (100 -> 256 ->
256 -> 47); 5 = one partition's quantised exchange (30% marginal rows of a
2^20-node R-MAT graph, 256 wide) followed by the aggregation.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gcn3_rmat20_hbm_counters.md")


def measured_traffic():
    """HBM bytes per launch of the 256-wide aggregation, read from the
    committed rocprofv3 counter summary; None when spmm.hip has changed
    since the counters were taken (the summary records the source's sha1)."""
    import hashlib
    import re
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
        nbytes = re.search(r"^- traffic bytes per launch: (\d+)$", text, re.M)
        sha = re.search(r"^- spmm\.hip sha1: ([0-9a-f]{40})$", text, re.M)
        src = os.path.join(ROOT, "sparse_message_passing_amd", "csrc", "spmm.hip")
        with open(src, "rb") as f:
            cur = hashlib.sha1(f.read()).hexdigest()
    except OSError:
        return None
    if nbytes is None or sha is None or sha.group(1) != cur:
        return None
    return int(nbytes.group(1))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    return ap.parse_args()


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


def spmm_compulsory_bytes(n, nnz, d, s_in=4, s_out=4, edge_weights=True):
    """row_ptr (int64) + col (int32) + the GCN weights (one f32 per edge as
    stored, else dinv, one f32 per node) + each input row once + each output
    row once."""
    w = 4 * nnz if edge_weights else 4 * n
    return 8 * (n + 1) + 4 * nnz + w + s_in * n * d + s_out * n * d


def oracle_graph(k):
    from oracle.graph import build_graph
    from sparse_message_passing_amd import synth
    inp = synth.workload_inputs(k)
    return build_graph(inp["src"], inp["dst"], int(inp["n"]), synth.WORKLOADS[k]["symmetric"]), inp


def row_sample(og, edges):
    """Consecutive rows from inside the id range (R-MAT makes ids with few
    one bits its hubs, so the start 0.7071 n has a typical mix) holding about
    `edges` edges, as an oracle graph of their own (column ids stay global).
    Returns it and its first edge slot."""
    import oracle
    r0 = int(og.n * 0.7071)
    e0 = int(og.row_ptr[r0])
    r1 = int(np.searchsorted(og.row_ptr, e0 + edges))
    r1 = max(r0 + 1, min(r1, og.n))
    e1 = int(og.row_ptr[r1])
    rp = og.row_ptr[r0:r1 + 1] - e0
    return oracle.OracleGraph(r1 - r0, rp, og.col[e0:e1].copy(), (og.dst[e0:e1] - r0).astype(np.int32)), e0


def cpu_oracle_kernels(k, og, inp, edges=1_000_000):
    """The oracle's own steps timed on one host thread and on all of them, on
    a bounded sample of the workload: the 256-wide aggregation (GCN
    workloads), the SDDMM dot and the edge softmax (GAT), the quantiser over
    the marginal rows (quantised exchange).  Rates in the bench's units."""
    import oracle
    from sparse_message_passing_amd import synth
    allt = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cfg = synth.WORKLOADS[k]
    out = {"threads_all": allt}
    jobs = []
    # inputs already in the oracle's float64, so the timed calls convert nothing
    if cfg["kind"] == "gcn" or cfg["kind"] == "quant":
        sub, e0 = row_sample(og, edges)
        X = np.random.default_rng(77).standard_normal((og.n, 256))
        w = og.gcn_norm()[1][e0:e0 + sub.nnz].astype(np.float64)
        jobs.append(("spmm_d256_gedge_feat_s", lambda: oracle.spmm(sub, X, w), sub.nnz * 256, f"{sub.n} rows, {sub.nnz} edges"))
    if cfg["kind"] == "gat":
        sub, e0 = row_sample(og, edges)
        A = np.random.default_rng(78).standard_normal((sub.n, 256))   # destination rows of the sample
        B = np.random.default_rng(79).standard_normal((og.n, 256))
        E = np.random.default_rng(80).standard_normal((sub.nnz, 4))
        jobs.append(("sddmm_dot_gedge_feat_s", lambda: oracle.sddmm_dot(sub, A, B, 4), sub.nnz * 256,
                     f"{sub.n} rows, {sub.nnz} edges, 4 heads x 64"))
        jobs.append(("edge_softmax_gedge_s", lambda: oracle.edge_softmax(sub, E), sub.nnz, f"{sub.nnz} edges, 4 heads"))
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


def cpu_baseline_gcn(min_seconds=10.0, max_passes=3):
    """The oracle's 3-layer forward+backward on the full workload, repeated
    until at least `min_seconds` of CPU work (at most `max_passes` passes);
    also returns the oracle graph and inputs for the per-step timings."""
    import oracle
    og, inp = oracle_graph(2)
    Ws = [inp["W0"], inp["W1"], inp["W2"]]
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        oracle.gcn_forward_backward(og, inp["X"], Ws, inp["labels"])
        dt += time.perf_counter() - t0
        passes += 1
    # same aggregation count as the GPU step: 128 + 256 + 41 forward, 256 + 41 backward
    work = passes * og.nnz * (128 + 256 + 41 + 256 + 41)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=work / dt / 1e9, unit="GEdge*feat/s", cores=threads, kind="oracle",
                sample=f"{passes} full 3-layer forward+backward pass(es) of the same workload "
                       f"(2^20 nodes, nnz {og.nnz}), {dt:.2f} s"), og, inp


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported (sharding is a design note, "
              "not a measured path)", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_message_passing_amd import gnnmp, synth
    from sparse_message_passing_amd.step import GatLayer, GcnStack, OverlapExchange, QuantExchange

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
    with torch.cuda.stream(stream):
        if cfg["kind"] == "gcn":
            Ws = [T(inp[f"W{i}"]) for i in range(3)]
            runner = GcnStack(g, T(inp["X"]), Ws, T(inp["labels"]), dtype=cfg.get("dtype", "f32"))
            work = runner.spmm_edge_feats()
            metric_work = work
        elif cfg["kind"] == "gat":
            runner = GatLayer(g, T(inp["X"]), T(inp["W"]), T(inp["a_src"]), T(inp["a_dst"]), cfg["heads"],
                              cfg["d_head"], cfg["slope"], T(inp["dY"]))
            hd = cfg["heads"] * cfg["d_head"]
            metric_work = g.nnz * hd * 3  # weighted SpMM, SDDMM dot, transposed SpMM
        else:
            runner = QuantExchange(g, T(inp["H"]), inp["rows"], inp["mixed_bits"], int(inp["philox_seed"]))
            metric_work = g.nnz * cfg["d"]
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
    ms = start.elapsed_time(end) / a.steps
    print(f"# timed {a.steps} steps: {ms:.3f} ms/step (wall {wall:.2f} s)", file=sys.stderr, flush=True)
    value = metric_work / (ms * 1e-3) / 1e9

    # --- dominant kernel: the aggregation (SpMM) ---------------------------
    roofline = None
    if cfg["kind"] == "gcn":
        d = 256
        X = runner.H[1]                       # a 256-wide activation
        Y = torch.empty_like(X)
        ws = torch.empty(max(gnnmp.lib().gnn_spmm_workspace_size(g.h, 0, d), 1), dtype=torch.uint8, device=dev)
        spmm_ms = event_time(lambda: gnnmp.gnn_spmm(g, X, Y, ws=ws), a.kernel_reps, stream)
        es = X.element_size()
        byts = spmm_compulsory_bytes(g.n, g.nnz, d, s_in=es, s_out=es)
        ach = byts / (spmm_ms * 1e-3) / 1e9
        traffic = measured_traffic() if a.config == 2 else None
        roofline = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic)
        extra["spmm_d256_ms"] = round(spmm_ms, 4)
        extra["spmm_d256_gedge_feat_s"] = round(g.nnz * d / (spmm_ms * 1e-3) / 1e9, 2)
        extra["spmm_d256_compulsory_bytes"] = byts
        extra["spmm_d256_compulsory_bytes_dinv"] = spmm_compulsory_bytes(g.n, g.nnz, d, s_in=es, s_out=es,
                                                                         edge_weights=False)
        extra["spmm_d256_gather_model_bytes"] = 8 * (g.n + 1) + 8 * g.nnz + es * g.nnz * d + es * g.n * d
        if traffic:
            extra["spmm_d256_counter_GBs"] = round(traffic / (spmm_ms * 1e-3) / 1e9, 1)
            extra["spmm_d256_traffic_amplification"] = round(traffic / byts, 2)
        # the update GEMM of the 256 -> 256 layer on the matrix cores
        Wt = runner.Ws[1]
        Z = torch.empty_like(X)
        gws = torch.empty(max(gnnmp.lib().gnn_gemm_workspace_size(0, 0, g.n, d, d), 1), dtype=torch.uint8, device=dev)
        gemm_ms = event_time(lambda: gnnmp.gnn_gemm(X, Wt, Z, ws=gws), a.kernel_reps, stream)
        tf = 2.0 * g.n * d * d / (gemm_ms * 1e-3) / 1e12
        extra["gemm_256x256_ms"] = round(gemm_ms, 4)
        extra["gemm_256x256_tflops"] = round(tf, 2)
        extra["gemm_256x256_frac_fp32_mfma"] = round(tf / FP32_MFMA_PEAK_TFLOPS, 4)
        # the weight-gradient GEMM (K = number of nodes, split over K)
        dW = torch.empty((d, d), device=dev)
        gws2 = torch.empty(max(gnnmp.lib().gnn_gemm_workspace_size(1, 0, d, d, g.n), 1), dtype=torch.uint8,
                           device=dev)
        dw_ms = event_time(lambda: gnnmp.gnn_gemm(X, Z, dW, transA=True, ws=gws2), a.kernel_reps, stream)
        extra["gemm_dW_256x256_ms"] = round(dw_ms, 4)
        # Tango's quantisation-aware variant of the same update (maxima,
        # stochastic 8-bit quantisation of both operands, int8 matrix cores):
        # f32 in and out, so only on the f32 workload
        if X.dtype == torch.float32:
            qws = torch.empty(gnnmp.lib().gnn_gemm_q8_workspace_size(g.n, d, d), dtype=torch.uint8, device=dev)
            q8_ms = event_time(lambda: gnnmp.gnn_gemm_q8(X, Wt, Z, seed=5, ws=qws), a.kernel_reps, stream)
            extra["gemm_q8_256x256_ms"] = round(q8_ms, 4)
            extra["gemm_q8_256x256_tops_incl_quantise"] = round(2.0 * g.n * d * d / (q8_ms * 1e-3) / 1e12, 2)
        extra["gemm_dW_256x256_tflops"] = round(2.0 * g.n * d * d / (dw_ms * 1e-3) / 1e12, 2)
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
        # the attention-gradient SDDMM dot as a primitive (f32), and Tango's
        # variant on 8-bit codes (maxima + quantisation of both operands +
        # the gather of 1-byte codes), on the layer's own H' and a dY
        h, dh = cfg["heads"], cfg["d_head"]
        Hp = runner.saved[:g.n * h * dh * 4].view(torch.float32).view(g.n, h * dh)
        dYs = runner.dY
        dal = torch.empty((g.nnz, h), device=dev)
        extra["sddmm_dot_f32_ms"] = round(event_time(
            lambda: gnnmp.gnn_sddmm(g, "dot", Hp, dYs, h, dh, dal), a.kernel_reps, stream), 4)
        sws = torch.empty(gnnmp.lib().gnn_sddmm_q8_workspace_size(g.h, h * dh), dtype=torch.uint8, device=dev)
        extra["sddmm_q8_ms"] = round(event_time(
            lambda: gnnmp.gnn_sddmm_q8(g, Hp, dYs, h, dh, dal, seed=5, ws=sws), a.kernel_reps, stream), 4)
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
        if a.config == 2:
            cpu, og, oinp = cpu_baseline_gcn()
        else:
            og, oinp = oracle_graph(a.config)
        extra["cpu_oracle"] = cpu_oracle_kernels(a.config, og, oinp)
        print("# CPU oracle timed", file=sys.stderr, flush=True)
    out = {
        "metric": "GNN layer fwd+bwd GEdge*feat/s; SpMM/SDDMM HBM GB/s as % of peak",
        "value": round(value, 3),
        "unit": "GEdge*feat/s",
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
