"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times, on outputs the oracle computes one by one (sampled rows,
columns or edges), plus bit-exact checks where the whole output is cheap for
the oracle (graph arrays, SDDMM add, quantisation codes)."""
import time

import numpy as np
import pytest
import torch

import oracle
from oracle.graph import build_graph
from parity import (RTOL16, RTOL32, bf16_values, check_close, check_gcn_stack_step, from_dev, saved_alpha,
                    softmax_row_stats, sub_rows, to_dev)
from sparse_message_passing_amd import gnnmp, synth
from sparse_message_passing_amd.step import GatLayer, GcnStack

pytestmark = pytest.mark.gpu


def log(msg):
    print(f"[fullsize] {msg}", flush=True)


def sample_rows(og, k, seed):
    """The k/4 highest in-degree rows (chunked, workgroup paths) and 3k/4 random rows."""
    r = np.random.default_rng(seed)
    top = og.degree_perm()[: k // 4]
    rnd = r.choice(og.n, k - k // 4, replace=False)
    return np.unique(np.concatenate([top, rnd])).astype(np.int64)


@pytest.fixture(scope="module")
def c2():
    t = time.time()
    inp = synth.workload_inputs(2)
    n = int(inp["n"])
    g = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=True)
    og = build_graph(inp["src"], inp["dst"], n, True)
    log(f"C2 graph n={n} nnz={og.nnz} ({time.time() - t:.1f} s)")
    return g, og, inp


def test_c2_graph_bit_exact(c2):
    g, og, _ = c2
    ex = gnnmp.gnn_graph_export(g)
    assert np.array_equal(ex["row_ptr"], og.row_ptr) and np.array_equal(ex["col"], og.col)
    dinv, w = og.gcn_norm()
    assert np.array_equal(ex["dinv"].view(np.uint32), dinv.view(np.uint32))
    assert np.array_equal(ex["w"].view(np.uint32), w.view(np.uint32))
    assert np.array_equal(ex["perm"], og.degree_perm())
    assert np.array_equal(ex["bucket_off"], og.bucket_offsets([2048, 512]))


def test_c2_gcn_step_chain(c2):
    # the 3-layer step the benchmark times (GcnStack) at 2^20 nodes, every
    # element of every layer output, saved aggregate, loss gradient, input
    # gradient and weight gradient, each layer against the oracle's layer on
    # the GPU's own inputs of that layer (padded strides, the fused input
    # ReLU masks and the reused buffers included)
    g, og, inp = c2
    Ws = [inp[f"W{i}"] for i in range(3)]
    st = GcnStack(g, to_dev(inp["X"]), [to_dev(w) for w in Ws], to_dev(inp["labels"]), dtype="f32")
    st.step()
    torch.cuda.synchronize()
    check_gcn_stack_step(og, st, Ws, inp["labels"], "f32", log=log)


@pytest.mark.parametrize("d", [256, 128, 41])
def test_c2_aggregation_sampled_rows(c2, d):
    g, og, _ = c2
    X = synth.normal((og.n, d), 77 + d)
    ld = (d + 3) // 4 * 4
    Xb = torch.zeros((og.n, ld), device="cuda")
    Xb[:, :d] = to_dev(X)
    Yb = torch.empty((og.n, ld), device="cuda")
    gnnmp.gnn_spmm(g, Xb[:, :d], Yb[:, :d])
    rows = sample_rows(og, 4096, d)
    sg, eids = sub_rows(og, rows)
    w = og.gcn_norm()[1][eids]
    ref = oracle.spmm(sg, X, w)
    mag = oracle.spmm(sg, np.abs(X), np.abs(w))
    check_close(from_dev(Yb[:, :d])[rows], ref, mag, what=f"C2 aggregation d={d}")


def test_c2_mean_aggregation_sampled(c2):
    # GraphSAGE's mean aggregator at 2^20 nodes, 256 wide (weight 1/row
    # length), and its transpose over the CSC view (the layer backward)
    _, og, inp = c2
    gs = gnnmp.gnn_graph_create(og.n, inp["src"], inp["dst"], symmetrize=True, csc=True)
    d = 256
    X = synth.normal((og.n, d), 91)
    Xd = to_dev(X)
    Y = torch.empty_like(Xd)
    w = og.mean_weights()
    gnnmp.gnn_spmm(gs, Xd, Y, weights="mean")
    rows = sample_rows(og, 4096, 91)
    sg, eids = sub_rows(og, rows)
    check_close(from_dev(Y)[rows], oracle.spmm(sg, X, w[eids]), oracle.spmm(sg, np.abs(X), w[eids]),
                what="C2 mean aggregation")
    gnnmp.gnn_spmm(gs, Xd, Y, weights="mean", transpose=True)
    # output row u of the transpose sums w[e] X[v] over u's out-edges (u -> v)
    colptr, crow, ceid = og.csc()
    cols = sample_rows(og, 4096, 92)
    lens = colptr[cols + 1] - colptr[cols]
    idx = np.concatenate([np.arange(colptr[u], colptr[u + 1]) for u in cols])
    rp = np.zeros(cols.size + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    tg = oracle.OracleGraph(cols.size, rp, crow[idx].astype(np.int32), np.repeat(cols.astype(np.int32), lens))
    wt = w[ceid[idx]]
    check_close(from_dev(Y)[cols], oracle.spmm(tg, X, wt), oracle.spmm(tg, np.abs(X), wt),
                what="C2 transposed mean aggregation")


@pytest.mark.parametrize("c", [41, 47])
def test_full_softmax_xent(c2, c):
    # the loss at the GCN workloads' logit shapes (2^20 x 41; 47 classes as
    # the bf16 workload's, on the same rows): loss and every gradient entry
    _, og, _ = c2
    n = og.n
    z = 3 * synth.normal((n, c), 60 + c)
    lab = synth.labels(n, c, 70 + c).astype(np.int32)
    loss_ref, dz_ref = oracle.softmax_xent(z, lab)
    loss = torch.empty(1, device="cuda")
    dz = torch.empty((n, c), device="cuda")
    gnnmp.gnn_softmax_xent(to_dev(z), to_dev(lab), loss, dz)
    assert abs(float(loss.item()) - loss_ref) <= RTOL32 * (abs(loss_ref) + np.abs(z).max())
    check_close(from_dev(dz), dz_ref, np.abs(dz_ref) + 2.0 / n, what=f"loss gradient {n}x{c}")


def test_c2_first_layer_forward_sampled_rows(c2):
    # ReLU((A_hat X) W1) at 2^20 nodes, 128 -> 256 (aggregate first)
    g, og, inp = c2
    X, W = inp["X"], inp["W0"]
    Y = torch.empty((og.n, 256), device="cuda")
    saved = torch.empty((og.n, 128), device="cuda")
    gnnmp.gnn_gcn_layer_fwd(g, to_dev(X), to_dev(W), Y, relu=True, saved=saved)
    rows = sample_rows(og, 2048, 5)
    sg, eids = sub_rows(og, rows)
    w = og.gcn_norm()[1][eids]
    AX = oracle.to_f32(oracle.spmm(sg, X, w))
    ref = np.maximum(AX.astype(np.float64) @ W, 0)
    mag = oracle.spmm(sg, np.abs(X), np.abs(w)) @ np.abs(W)
    check_close(from_dev(Y)[rows], ref, mag, what="C2 layer-1 forward")


def test_c2_gcn_layer_256_fwd_bwd(c2):
    # the 256 -> 256 ReLU layer at 2^20 nodes (GEMM, then aggregation):
    # Y on sampled rows; the backward from the oracle's Y (so the ReLU mask is
    # the same decision on both sides): dW in full, dX on sampled rows
    g, og, inp = c2
    n = og.n
    X = synth.normal((n, 256), 81)
    W = inp["W1"]
    dY = synth.normal((n, 256), 82)
    Xd, Wd = to_dev(X), to_dev(W)
    Y = torch.empty((n, 256), device="cuda")
    gnnmp.gnn_gcn_layer_fwd(g, Xd, Wd, Y, relu=True)
    dW = torch.empty((256, 256), device="cuda")
    dX = torch.empty((n, 256), device="cuda")
    Y_ref, _ = oracle.gcn_layer_fwd(og, X, W, True)
    log("C2 256-wide layer: oracle forward done")
    gnnmp.gnn_gcn_layer_bwd(g, Xd, Wd, to_dev(Y_ref), to_dev(dY), True, dW, dX=dX)
    rows = sample_rows(og, 4096, 83)
    sg, eids = sub_rows(og, rows)
    w = og.gcn_norm()[1]
    need = np.unique(sg.col)
    mZ = np.zeros((n, 256))
    mZ[need] = np.abs(X[need]).astype(np.float64) @ np.abs(W)
    check_close(from_dev(Y)[rows], Y_ref[rows], oracle.spmm(sg, mZ, w[eids]), what="C2 256-wide layer Y")
    dX_ref, dW_ref = oracle.gcn_layer_bwd(og, X, None, Y_ref, dY, W, True)
    log("C2 256-wide layer: oracle backward done")
    m_dZ = oracle.spmm(og, np.abs(np.where(Y_ref > 0, dY, 0.0)), w)
    check_close(from_dev(dW), dW_ref, np.abs(X).T.astype(np.float64) @ m_dZ, what="C2 256-wide layer dW")
    check_close(from_dev(dX)[rows], dX_ref[rows], m_dZ[rows] @ np.abs(W).T, what="C2 256-wide layer dX")


@pytest.mark.parametrize("shape", [("nn", 256, 256), ("nn", 128, 256), ("nn", 256, 41), ("nt", 256, 256),
                                   ("nt", 41, 256), ("tn", 256, 256)])
def test_c2_gemm_sampled(shape):
    kind, a, b = shape
    n = 1 << 20
    r = np.random.default_rng(a * b)
    if kind == "nn":      # [n, a] @ [a, b]
        A = synth.normal((n, a), 11)
        B = synth.glorot(a, b, 12)
        C = torch.empty((n, b), device="cuda")
        gnnmp.gnn_gemm(to_dev(A), to_dev(B), C)
        rows = r.choice(n, 4096, replace=False)
        ref = A[rows].astype(np.float64) @ B
        mag = np.abs(A[rows]).astype(np.float64) @ np.abs(B)
        check_close(from_dev(C)[rows], ref, mag, what=f"gemm nn {a}x{b}")
    elif kind == "nt":    # [n, a] @ [b, a]^T
        A = synth.normal((n, a), 13)
        B = synth.glorot(b, a, 14)
        C = torch.empty((n, b), device="cuda")
        gnnmp.gnn_gemm(to_dev(A), to_dev(B), C, transB=True)
        rows = r.choice(n, 4096, replace=False)
        ref = A[rows].astype(np.float64) @ B.T.astype(np.float64)
        mag = np.abs(A[rows]).astype(np.float64) @ np.abs(B).T
        check_close(from_dev(C)[rows], ref, mag, what=f"gemm nt {a}x{b}")
    else:                 # [n, a]^T @ [n, b], K = n (split over K)
        A = synth.normal((n, a), 15)
        B = synth.normal((n, b), 16)
        C = torch.empty((a, b), device="cuda")
        gnnmp.gnn_gemm(to_dev(A), to_dev(B), C, transA=True)
        cols = r.choice(b, 8, replace=False)
        ref = A.T.astype(np.float64) @ B[:, cols].astype(np.float64)
        mag = np.abs(A).T.astype(np.float64) @ np.abs(B[:, cols]).astype(np.float64)
        check_close(from_dev(C)[:, cols], ref, mag, what="gemm tn (weight gradient)")


@pytest.mark.parametrize("kind", ["nn", "tn"])
def test_c4_bf16_gemm_sampled(kind):
    # the bf16 workload's 256-wide products over 2.45M rows (a ragged last
    # tile): the bf16 x f32 update into bf16 and the bf16 x bf16 weight
    # gradient (split over K), both on the two-slabs-ahead load pipeline
    n = synth.WORKLOADS[4]["n"]
    r = np.random.default_rng(44)
    A = bf16_values(synth.normal((n, 256), 41))
    if kind == "nn":
        W = synth.glorot(256, 256, 42)
        C = torch.empty((n, 256), dtype=torch.bfloat16, device="cuda")
        gnnmp.gnn_gemm(to_dev(A, torch.bfloat16), to_dev(W), C)
        rows = np.unique(np.concatenate([r.choice(n, 4096, replace=False), np.arange(n - 64, n)]))
        ref = A[rows].astype(np.float64) @ W
        mag = np.abs(A[rows]).astype(np.float64) @ np.abs(W)
        check_close(from_dev(C)[rows], ref, mag, bf16_out=True, what="bf16 update nn 256x256")
    else:
        B = bf16_values(synth.normal((n, 256), 43))
        C = torch.empty((256, 256), device="cuda")
        gnnmp.gnn_gemm(to_dev(A, torch.bfloat16), to_dev(B, torch.bfloat16), C, transA=True)
        cols = r.choice(256, 6, replace=False)
        ref = np.zeros((256, cols.size))
        mag = np.zeros((256, cols.size))
        for i in range(0, n, 1 << 18):  # float64 in row chunks
            a = A[i:i + (1 << 18)].astype(np.float64)
            bc = B[i:i + (1 << 18), cols].astype(np.float64)
            ref += a.T @ bc
            mag += np.abs(a).T @ np.abs(bc)
        check_close(from_dev(C)[:, cols], ref, mag, what="bf16 weight gradient tn 256x256")


def test_c2_gemm_q8_sampled_rows_bit_exact():
    # the quantisation-aware GEMM at the 256 -> 256 update's full shape: the
    # tensor-wide scales and the codes of the sampled rows from the oracle,
    # the sampled output rows bit for bit
    n = 1 << 20
    A = synth.normal((n, 256), 17)
    B = synth.glorot(256, 256, 18)
    qa, sa = oracle.quantize_sym8(A, 99, 0)
    qb, sb = oracle.quantize_sym8(B, 99, 1)
    C = torch.empty((n, 256), device="cuda")
    gnnmp.gnn_gemm_q8(to_dev(A), to_dev(B), C, seed=99, stream_id=0)
    rows = np.random.default_rng(19).choice(n, 4096, replace=False)
    acc = qa[rows].astype(np.int64) @ qb.astype(np.int64)
    ref = acc.astype(np.float32) * (np.float32(sa) * np.float32(sb))
    assert np.array_equal(from_dev(C)[rows].view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------------------
# GAT layer at 2^21 nodes, 4 heads x 64, input 256
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def c3():
    t = time.time()
    inp = synth.workload_inputs(3)
    n = int(inp["n"])
    g = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=False, csc=True)
    og = build_graph(inp["src"], inp["dst"], n, False)
    log(f"C3 graph n={n} nnz={og.nnz} ({time.time() - t:.1f} s)")
    return g, og, inp


def test_c3_graph_bit_exact(c3):
    # the directed 2^21-node graph: CSR, the CSC view with its CSR slots, and
    # both degree orders
    g, og, _ = c3
    ex = gnnmp.gnn_graph_export(g)
    assert np.array_equal(ex["row_ptr"], og.row_ptr) and np.array_equal(ex["col"], og.col)
    colptr, crow, ceid = og.csc()
    assert np.array_equal(ex["col_ptr"], colptr) and np.array_equal(ex["csc_row"], crow)
    assert np.array_equal(ex["csc_eid"], ceid)
    assert np.array_equal(ex["perm"], og.degree_perm())
    outdeg = np.diff(colptr)
    assert np.array_equal(ex["perm_t"], np.lexsort((np.arange(og.n), -outdeg)).astype(np.int32))
    assert np.array_equal(ex["bucket_off"], og.bucket_offsets([2048, 512]))
    assert np.array_equal(ex["bucket_off_t"], og.bucket_offsets([2048, 2048], by_out=True))


@pytest.fixture(scope="module")
def c3_step(c3):
    """One GatLayer step (forward, then backward for the seeded upstream
    gradient) on the 2^21-node workload: the object and the launch
    configuration the benchmark times."""
    g, og, inp = c3
    cfg = synth.WORKLOADS[3]
    L = GatLayer(g, to_dev(inp["X"]), to_dev(inp["W"]), to_dev(inp["a_src"]), to_dev(inp["a_dst"]), cfg["heads"],
                 cfg["d_head"], cfg["slope"], to_dev(inp["dY"]))
    L.step()
    torch.cuda.synchronize()
    log("C3 GatLayer step done")
    return L


def test_c3_gat_forward_sampled(c3, c3_step):
    g, og, inp = c3
    cfg = synth.WORKLOADS[3]
    h, dh, slope = cfg["heads"], cfg["d_head"], cfg["slope"]
    X, W, a_s, a_d = inp["X"], inp["W"], inp["a_src"], inp["a_dst"]
    Y = c3_step.Y
    Hp_d, S_d, D_d, M_d, Z_d = gnnmp.gat_saved_views(g, c3_step.saved, h, dh)
    rows = sample_rows(og, 1024, 3)
    sg, eids = sub_rows(og, rows)
    # every node the sampled rows touch, and the sub-graph in that local numbering
    need = np.unique(np.concatenate([sg.col, rows])).astype(np.int64)
    loc = oracle.OracleGraph(sg.n, sg.row_ptr, np.searchsorted(need, sg.col).astype(np.int32),
                             np.searchsorted(need, sg.dst).astype(np.int32))
    Hp = oracle.to_f32(X[need].astype(np.float64) @ W)
    S = oracle.to_f32(oracle.gat_scores(Hp, a_s, h))
    D = oracle.to_f32(oracle.gat_scores(Hp, a_d, h))
    mHp = np.abs(X[need]).astype(np.float64) @ np.abs(W)
    nd = torch.from_numpy(need).cuda()
    check_close(from_dev(Hp_d[nd]), Hp, mHp, what="C3 H'")
    mS = oracle.gat_scores(mHp, np.abs(a_s), h)
    mD = oracle.gat_scores(mHp, np.abs(a_d), h)
    check_close(from_dev(S_d[nd]), S, mS, what="C3 S")
    check_close(from_dev(D_d[nd]), D, mD, what="C3 D")
    Ep, E = oracle.sddmm_add(loc, S, D, slope)
    mE = mS[loc.col] + mD[loc.dst]
    rowmax_v = np.maximum.reduceat(mE, loc.row_ptr[:-1], axis=0)
    M_ref, Z_ref = softmax_row_stats(loc, E)
    rd = torch.from_numpy(rows.astype(np.int64)).cuda()
    check_close(from_dev(M_d[rd]), M_ref, rowmax_v, what="C3 softmax row maximum")
    check_close(from_dev(Z_d[rd]), Z_ref, Z_ref * (2 * rowmax_v + 1), what="C3 softmax 1/sum")
    alpha = oracle.to_f32(oracle.edge_softmax(loc, E))
    rowmax = rowmax_v[np.repeat(np.arange(loc.n), np.diff(loc.row_ptr))]
    m_al = alpha * (2 * rowmax + 1)
    # the attention weights the backward forms again from the saved S, D, M, Z
    check_close(saved_alpha(og, S_d, D_d, M_d, Z_d, slope, eids), alpha, m_al, what="C3 alpha")
    ref = oracle.spmm(loc, Hp, alpha, h)
    mY = oracle.spmm(loc, mHp, m_al, h) + oracle.spmm(loc, np.abs(Hp), alpha, h)
    check_close(from_dev(Y)[rows], ref, mY, what="C3 GAT output")


def test_c3_gat_backward_sampled(c3, c3_step):
    # the layer backward at 2^21 nodes in the launch configuration the bench
    # times, dX on sampled nodes u: every step between dY and dX (SDDMM dot,
    # softmax backward, LeakyReLU', in- and out-edge sums, the transposed
    # SpMM, the rank-1 terms, the GEMM) recomputed by the oracle from X, W,
    # a and dY for those nodes only.  u needs the full in-edge rows of u and
    # of every destination of u's out-edges.
    g, og, inp = c3
    cfg = synth.WORKLOADS[3]
    h, dh, slope = cfg["heads"], cfg["d_head"], cfg["slope"]
    hd = h * dh
    X, W, a_s, a_d, dY = inp["X"], inp["W"], inp["a_src"], inp["a_dst"], inp["dY"]
    dX = c3_step.dX
    colptr, crow, _ = og.csc()
    outdeg = np.diff(colptr)
    r = np.random.default_rng(7)
    U = np.unique(np.concatenate([np.argsort(-outdeg, kind="stable")[:2],
                                  r.choice(og.n, 126, replace=False)])).astype(np.int64)
    dX_gpu = from_dev(dX[torch.from_numpy(U).cuda()])
    V = np.unique(np.concatenate([U] + [crow[colptr[u]:colptr[u + 1]].astype(np.int64) for u in U]))
    sg, _ = sub_rows(og, V)
    need = np.unique(np.concatenate([sg.col.astype(np.int64), V]))
    loc = oracle.OracleGraph(sg.n, sg.row_ptr, np.searchsorted(need, sg.col).astype(np.int32),
                             np.searchsorted(need, sg.dst).astype(np.int32))
    row_e = np.repeat(np.arange(loc.n), np.diff(loc.row_ptr))
    log(f"C3 backward oracle: {U.size} nodes, {V.size} rows, {loc.nnz} edges, {need.size} rows of H'")
    Hp = oracle.to_f32(X[need].astype(np.float64) @ W)
    S = oracle.to_f32(oracle.gat_scores(Hp, a_s, h))
    D = oracle.to_f32(oracle.gat_scores(Hp, a_d, h))
    Ep, E = oracle.sddmm_add(loc, S, D, slope)
    alpha = oracle.to_f32(oracle.edge_softmax(loc, E))
    dYV = dY[V]
    dal = oracle.to_f32(oracle.sddmm_dot(loc, dYV, Hp, h))
    dE = oracle.to_f32(oracle.edge_softmax_bwd(loc, alpha, dal))
    fac = np.where(Ep > 0, 1.0, float(np.float32(slope)))
    dEp = oracle.to_f32(dE * fac)
    ru = np.searchsorted(V, U)
    dD = oracle.to_f32(oracle.edge_reduce(loc, dEp))[ru]
    # the out-edges of u are the edges whose source is u
    nu = np.searchsorted(need, U)
    out_e = np.nonzero(np.isin(loc.col, nu))[0]
    pos = np.searchsorted(nu, loc.col[out_e])
    dS = np.zeros((U.size, h))
    np.add.at(dS, pos, dEp[out_e].astype(np.float64))
    dS = oracle.to_f32(dS)
    agg = np.zeros((U.size, hd))
    contrib = alpha[out_e].astype(np.float64)[:, :, None] * dYV[row_e[out_e]].astype(np.float64).reshape(-1, h, dh)
    np.add.at(agg, pos, contrib.reshape(-1, hd))
    rank1 = (dS.astype(np.float64)[:, :, None] * a_s[None] + dD.astype(np.float64)[:, :, None] * a_d[None])
    dHp = oracle.to_f32(agg + rank1.reshape(-1, hd))
    ref = dHp.astype(np.float64) @ W.T.astype(np.float64)
    # magnitudes: each term's absolute value carried through the same steps
    A = np.abs(alpha).astype(np.float64)
    m_dal = oracle.sddmm_dot(loc, np.abs(dYV), np.abs(Hp), h)
    m_dEp = A * (m_dal + oracle.edge_reduce(loc, A * m_dal)[row_e]) * fac
    m_dD = oracle.edge_reduce(loc, m_dEp)[ru]
    m_dS = np.zeros((U.size, h))
    np.add.at(m_dS, pos, m_dEp[out_e])
    m_agg = np.zeros((U.size, hd))
    m_c = A[out_e][:, :, None] * np.abs(dYV[row_e[out_e]]).astype(np.float64).reshape(-1, h, dh)
    np.add.at(m_agg, pos, m_c.reshape(-1, hd))
    m_dHp = m_agg + (m_dS[:, :, None] * np.abs(a_s)[None] + m_dD[:, :, None] * np.abs(a_d)[None]).reshape(-1, hd)
    check_close(dX_gpu, ref, m_dHp @ np.abs(W).T, what="C3 GAT dX")


def test_c3_gat_step_attention_and_weight_gradients(c3, c3_step):
    # the step's da_src, da_dst (every entry) and dW (every row of 8 sampled
    # columns, one or more per head) at 2^21 nodes: the oracle runs the whole
    # forward and the backward's edge steps (SDDMM dot, softmax backward,
    # LeakyReLU', in- and out-edge sums) over all 42M edges, and the
    # transposed aggregation for the sampled columns only
    g, og, inp = c3
    cfg = synth.WORKLOADS[3]
    h, dh, slope = cfg["heads"], cfg["d_head"], cfg["slope"]
    hd = h * dh
    X, W, a_s, a_d, dY = inp["X"], inp["W"], inp["a_src"], inp["a_dst"], inp["dY"]
    fw = oracle.gat_layer_fwd(og, X, W, a_s, a_d, h, slope)
    log("C3 oracle forward done")
    Hp, alpha = fw["Hp"], fw["alpha"]
    fac = np.where(fw["E_pre"] > 0, 1.0, float(np.float32(slope)))
    dal = oracle.to_f32(oracle.sddmm_dot(og, dY, Hp, h))
    dEp = oracle.to_f32(oracle.to_f32(oracle.edge_softmax_bwd(og, alpha, dal)) * fac)
    dD = oracle.to_f32(oracle.edge_reduce(og, dEp))
    dS = oracle.to_f32(oracle.edge_reduce(og, dEp, by_src=True))
    log("C3 oracle edge backward done")
    # magnitudes carried through the same steps
    A = np.abs(alpha).astype(np.float64)
    row_e = og.dst
    m_Hp = np.abs(X).astype(np.float64) @ np.abs(W)
    m_dal = oracle.sddmm_dot(og, np.abs(dY), np.abs(Hp), h)
    m_dEp = A * (m_dal + oracle.edge_reduce(og, A * m_dal)[row_e]) * fac
    m_dD = oracle.edge_reduce(og, m_dEp)
    m_dS = oracle.edge_reduce(og, m_dEp, by_src=True)
    H3, mH3 = Hp.astype(np.float64).reshape(-1, h, dh), m_Hp.reshape(-1, h, dh)
    for name, coef, mcoef, got in (("da_src", dS, m_dS, c3_step.da_src), ("da_dst", dD, m_dD, c3_step.da_dst)):
        ref = np.einsum("nk,nkj->kj", coef.astype(np.float64), H3)
        mag = np.einsum("nk,nkj->kj", mcoef, np.abs(H3)) + np.einsum("nk,nkj->kj", np.abs(coef), mH3)
        check_close(from_dev(got), ref, mag, what=f"C3 step {name}")
    r = np.random.default_rng(17)
    cols = np.unique(np.concatenate([np.arange(h) * dh, r.choice(hd, 8 - h, replace=False)]))
    dW_gpu = from_dev(c3_step.dW)[:, cols]
    for ci, c in enumerate(cols):
        k, j = divmod(int(c), dh)
        agg = oracle.spmm(og, dY[:, c:c + 1], alpha[:, k], transpose=True)[:, 0]
        m_agg = oracle.spmm(og, np.abs(dY[:, c:c + 1]), A[:, k], transpose=True)[:, 0]
        dHp_c = oracle.to_f32(agg + dS[:, k].astype(np.float64) * a_s[k, j] + dD[:, k].astype(np.float64) * a_d[k, j])
        m_dHp_c = m_agg + m_dS[:, k] * abs(a_s[k, j]) + m_dD[:, k] * abs(a_d[k, j])
        ref = X.T.astype(np.float64) @ dHp_c.astype(np.float64)
        mag = np.abs(X).T.astype(np.float64) @ m_dHp_c
        check_close(dW_gpu[:, ci], ref, mag, what=f"C3 step dW column {c}")


def test_c3_sddmm_add_full_bit_exact(c3):
    # every edge of the 42M-edge graph, scores drawn at random
    g, og, _ = c3
    S = synth.normal((og.n, 4), 31)
    D = synth.normal((og.n, 4), 32)
    out = torch.empty((og.nnz, 4), device="cuda")
    pre = torch.empty_like(out)
    gnnmp.gnn_sddmm(g, "add", to_dev(S), to_dev(D), 4, 1, out, slope=0.2, out_pre=pre)
    Ep, E = oracle.sddmm_add(og, S, D, 0.2)
    assert np.array_equal(from_dev(pre).view(np.uint32), Ep.view(np.uint32))
    assert np.array_equal(from_dev(out).view(np.uint32), E.view(np.uint32))


# ---------------------------------------------------------------------------
# quantised exchange of one partition (2^20 nodes, 314,573 marginal rows)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [2, 4, 8, "mixed"])
def test_c5_quantise_full_bit_exact(bits):
    inp = synth.workload_inputs(5)
    H, rows, seed = inp["H"], inp["rows"], int(inp["philox_seed"])
    b = inp["mixed_bits"] if bits == "mixed" else np.full(rows.size, bits, np.int32)
    Hd = to_dev(H)
    Hmix = Hd.clone()
    Hmix_ref = H.copy()
    for bb in (2, 4, 8):
        sel = rows[b == bb]
        if sel.size == 0:
            continue
        pk, sc, zr = oracle.quantize(H, sel, bb, seed)
        pkd = torch.empty(pk.shape, dtype=torch.uint8, device="cuda")
        scd = torch.empty(sel.size, device="cuda")
        zrd = torch.empty(sel.size, device="cuda")
        sd = to_dev(sel)
        gnnmp.gnn_quantize(Hd, sd, bb, seed, pkd, scd, zrd)
        assert np.array_equal(from_dev(pkd), pk)
        assert np.array_equal(from_dev(scd).view(np.uint32), sc.view(np.uint32))
        assert np.array_equal(from_dev(zrd).view(np.uint32), zr.view(np.uint32))
        gnnmp.gnn_dequantize(pkd, scd, zrd, sd, bb, Hmix)
        oracle.dequantize(pk, sc, zr, sel, H.shape[1], bb, Hmix_ref)
    assert np.array_equal(from_dev(Hmix).view(np.uint32), Hmix_ref.view(np.uint32))


def test_c5_mixed_aggregate_sampled_rows():
    inp = synth.workload_inputs(5)
    n = int(inp["n"])
    g = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=True)
    og = build_graph(inp["src"], inp["dst"], n, True)
    H, rows, seed = inp["H"], inp["rows"], int(inp["philox_seed"])
    Hmix_ref = H.copy()
    for bb in (2, 4, 8):
        sel = rows[inp["mixed_bits"] == bb]
        pk, sc, zr = oracle.quantize(H, sel, bb, seed)
        oracle.dequantize(pk, sc, zr, sel, H.shape[1], bb, Hmix_ref)
    Y = torch.empty((n, 256), device="cuda")
    gnnmp.gnn_spmm(g, to_dev(Hmix_ref), Y)
    sr = sample_rows(og, 4096, 9)
    sg, eids = sub_rows(og, sr)
    w = og.gcn_norm()[1][eids]
    check_close(from_dev(Y)[sr], oracle.spmm(sg, Hmix_ref, w), oracle.spmm(sg, np.abs(Hmix_ref), np.abs(w)),
                what="C5 aggregation of the mixed matrix")


def test_c5_dequant_in_gather_forward_and_backward():
    # the exchange at full size with the dequantisation in the gather: the
    # whole output bitwise equal to the two-kernel path, sampled rows against
    # the oracle; then the backward exchange of the embedding gradients
    from sparse_message_passing_amd.step import QuantExchange
    inp = synth.workload_inputs(5)
    n = int(inp["n"])
    g = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=True)
    og = build_graph(inp["src"], inp["dst"], n, True)
    H, rows, seed, bits = inp["H"], inp["rows"], int(inp["philox_seed"]), inp["mixed_bits"]
    Hd = to_dev(H)
    plain = QuantExchange(g, Hd, rows, bits, seed)
    fused = QuantExchange(g, Hd, rows, bits, seed, fused=True)
    Y1 = plain.step().clone()
    Y2 = fused.step().clone()
    assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))
    sr = sample_rows(og, 4096, 10)
    sg, eids = sub_rows(og, sr)
    w = og.gcn_norm()[1][eids]

    def mixed(M, stream):
        out = M.copy()
        for bb in (2, 4, 8):
            sel = rows[bits == bb]
            pk, sc, zr = oracle.quantize(M, sel, bb, seed, stream)
            oracle.dequantize(pk, sc, zr, sel, M.shape[1], bb, out)
        return out

    Hmix_ref = mixed(H, 0)
    check_close(from_dev(Y2)[sr], oracle.spmm(sg, Hmix_ref, w), oracle.spmm(sg, np.abs(Hmix_ref), np.abs(w)),
                what="C5 dequant-in-gather forward")
    del Hmix_ref, Y1, Y2
    dY = synth.normal((n, 256), 5077)
    dH = fused.backward(to_dev(dY))
    dmix_ref = mixed(dY, 1)
    check_close(from_dev(dH)[sr], oracle.spmm(sg, dmix_ref, w), oracle.spmm(sg, np.abs(dmix_ref), np.abs(w)),
                what="C5 backward gradient exchange")


def test_c5_overlapped_exchange_schedules():
    # the split exchange at full size: three schedules bitwise equal, the
    # whole output against the oracle's local + remote sums
    from sparse_message_passing_amd.step import OverlapExchange
    inp = synth.workload_inputs(5)
    n = int(inp["n"])
    g = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=True)
    og = build_graph(inp["src"], inp["dst"], n, True)
    H, rows, seed, bits = inp["H"], inp["rows"], int(inp["philox_seed"]), inp["mixed_bits"]
    ex = OverlapExchange(g, to_dev(H), rows, bits, seed)
    outs = [step().clone() for step in (ex.step_sequential, ex.step_free, ex.step_staged)]
    assert all(torch.equal(outs[0].view(torch.int32), o.view(torch.int32)) for o in outs[1:])
    yl, yr, ref, Hmix = oracle.split_aggregate(og, H, rows, bits, seed)
    sr = sample_rows(og, 8192, 11)
    mag = oracle.spmm_mag(og, Hmix, og.gcn_norm()[1])[sr]
    check_close(from_dev(outs[0])[sr], ref[sr], mag, what="C5 overlapped exchange")


def test_c5_bit_width_statistics():
    # per-row range (bit-exact) and beta of every marginal row at full size
    inp = synth.workload_inputs(5)
    n = int(inp["n"])
    g = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=True)
    og = build_graph(inp["src"], inp["dst"], n, True)
    H, rows = inp["H"], inp["rows"]
    beta = torch.empty(rows.size, device="cuda")
    rng = torch.empty(rows.size, device="cuda")
    gnnmp.gnn_quant_stats(g, to_dev(H), to_dev(rows.astype(np.int32)), beta, rng)
    beta_ref, rng_ref = oracle.quant_stats(og, H, rows)
    assert np.array_equal(from_dev(rng).view(np.uint32), rng_ref.view(np.uint32))
    np.testing.assert_allclose(from_dev(beta), beta_ref, rtol=2e-6, atol=0)


# ---------------------------------------------------------------------------
# bf16 storage at 2.45M nodes (heavy-tailed, max degree ~17K)
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def c4():
    t = time.time()
    inp = synth.workload_inputs(4)
    n = int(inp["n"])
    g = gnnmp.gnn_graph_create(n, inp["src"], inp["dst"], symmetrize=True)
    og = build_graph(inp["src"], inp["dst"], n, True)
    log(f"C4 graph n={n} nnz={og.nnz} max degree {og.deg.max()} ({time.time() - t:.1f} s)")
    return g, og, inp


def test_c4_gcn_step_chain(c4):
    # the bf16 3-layer step the benchmark times (GcnStack) at 2.45M nodes:
    # every layer output, saved aggregate and input gradient on sampled rows,
    # the loss, its gradient and every weight gradient in full, each layer
    # against the oracle's layer on the GPU's own inputs of that layer
    g, og, inp = c4
    Ws = [inp[f"W{i}"] for i in range(3)]
    st = GcnStack(g, to_dev(inp["X"]), [to_dev(w) for w in Ws], to_dev(inp["labels"]), dtype="bf16")
    st.step()
    torch.cuda.synchronize()
    check_gcn_stack_step(og, st, Ws, inp["labels"], "bf16", rows=sample_rows(og, 4096, 9), log=log)


def test_c4_graph_bit_exact(c4):
    g, og, _ = c4
    ex = gnnmp.gnn_graph_export(g)
    assert np.array_equal(ex["row_ptr"], og.row_ptr) and np.array_equal(ex["col"], og.col)
    assert np.array_equal(ex["dinv"].view(np.uint32), og.gcn_norm()[0].view(np.uint32))
    assert np.array_equal(ex["bucket_off"], og.bucket_offsets([2048, 512]))


def test_c4_bf16_first_layer_and_aggregation_sampled(c4):
    g, og, inp = c4
    X = bf16_values(inp["X"])
    W = inp["W0"]
    Xd = to_dev(X, torch.bfloat16)
    # layer 1, 100 -> 256, aggregate first, bf16 storage
    Y = torch.empty((og.n, 256), dtype=torch.bfloat16, device="cuda")
    saved = torch.empty((og.n, 100), dtype=torch.bfloat16, device="cuda")
    gnnmp.gnn_gcn_layer_fwd(g, Xd, to_dev(W), Y, relu=True, saved=saved)
    rows = sample_rows(og, 2048, 4)
    sg, eids = sub_rows(og, rows)
    w = og.gcn_norm()[1][eids]
    AX = oracle.to_bf16(oracle.spmm(sg, X, w))
    check_close(from_dev(saved)[rows], AX, oracle.spmm(sg, np.abs(X), np.abs(w)), rtol=RTOL16, bf16_out=True,
                what="C4 A_hat X (bf16)")
    ref = np.maximum(AX.astype(np.float64) @ W, 0)
    mag = oracle.spmm(sg, np.abs(X), np.abs(w)) @ np.abs(W)
    check_close(from_dev(Y)[rows], ref, mag, rtol=RTOL16, bf16_out=True, what="C4 layer-1 forward (bf16)")
    # 256-wide bf16 aggregation (the hidden layers' SpMM)
    H = bf16_values(synth.normal((og.n, 256), 41))
    Hd = to_dev(H, torch.bfloat16)
    Z = torch.empty_like(Hd)
    gnnmp.gnn_spmm(g, Hd, Z)
    check_close(from_dev(Z)[rows], oracle.spmm(sg, H, w), oracle.spmm(sg, np.abs(H), np.abs(w)), rtol=RTOL16,
                bf16_out=True, what="C4 aggregation d=256 (bf16)")


def test_c4_bf16_layer_256_fwd_bwd(c4):
    # the bf16 workload's 256 -> 256 ReLU layer at 2.45M nodes (bf16 features
    # and gradients, binary32 weights and accumulators): Y on sampled rows;
    # the backward from the oracle's Y: dW in full, dX on sampled rows
    g, og, inp = c4
    n = og.n
    X = bf16_values(synth.normal((n, 256), 85))
    W = inp["W1"]
    dY = bf16_values(synth.normal((n, 256), 86))
    Xd, Wd = to_dev(X, torch.bfloat16), to_dev(W)
    Y = torch.empty((n, 256), dtype=torch.bfloat16, device="cuda")
    gnnmp.gnn_gcn_layer_fwd(g, Xd, Wd, Y, relu=True)
    rows = sample_rows(og, 4096, 87)
    Y_gpu_rows = from_dev(Y)[rows]
    del Y
    Y_ref, _ = oracle.gcn_layer_fwd(og, X, W, True, dt="bf16")
    log("C4 256-wide bf16 layer: oracle forward done")
    sg, eids = sub_rows(og, rows)
    w = og.gcn_norm()[1]
    need = np.unique(sg.col)
    mZ = np.zeros((n, 256))
    mZ[need] = np.abs(X[need]).astype(np.float64) @ np.abs(W)
    check_close(Y_gpu_rows, Y_ref[rows], oracle.spmm(sg, mZ, w[eids]), rtol=RTOL16, bf16_out=True,
                what="C4 256-wide layer Y (bf16)")
    dW = torch.empty((256, 256), device="cuda")
    dX = torch.empty((n, 256), dtype=torch.bfloat16, device="cuda")
    gnnmp.gnn_gcn_layer_bwd(g, Xd, Wd, to_dev(Y_ref, torch.bfloat16), to_dev(dY, torch.bfloat16), True, dW, dX=dX)
    dX_rows = from_dev(dX)[rows]
    dX_ref, dW_ref = oracle.gcn_layer_bwd(og, X, None, Y_ref, dY, W, True, dt="bf16")
    log("C4 256-wide bf16 layer: oracle backward done")
    m_dZ = oracle.spmm(og, np.abs(np.where(Y_ref > 0, dY, 0.0)), w)
    check_close(from_dev(dW), dW_ref, np.abs(X).T.astype(np.float64) @ m_dZ, rtol=RTOL16,
                what="C4 256-wide layer dW")
    check_close(dX_rows, dX_ref[rows], m_dZ[rows] @ np.abs(W).T, rtol=RTOL16, bf16_out=True,
                what="C4 256-wide layer dX (bf16)")


def test_c3_sddmm_q8_sampled_bit_exact(c3):
    # Tango's quantised SDDMM dot at the full 2^21-node size: both 2 GB
    # operands quantised over the whole tensor, sampled rows bit-exact
    g, og, inp = c3
    cfg = synth.WORKLOADS[3]
    h, dh = cfg["heads"], cfg["d_head"]
    S = synth.normal((og.n, h * dh), 3101)
    D = synth.normal((og.n, h * dh), 3102)
    out = torch.empty((og.nnz, h), device="cuda")
    gnnmp.gnn_sddmm_q8(g, to_dev(S), to_dev(D), h, dh, out, seed=31, stream_id=1)
    rows = sample_rows(og, 512, 5)
    sg, eids = sub_rows(og, rows)
    ref, *_ = oracle.sddmm_q8(sg, S, D, h, seed=31, stream=1)
    got = from_dev(out[torch.from_numpy(eids).cuda()])
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
