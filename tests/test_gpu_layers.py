"""GPU parity of the layer entry points (GCN and GAT, forward and backward)
against the oracle's compositions.  Backward tests feed both sides the
oracle's forward tensors, so ReLU / LeakyReLU decisions are identical and
every output is checked element by element; the multi-layer step is checked
layer by layer, element by element, each layer against the oracle applied to
the GPU's own inputs of that layer."""
import numpy as np
import pytest
import torch

import oracle
from parity import (RTOL16, RTOL32, check_close, check_gcn_stack_step, from_dev, graph_pair, hub_edges, rmat_graph,
                    saved_alpha, softmax_row_stats, to_dev)
from sparse_message_passing_amd import gnnmp, synth
from sparse_message_passing_amd.step import GcnStack

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def gcn_mag(og, X, W):
    """Magnitude |A_hat| |X| |W| of a GCN layer output (either operand order)."""
    w = og.gcn_norm()[1]
    return oracle.spmm(og, np.abs(X) @ np.abs(W), np.abs(w))


def gcn_bwd_mags(og, X, W, G):
    """Magnitudes of the GCN layer's dW and dX for the (masked) upstream
    gradient G, in the operand order the layer takes."""
    w = np.abs(og.gcn_norm()[1])
    G = np.abs(np.asarray(G, np.float64))
    d_in, d_out = W.shape
    if d_out <= d_in:
        MdZ = oracle.spmm(og, G, w, transpose=True)
        return np.abs(X).T.astype(np.float64) @ MdZ, MdZ @ np.abs(W).T
    return oracle.spmm(og, np.abs(X), w).T @ G, oracle.spmm(og, G @ np.abs(W).T, w, transpose=True)


@pytest.fixture(scope="module")
def c1():
    inp = synth.workload_inputs(1)
    g, og = graph_pair(inp["src"], inp["dst"], int(inp["n"]), True, csc=False)
    return g, og, inp


def test_c1_gcn_layer_forward(c1):
    # ReLU(A_hat (H W)): 1000 nodes, G(n, m) + self-loops, 64 -> 64
    g, og, inp = c1
    X, W = inp["X"], inp["W0"]
    ref, _ = oracle.gcn_layer_fwd(og, X, W, relu=True)
    Y = torch.empty((og.n, 64), device="cuda")
    gnnmp.gnn_gcn_layer_fwd(g, to_dev(X), to_dev(W), Y, relu=True)
    check_close(from_dev(Y), ref, gcn_mag(og, X, W), what="C1 forward")


@pytest.fixture(scope="module")
def hubsym():
    s, t = hub_edges(6000, 40000, 2500, 31)
    return graph_pair(s, t, 6000, True, csc=False)


GCN_CASES = [  # d_in, d_out, relu, storage dtype, output dtype
    (64, 64, True, "f32", "f32"),
    (48, 96, True, "f32", "f32"),
    (256, 41, False, "f32", "f32"),
    (100, 256, True, "bf16", "bf16"),
    (256, 47, False, "bf16", "f32"),
    (256, 256, True, "bf16", "bf16"),
]


@pytest.fixture(scope="module")
def hubdir():
    s, t = hub_edges(6000, 40000, 2500, 33)
    return graph_pair(s, t, 6000, False, csc=True)


GCN_DIRECTED_CASES = [GCN_CASES[0], GCN_CASES[1], GCN_CASES[3]]


@pytest.mark.parametrize("which,case", [("hubsym", c) for c in GCN_CASES] + [("hubdir", c) for c in GCN_DIRECTED_CASES],
                         ids=lambda c: c if isinstance(c, str) else "-".join(map(str, c)))
def test_gcn_layer_fwd_bwd(request, which, case):
    # on the directed graph A_hat is not symmetric, so the backward runs over
    # the CSC view (A_hat^T); on the symmetrised one over the CSR view
    d_in, d_out, relu, dt, out_dt = case
    g, og = request.getfixturevalue(which)
    r = np.random.default_rng(d_in * d_out)
    X = oracle.store(r.standard_normal((og.n, d_in)), dt)
    W = synth.glorot(d_in, d_out, 5)
    rtol = RTOL16 if dt == "bf16" else RTOL32
    # forward
    Y_ref, saved_ref = oracle.gcn_layer_fwd(og, X, W, relu, dt=dt, out_dt=out_dt)
    Xd = to_dev(X, TDT[dt])
    Wd = to_dev(W)
    Y = torch.empty((og.n, d_out), dtype=TDT[out_dt], device="cuda")
    saved = torch.empty((og.n, d_in), dtype=TDT[dt], device="cuda") if d_out > d_in else None
    gnnmp.gnn_gcn_layer_fwd(g, Xd, Wd, Y, relu=relu, saved=saved)
    check_close(from_dev(Y), Y_ref, gcn_mag(og, X, W), rtol=rtol, bf16_out=out_dt == "bf16", what="gcn fwd")
    # backward from the oracle's forward tensors
    dY = oracle.store(r.standard_normal((og.n, d_out)), out_dt)
    dX_ref, dW_ref = oracle.gcn_layer_bwd(og, X, saved_ref, Y_ref, dY, W, relu, need_dX=True, dt=dt)
    mag_dW, mag_dX = gcn_bwd_mags(og, X, W, np.where(Y_ref > 0, dY, 0.0) if relu else dY)
    dYd = to_dev(dY, TDT[out_dt])
    Yd = to_dev(Y_ref, TDT[out_dt])
    sv = to_dev(saved_ref, TDT[dt]) if saved_ref is not None else None
    dW = torch.empty((d_in, d_out), device="cuda")
    dX = torch.empty((og.n, d_in), dtype=TDT[dt], device="cuda")
    gnnmp.gnn_gcn_layer_bwd(g, Xd, Wd, Yd, dYd, relu, dW, dX=dX, saved=sv)
    check_close(from_dev(dW), dW_ref, mag_dW, rtol=rtol, what="gcn dW")
    check_close(from_dev(dX), dX_ref, mag_dX, rtol=rtol, bf16_out=dt == "bf16", what="gcn dX")
    # the input gradient times the previous layer's ReLU derivative, fused
    dX2 = torch.empty_like(dX)
    gnnmp.gnn_gcn_layer_bwd(g, Xd, Wd, Yd, dYd, relu, dW, dX=dX2, saved=sv, relu_in=True)
    keep = X > 0
    check_close(from_dev(dX2), np.where(keep, dX_ref, 0.0), np.where(keep, mag_dX, 0.0) + 1e-30, rtol=rtol,
                bf16_out=dt == "bf16", what="gcn dX (relu_in)")


SAGE_CASES = [  # d_in, d_out, relu, storage dtype
    (64, 64, True, "f32"),
    (48, 96, True, "f32"),
    (256, 41, False, "f32"),
    (100, 256, True, "bf16"),
]


@pytest.mark.parametrize("case", SAGE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_sage_layer_fwd_bwd(hubdir, case):
    # GraphSAGE mean aggregation on a directed graph: the backward must use
    # the transposed mean operator (over the CSC view)
    d_in, d_out, relu, dt = case
    g, og = hubdir
    r = np.random.default_rng(d_in + 7 * d_out)
    X = oracle.store(r.standard_normal((og.n, d_in)), dt)
    W = synth.glorot(d_in, d_out, 8)
    rtol = RTOL16 if dt == "bf16" else RTOL32
    w = og.mean_weights()
    Y_ref, saved_ref = oracle.sage_layer_fwd(og, X, W, relu, dt=dt)
    Xd, Wd = to_dev(X, TDT[dt]), to_dev(W)
    Y = torch.empty((og.n, d_out), dtype=TDT[dt], device="cuda")
    saved = torch.empty((og.n, d_in), dtype=TDT[dt], device="cuda") if d_out > d_in else None
    gnnmp.gnn_sage_layer_fwd(g, Xd, Wd, Y, relu=relu, saved=saved)
    check_close(from_dev(Y), Y_ref, oracle.spmm(og, np.abs(X) @ np.abs(W), w), rtol=rtol, bf16_out=dt == "bf16",
                what="sage fwd")
    dY = oracle.store(r.standard_normal((og.n, d_out)), dt)
    dX_ref, dW_ref = oracle.sage_layer_bwd(og, X, saved_ref, Y_ref, dY, W, relu, dt=dt)
    G = np.abs(np.where(Y_ref > 0, dY, 0.0)) if relu else np.abs(dY)
    if d_out <= d_in:
        MdZ = oracle.spmm(og, G, w, transpose=True)
        mag_dW, mag_dX = np.abs(X).T.astype(np.float64) @ MdZ, MdZ @ np.abs(W).T
    else:
        mag_dW = oracle.spmm(og, np.abs(X), w).T @ G
        mag_dX = oracle.spmm(og, G @ np.abs(W).T, w, transpose=True)
    dW = torch.empty((d_in, d_out), device="cuda")
    dX = torch.empty((og.n, d_in), dtype=TDT[dt], device="cuda")
    gnnmp.gnn_sage_layer_bwd(g, Xd, Wd, to_dev(Y_ref, TDT[dt]), to_dev(dY, TDT[dt]), relu, dW, dX=dX,
                             saved=to_dev(saved_ref, TDT[dt]) if saved_ref is not None else None)
    check_close(from_dev(dW), dW_ref, mag_dW, rtol=rtol, what="sage dW")
    check_close(from_dev(dX), dX_ref, mag_dX, rtol=rtol, bf16_out=dt == "bf16", what="sage dX")


def test_gcn_bwd_directed_requires_csc():
    # A_hat of a graph that is not symmetrised has no symmetric CSR shortcut
    s, t = hub_edges(500, 2000, 100, 35)
    g, og = graph_pair(s, t, 500, False, csc=False)
    X = torch.zeros((og.n, 8), device="cuda")
    W = torch.zeros((8, 8), device="cuda")
    with pytest.raises(gnnmp.GnnError, match="CSC"):
        gnnmp.gnn_gcn_layer_bwd(g, X, W, X, X, True, torch.empty_like(W), dX=torch.empty_like(X))


def test_sage_bwd_requires_csc(hubsym):
    g, og = hubsym
    X = torch.zeros((og.n, 8), device="cuda")
    W = torch.zeros((8, 8), device="cuda")
    with pytest.raises(gnnmp.GnnError, match="CSC"):
        gnnmp.gnn_sage_layer_bwd(g, X, W, X, X, True, torch.empty_like(W), dX=torch.empty_like(X))


def test_gcn_layer_bwd_column_slabs():
    # Source matrices over 256 MB are aggregated in 64-column slabs (300K rows
    # x 256 f32 = 307 MB): the aggregate-first backward at that size, with the
    # output-ReLU gradient mask and the fused input-ReLU mask on the slabbed
    # aggregation, and a 2000-in-neighbour hub (chunked partial rows).
    n, d_in, d_out = 300_000, 256, 288
    s, t = hub_edges(n, 1_500_000, 2000, 41)
    g, og = graph_pair(s, t, n, True, csc=False)
    r = np.random.default_rng(17)
    X = r.standard_normal((n, d_in)).astype(np.float32)
    W = synth.glorot(d_in, d_out, 6)
    Y_ref, saved_ref = oracle.gcn_layer_fwd(og, X, W, True)
    dY = r.standard_normal((n, d_out)).astype(np.float32)
    dX_ref, dW_ref = oracle.gcn_layer_bwd(og, X, saved_ref, Y_ref, dY, W, True)
    w = og.gcn_norm()[1]
    G = np.abs(np.where(Y_ref > 0, dY, 0.0))
    mag_dW = oracle.spmm(og, np.abs(X), np.abs(w)).T @ G
    mag_dX = oracle.spmm(og, G @ np.abs(W).T, np.abs(w))
    dW = torch.empty((d_in, d_out), device="cuda")
    dX = torch.empty((n, d_in), device="cuda")
    gnnmp.gnn_gcn_layer_bwd(g, to_dev(X), to_dev(W), to_dev(Y_ref), to_dev(dY), True, dW, dX=dX,
                            saved=to_dev(saved_ref), relu_in=True)
    check_close(from_dev(dW), dW_ref, mag_dW, what="slabbed dW")
    keep = X > 0
    check_close(from_dev(dX), np.where(keep, dX_ref, 0.0), np.where(keep, mag_dX, 0.0) + 1e-30,
                what="slabbed dX (relu_in)")


def test_gcn_layer_row_strided(hubsym):
    # X, Y, saved and the gradients as row-strided views (widths 41 and 47 padded to 44 / 48)
    g, og = hubsym
    r = np.random.default_rng(9)
    for d_in, d_out in ((41, 47), (47, 41)):
        X = r.standard_normal((og.n, d_in)).astype(np.float32)
        W = synth.glorot(d_in, d_out, 2)
        Y_ref, saved_ref = oracle.gcn_layer_fwd(og, X, W, relu=True)
        pad = lambda d: torch.zeros((og.n, (d + 3) // 4 * 4 + 4), device="cuda")[:, :d]
        Xd = pad(d_in)
        Xd.copy_(to_dev(X))
        Y = pad(d_out)
        saved = pad(d_in) if d_out > d_in else None
        gnnmp.gnn_gcn_layer_fwd(g, Xd, to_dev(W), Y, relu=True, saved=saved)
        check_close(from_dev(Y), Y_ref, gcn_mag(og, X, W), what=f"strided fwd {d_in}->{d_out}")
        dY = r.standard_normal((og.n, d_out)).astype(np.float32)
        dYd = pad(d_out)
        dYd.copy_(to_dev(dY))
        Yd = pad(d_out)
        Yd.copy_(to_dev(Y_ref))
        sv = None
        if saved_ref is not None:
            sv = pad(d_in)
            sv.copy_(to_dev(saved_ref))
        dX_ref, dW_ref = oracle.gcn_layer_bwd(og, X, saved_ref, Y_ref, dY, W, True)
        dX = pad(d_in)
        dW = torch.empty((d_in, d_out), device="cuda")
        gnnmp.gnn_gcn_layer_bwd(g, Xd, to_dev(W), Yd, dYd, True, dW, dX=dX, saved=sv)
        m_dW, m_dX = gcn_bwd_mags(og, X, W, np.where(Y_ref > 0, dY, 0.0))
        check_close(from_dev(dW), dW_ref, m_dW, what=f"strided dW {d_in}->{d_out}")
        check_close(from_dev(dX), dX_ref, m_dX, what=f"strided dX {d_in}->{d_out}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gcn_three_layer_step(dt):
    # the multi-layer forward + backward + loss of the 3-layer workloads,
    # scaled down, through the same GcnStack the benchmark times: every layer
    # output, saved aggregate, loss gradient, input gradient and weight
    # gradient element by element against the oracle's layer on the GPU's own
    # inputs of that layer
    s, t, n = rmat_graph(13, 16, True, 2001)
    g, og = graph_pair(s, t, n, True, csc=False)
    r = np.random.default_rng(1)
    widths = [128, 256, 256, 41] if dt == "f32" else [100, 256, 256, 47]
    X = oracle.store(r.standard_normal((n, widths[0])), dt)
    Ws = [synth.glorot(widths[i], widths[i + 1], 10 + i) for i in range(3)]
    lab = r.integers(0, widths[-1], n).astype(np.int32)
    st = GcnStack(g, to_dev(X, TDT[dt]), [to_dev(w) for w in Ws], to_dev(lab), dtype=dt)
    st.step()
    torch.cuda.synchronize()
    check_gcn_stack_step(og, st, Ws, lab, dt, log=lambda m: None)
    # and the whole step against the oracle's own composition (in norm: a
    # ReLU decision within rounding of zero may differ between the two)
    ref = oracle.gcn_forward_backward(og, X, Ws, lab, dt=dt)
    tol = 1e-4 if dt == "f32" else 2e-2
    assert abs(st.loss.item() - ref["loss"]) <= tol * abs(ref["loss"])
    # deterministic: a second step gives the same bits
    dW0 = [w.clone() for w in st.dW]
    st.step()
    assert all(torch.equal(a, b) for a, b in zip(dW0, st.dW))


# ---------------------------------------------------------------------------
# GAT
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def gatg():
    s, t = hub_edges(3000, 30000, 2300, 41)
    return graph_pair(s, t, 3000, False, csc=True)


# every group width of the backward's out-edge pass (d_head/4 = 1 ... 64 lanes)
# and every head count it instantiates
@pytest.mark.parametrize("heads,dh,din", [(4, 64, 256), (2, 32, 48), (1, 64, 64), (8, 8, 32), (1, 4, 16),
                                          (8, 16, 24), (2, 128, 64), (1, 256, 40)])
def test_gat_layer_fwd_bwd(gatg, heads, dh, din):
    g, og = gatg
    n, hd = og.n, heads * dh
    r = np.random.default_rng(heads * dh + din)
    X = r.standard_normal((n, din)).astype(np.float32)
    W = synth.glorot(din, hd, 3)
    a_s = synth.glorot(dh, 1, 4, shape=(heads, dh))
    a_d = synth.glorot(dh, 1, 5, shape=(heads, dh))
    slope = 0.2
    fw = oracle.gat_layer_fwd(og, X, W, a_s, a_d, heads, slope)
    Xd, Wd, asd, add = to_dev(X), to_dev(W), to_dev(a_s), to_dev(a_d)
    Y = torch.empty((n, hd), device="cuda")
    saved = torch.empty(gnnmp.gnn_gat_saved_size(g, heads, dh), dtype=torch.uint8, device="cuda")
    gnnmp.gnn_gat_layer_fwd(g, Xd, Wd, asd, add, heads, dh, slope, Y, saved)
    Hp, S, D, M, Z = gnnmp.gat_saved_views(g, saved, heads, dh)
    mHp = np.abs(X) @ np.abs(W)
    check_close(from_dev(Hp), fw["Hp"], mHp, what="H'")
    mS = oracle.gat_scores(mHp, np.abs(a_s), heads)
    mD = oracle.gat_scores(mHp, np.abs(a_d), heads)
    check_close(from_dev(S), fw["S"], mS, what="S")
    check_close(from_dev(D), fw["D"], mD, what="D")
    mE = mS[og.col] + mD[og.dst]
    # each row's softmax maximum moves with the scores; 1 / sum by at most
    # (1 / sum) * 2 max|dE| over the row, like alpha
    M_ref, Z_ref = softmax_row_stats(og, fw["E"])
    has = np.diff(og.row_ptr) > 0
    rowmax_v = np.maximum.reduceat(mE, og.row_ptr[:-1], axis=0)
    check_close(from_dev(M)[has], M_ref[has], rowmax_v[has], what="softmax row maximum")
    check_close(from_dev(Z)[has], Z_ref[has], Z_ref[has] * (2 * rowmax_v[has] + 1), what="softmax 1/sum")
    # alpha moves by at most alpha * 2 max|dE| over the destination's in-edges
    rowmax = rowmax_v[og.dst]
    m_al = fw["alpha"] * (2 * rowmax + 1)
    # the attention weights the backward forms again from the saved S, D, M, Z
    check_close(saved_alpha(og, S, D, M, Z, slope), fw["alpha"], m_al, what="alpha")
    mY = oracle.spmm(og, mHp, m_al, heads) + oracle.spmm(og, np.abs(fw["Hp"]), fw["alpha"], heads)
    check_close(from_dev(Y), fw["Y"], mY, what="GAT Y")

    _check_gat_bwd(g, og, fw, X, W, a_s, a_d, heads, dh, slope, saved, r)


def _check_gat_bwd(g, og, fw, X, W, a_s, a_d, heads, dh, slope, saved, r):
    """Backward from the oracle's forward tensors (copied into `saved`), every
    gradient checked element by element."""
    n, hd, din = og.n, heads * dh, X.shape[1]
    Xd, Wd, asd, add = to_dev(X), to_dev(W), to_dev(a_s), to_dev(a_d)
    Hp, S, D, M, Z = gnnmp.gat_saved_views(g, saved, heads, dh)
    M_ref, Z_ref = softmax_row_stats(og, fw["E"])
    for view, val in zip((Hp, S, D, M, Z), (fw["Hp"], fw["S"], fw["D"], M_ref, Z_ref)):
        view.copy_(to_dev(val))
    dY = r.standard_normal((n, hd)).astype(np.float32)
    bw = oracle.gat_layer_bwd(og, fw, X, W, a_s, a_d, dY, heads, slope)
    dX = torch.empty((n, din), device="cuda")
    dW = torch.empty((din, hd), device="cuda")
    das = torch.empty((heads, dh), device="cuda")
    dad = torch.empty((heads, dh), device="cuda")
    gnnmp.gnn_gat_layer_bwd(g, Xd, Wd, asd, add, heads, dh, slope, to_dev(fw["Y"]), to_dev(dY), saved, dW, das, dad,
                            dX=dX)
    A = np.abs(fw["alpha"])
    m_dal = oracle.sddmm_dot(og, np.abs(dY), np.abs(fw["Hp"]), heads)
    m_dE = A * (m_dal + oracle.edge_reduce(og, A * m_dal)[og.dst])
    fac = np.where(fw["E_pre"] > 0, 1.0, slope)
    m_dEp = m_dE * fac
    m_dD = oracle.edge_reduce(og, m_dEp)
    m_dS = oracle.edge_reduce(og, m_dEp, by_src=True)
    m_dHp = (oracle.spmm(og, np.abs(dY), A, heads, transpose=True)
             + (m_dS[:, :, None] * np.abs(a_s)[None] + m_dD[:, :, None] * np.abs(a_d)[None]).reshape(n, hd))
    H3 = np.abs(fw["Hp"]).reshape(n, heads, dh)
    check_close(from_dev(das), bw["da_src"], np.einsum("nk,nkj->kj", m_dS, H3), what="da_src")
    check_close(from_dev(dad), bw["da_dst"], np.einsum("nk,nkj->kj", m_dD, H3), what="da_dst")
    check_close(from_dev(dW), bw["dW"], np.abs(X).T @ m_dHp, what="GAT dW")
    check_close(from_dev(dX), bw["dX"], m_dHp @ np.abs(W).T, what="GAT dX")


def test_gat_layer_bwd_wide_weight():
    # d_in x heads*d_head above 2^22 elements: dX = dH' W^T takes W as given
    # (too large to transpose in the workspace first), and the dD a_dst term
    # of dH' must still enter that product
    s, t = hub_edges(300, 3000, 120, 47)
    g, og = graph_pair(s, t, 300, False, csc=True)
    heads, dh, din, slope = 8, 128, 4104, 0.2
    assert din * heads * dh > 1 << 22
    r = np.random.default_rng(48)
    X = r.standard_normal((og.n, din)).astype(np.float32)
    W = synth.glorot(din, heads * dh, 3)
    a_s = synth.glorot(dh, 1, 4, shape=(heads, dh))
    a_d = synth.glorot(dh, 1, 5, shape=(heads, dh))
    fw = oracle.gat_layer_fwd(og, X, W, a_s, a_d, heads, slope)
    saved = torch.empty(gnnmp.gnn_gat_saved_size(g, heads, dh), dtype=torch.uint8, device="cuda")
    _check_gat_bwd(g, og, fw, X, W, a_s, a_d, heads, dh, slope, saved, r)


def test_gat_layer_bwd_by_head_slabs():
    # H' and dY over 256 MB (300K rows x 4 heads x 64), the out-edge pass one
    # head at a time.  A hub with 5000 in-neighbours and ~5000 out-neighbours
    # exercises the chunked out-edge rows (partial rows summed afterwards) and
    # the whole-workgroup rows of the in-edge sum.
    n, heads, dh, din, slope = 300_000, 4, 64, 32, 0.2
    s, t = hub_edges(n, 2_000_000, 5000, 43)
    s = np.concatenate([s, np.full(5000, 7, np.int32)])
    t = np.concatenate([t, np.random.default_rng(44).choice(n, 5000, replace=False).astype(np.int32)])
    g, og = graph_pair(s, t, n, False, csc=True)
    r = np.random.default_rng(45)
    X = r.standard_normal((n, din)).astype(np.float32)
    W = synth.glorot(din, heads * dh, 3)
    a_s = synth.glorot(dh, 1, 4, shape=(heads, dh))
    a_d = synth.glorot(dh, 1, 5, shape=(heads, dh))
    fw = oracle.gat_layer_fwd(og, X, W, a_s, a_d, heads, slope)
    saved = torch.empty(gnnmp.gnn_gat_saved_size(g, heads, dh), dtype=torch.uint8, device="cuda")
    _check_gat_bwd(g, og, fw, X, W, a_s, a_d, heads, dh, slope, saved, r)


def test_gat_layer_deterministic(gatg):
    # no atomics anywhere in the layer: two forward + backward passes give the
    # same bits (hub rows chunked, partial rows summed in a fixed order)
    g, og = gatg
    from sparse_message_passing_amd.step import GatLayer
    r = np.random.default_rng(91)
    heads, dh, din = 4, 64, 256
    L = GatLayer(g, to_dev(r.standard_normal((og.n, din)).astype(np.float32)), to_dev(synth.glorot(din, heads * dh, 3)),
                 to_dev(synth.glorot(dh, 1, 4, shape=(heads, dh))), to_dev(synth.glorot(dh, 1, 5, shape=(heads, dh))),
                 heads, dh, 0.2, to_dev(r.standard_normal((og.n, heads * dh)).astype(np.float32)))
    L.step()
    first = [t.clone() for t in (L.Y, L.dX, L.dW, L.da_src, L.da_dst)]
    L.step()
    assert all(torch.equal(a, b) for a, b in zip(first, (L.Y, L.dX, L.dW, L.da_src, L.da_dst)))


@pytest.mark.parametrize("heads,dh", [(3, 16), (2, 12), (1, 512)])
def test_gat_bwd_rejects_unsupported_shapes(heads, dh):
    # the backward's out-edge pass needs 1, 2, 4 or 8 heads and d_head a power
    # of two from 4 to 256: anything else is refused before any launch
    s, t = hub_edges(64, 200, 10, 2)
    g = gnnmp.gnn_graph_create(64, s, t, csc=True)
    hd = heads * dh
    X = torch.zeros((64, 8), device="cuda")
    W = torch.zeros((8, hd), device="cuda")
    a = torch.zeros((heads, dh), device="cuda")
    Y = torch.zeros((64, hd), device="cuda")
    saved = torch.zeros(gnnmp.gnn_gat_saved_size(g, heads, dh), dtype=torch.uint8, device="cuda")
    with pytest.raises(gnnmp.GnnError, match="power of two"):
        gnnmp.gnn_gat_layer_bwd(g, X, W, a, a, heads, dh, 0.2, Y, Y, saved, torch.empty_like(W), torch.empty_like(a),
                                torch.empty_like(a))


@pytest.mark.parametrize("heads,dh", [(3, 16), (2, 12), (1, 512), (8, 256)])
def test_gat_fwd_rejects_unsupported_shapes(heads, dh):
    # refused before the first launch: Y and the saved tensors stay untouched
    s, t = hub_edges(64, 200, 10, 2)
    g = gnnmp.gnn_graph_create(64, s, t, csc=True)
    hd = heads * dh
    X = torch.ones((64, 8), device="cuda")
    W = torch.ones((8, hd), device="cuda")
    a = torch.ones((heads, dh), device="cuda")
    Y = torch.full((64, hd), 7.0, device="cuda")
    saved = torch.full((gnnmp.gnn_gat_saved_size(g, heads, dh),), 5, dtype=torch.uint8, device="cuda")
    with pytest.raises(gnnmp.GnnError, match="power of two"):
        gnnmp.gnn_gat_layer_fwd(g, X, W, a, a, heads, dh, 0.2, Y, saved)
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0)) and bool(torch.all(saved == 5))


def test_gat_bwd_requires_csc():
    s, t = hub_edges(100, 300, 10, 1)
    g = gnnmp.gnn_graph_create(100, s, t, csc=False)
    X = torch.zeros((100, 64), device="cuda")
    W = torch.zeros((64, 64), device="cuda")
    a = torch.zeros((1, 64), device="cuda")
    saved = torch.zeros(gnnmp.gnn_gat_saved_size(g, 1, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(gnnmp.GnnError, match="CSC"):
        gnnmp.gnn_gat_layer_bwd(g, X, W, a, a, 1, 64, 0.2, torch.zeros((100, 64), device="cuda"),
                                torch.zeros((100, 64), device="cuda"), saved,
                                torch.empty_like(W), torch.empty_like(a), torch.empty_like(a))
