"""Degenerate and limit cases of the primitives on the GPU: an empty node
set, graphs whose only edges are the self-loops (the operators reduce to the
identity), the widest rows each kernel takes, and the errors just past its
limits."""
import numpy as np
import pytest
import torch

import oracle
from parity import check_close, from_dev, graph_pair, hub_edges, to_dev
from sparse_message_passing_amd import gnnmp

pytestmark = pytest.mark.gpu


def test_zero_node_graph_calls_are_no_ops():
    g = gnnmp.gnn_graph_create(0, np.zeros(0, np.int32), np.zeros(0, np.int32), symmetrize=True, csc=True)
    assert g.n == 0 and g.nnz == 0
    X = torch.zeros((0, 64), device="cuda")
    Y = torch.zeros((0, 64), device="cuda")
    gnnmp.gnn_spmm(g, X, Y)
    gnnmp.gnn_spmm(g, X, Y, transpose=True, weights="mean")
    W = torch.zeros((64, 32), device="cuda")
    gnnmp.gnn_gcn_layer_fwd(g, X, W, torch.zeros((0, 32), device="cuda"), relu=True)
    rows = torch.zeros(0, dtype=torch.int32, device="cuda")
    pk = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    sc = torch.zeros(0, device="cuda")
    gnnmp.gnn_quantize(X, rows, 2, 1, pk, sc, sc)
    torch.cuda.synchronize()


@pytest.mark.parametrize("weights", ["gcn", "mean", "ones"])
def test_self_loops_only_is_the_identity(weights):
    # no edges but the self-loops: every row length is 1, so the GCN weight
    # dinv^2 and the mean weight are exactly 1 and the aggregation is X itself
    n = 3001
    g, og = graph_pair(np.zeros(0, np.int32), np.zeros(0, np.int32), n, True, csc=True)
    X = torch.randn((n, 96), device="cuda")
    Y = torch.empty_like(X)
    gnnmp.gnn_spmm(g, X, Y, weights=weights)
    assert torch.equal(Y, X)
    gnnmp.gnn_spmm(g, X, Y, weights=weights, transpose=True)
    assert torch.equal(Y, X)
    # edge softmax over one in-edge per row: alpha = 1 exactly
    E = torch.randn((n, 4), device="cuda")
    al = torch.empty_like(E)
    gnnmp.gnn_edge_softmax(g, E, al)
    assert torch.equal(al, torch.ones_like(E))


def test_widest_rows_and_limits():
    s, t = hub_edges(3000, 12000, 2600, 61)
    g, og = graph_pair(s, t, 3000, True, csc=True)
    r = np.random.default_rng(62)
    # 1024 features: the widest aggregation (four 16-byte passes per lane)
    X = r.standard_normal((3000, 1024)).astype(np.float32)
    Y = torch.empty((3000, 1024), device="cuda")
    gnnmp.gnn_spmm(g, to_dev(X), Y)
    w = og.gcn_norm()[1]
    check_close(from_dev(Y), oracle.spmm(og, X, w), oracle.spmm_mag(og, X, w), what="spmm d=1024")
    with pytest.raises(gnnmp.GnnError, match="too large"):
        Xb = torch.zeros((3000, 1028), device="cuda")
        gnnmp.gnn_spmm(g, Xb, torch.empty_like(Xb))
    # eight heads of an attention-weighted aggregation (the most the kernel takes)
    Xh = r.standard_normal((3000, 256)).astype(np.float32)
    al = r.random((og.nnz, 8)).astype(np.float32)
    Yh = torch.empty((3000, 256), device="cuda")
    gnnmp.gnn_spmm(g, to_dev(Xh), Yh, weights=to_dev(al), heads=8)
    check_close(from_dev(Yh), oracle.spmm(og, Xh, al, 8), oracle.spmm_mag(og, Xh, al, 8), what="8 heads")
    with pytest.raises(gnnmp.GnnError):
        gnnmp.gnn_spmm(g, to_dev(Xh), Yh, weights=to_dev(np.ones((og.nnz, 16), np.float32)), heads=16)
    # quantiser: 1024 features is the widest row; widths past it are refused
    rows = to_dev(np.arange(0, 3000, 7, dtype=np.int32))
    pk = torch.empty((rows.numel(), 1024), dtype=torch.uint8, device="cuda")
    sc = torch.empty(rows.numel(), device="cuda")
    zr = torch.empty_like(sc)
    gnnmp.gnn_quantize(to_dev(X), rows, 8, 5, pk, sc, zr)
    pk_ref, sc_ref, zr_ref = oracle.quantize(X, from_dev(rows), 8, 5)
    assert np.array_equal(from_dev(pk), pk_ref)
    with pytest.raises(gnnmp.GnnError, match="1024"):
        Xw = torch.zeros((3000, 1032), device="cuda")
        gnnmp.gnn_quantize(Xw, rows, 8, 5, torch.empty((rows.numel(), 1032), dtype=torch.uint8, device="cuda"),
                           sc, zr)


def test_gemm_empty_reduction_is_zero():
    A = torch.zeros((70, 0), device="cuda")
    B = torch.zeros((0, 33), device="cuda")
    C = torch.full((70, 33), float("nan"), device="cuda")
    gnnmp.gnn_gemm(A, B, C)
    assert not torch.isnan(C).any() and not C.any()


def test_zero_node_graph_attention_and_quantised_calls():
    # GAT forward/backward and the 8-bit SDDMM on an empty node set: nothing
    # to gather, and the parameter gradients are empty sums (zero)
    g = gnnmp.gnn_graph_create(0, np.zeros(0, np.int32), np.zeros(0, np.int32), csc=True)
    heads, dh, din = 4, 16, 8
    X = torch.zeros((0, din), device="cuda")
    W = torch.ones((din, heads * dh), device="cuda")
    a = torch.ones((heads, dh), device="cuda")
    Y = torch.zeros((0, heads * dh), device="cuda")
    saved = torch.zeros(max(gnnmp.gnn_gat_saved_size(g, heads, dh), 1), dtype=torch.uint8, device="cuda")
    gnnmp.gnn_gat_layer_fwd(g, X, W, a, a, heads, dh, 0.2, Y, saved)
    dW = torch.full_like(W, float("nan"))
    das = torch.full_like(a, float("nan"))
    dad = torch.full_like(a, float("nan"))
    gnnmp.gnn_gat_layer_bwd(g, X, W, a, a, heads, dh, 0.2, Y, Y, saved, dW, das, dad, dX=torch.zeros_like(X))
    assert not dW.any() and not das.any() and not dad.any()
    out = torch.zeros((0, heads), device="cuda")
    gnnmp.gnn_sddmm_q8(g, Y, Y, heads, dh, out, seed=1)
    torch.cuda.synchronize()


def test_gat_on_self_loops_only():
    # one in-edge per node (its self-loop): alpha = 1 exactly, so the layer
    # output is H' = X W bit for bit; in the backward the softmax term equals
    # the node's own attention gradient, dE = 0, dS = dD = 0, da_src = da_dst
    # = 0, and dH' = dY, so dW = X^T dY and dX = dY W^T
    n, heads, dh, din = 2000, 4, 64, 48
    g, og = graph_pair(np.zeros(0, np.int32), np.zeros(0, np.int32), n, False, csc=True)
    r = np.random.default_rng(70)
    X = to_dev(r.standard_normal((n, din)).astype(np.float32))
    W = to_dev((r.standard_normal((din, heads * dh)) * 0.1).astype(np.float32))
    a_s = to_dev(r.standard_normal((heads, dh)).astype(np.float32))
    a_d = to_dev(r.standard_normal((heads, dh)).astype(np.float32))
    Y = torch.empty((n, heads * dh), device="cuda")
    saved = torch.empty(gnnmp.gnn_gat_saved_size(g, heads, dh), dtype=torch.uint8, device="cuda")
    gnnmp.gnn_gat_layer_fwd(g, X, W, a_s, a_d, heads, dh, 0.2, Y, saved)
    Hp, S, D, M, Z = gnnmp.gat_saved_views(g, saved, heads, dh)
    # the forward's own score of each self-loop is bitwise S + D (the same
    # binary32 operations), so its maximum is that score and its sum exp(0) = 1
    E = S + D
    E = torch.where(E > 0, E, 0.2 * E)
    assert torch.equal(M, E) and torch.equal(Z, torch.ones_like(Z))
    assert torch.equal(Y, Hp)
    dY = torch.randn((n, heads * dh), device="cuda")
    dW = torch.empty_like(W)
    dX = torch.empty_like(X)
    das = torch.empty_like(a_s)
    dad = torch.empty_like(a_d)
    gnnmp.gnn_gat_layer_bwd(g, X, W, a_s, a_d, heads, dh, 0.2, Y, dY, saved, dW, das, dad, dX=dX)
    # |P| and |dalpha| are at most scale per row; dE = alpha (dalpha - P) is
    # zero up to a few roundings of that, and da sums n such terms times H'
    scale = float((dY.abs().sum(1) * Hp.abs().sum(1)).max())
    tol = 1e-6 * n * scale * float(Hp.abs().max())
    assert float(das.abs().max()) <= tol and float(dad.abs().max()) <= tol
    dW_ref = torch.empty_like(W)
    gnnmp.gnn_gemm(X, dY, dW_ref, transA=True)
    dX_ref = torch.empty_like(X)
    gnnmp.gnn_gemm(dY, W, dX_ref, transB=True)
    for got, ref, what in ((dW, dW_ref, "dW"), (dX, dX_ref, "dX")):
        err = float((got - ref).abs().max())
        assert err <= 1e-5 * float(ref.abs().max()) + tol, (what, err)
