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
