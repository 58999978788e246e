"""GPU parity of every C-ABI primitive against the CPU oracle, element by
element, on seeded inputs that span several tiles and a ragged tail, with
hub rows that take the chunked and whole-workgroup paths."""
import numpy as np
import pytest
import torch

import oracle
from parity import (RTOL32, bf16_values, check_close, from_dev, graph_pair, hub_edges, rmat_graph, to_dev)
from sparse_message_passing_amd import gnnmp, synth

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# graph layer: bit-exact
# ---------------------------------------------------------------------------
def _graph_cases():
    r = np.random.default_rng(0)
    s = r.integers(0, 37, 200).astype(np.int32)
    t = r.integers(0, 37, 200).astype(np.int32)
    s[:30] = t[:30]                                  # self-loops
    s = np.concatenate([s, s[:50]])                  # repeats
    t = np.concatenate([t, t[:50]])
    yield "tiny-directed", s, t, 37, False
    yield "tiny-sym", s, t, 37, True
    s1, t1 = synth.gnm_pairs(1000, 5000, 1001)
    yield "gnm1000", s1, t1, 1000, True
    s2, t2, n2 = rmat_graph(13, 16, True, 5)
    yield "rmat13-sym", s2, t2, n2, True
    s3, t3 = hub_edges(6000, 20000, 4500, 3)
    yield "hub-directed", s3, t3, 6000, False
    yield "empty", np.zeros(0, np.int32), np.zeros(0, np.int32), 5, True


@pytest.mark.parametrize("case", list(_graph_cases()), ids=lambda c: c[0])
def test_graph_build_bit_exact(case):
    _, s, t, n, sym = case
    g, og = graph_pair(s, t, n, sym, csc=True)
    ex = gnnmp.gnn_graph_export(g)
    assert g.n == og.n and g.nnz == og.nnz
    assert np.array_equal(ex["row_ptr"], og.row_ptr)
    assert np.array_equal(ex["col"], og.col)
    dinv, w = og.gcn_norm()
    assert np.array_equal(ex["dinv"].view(np.uint32), dinv.view(np.uint32))
    assert np.array_equal(ex["w"].view(np.uint32), w.view(np.uint32))
    assert np.array_equal(ex["perm"], og.degree_perm())
    colptr, row, eid = og.csc()
    assert np.array_equal(ex["col_ptr"], colptr)
    assert np.array_equal(ex["csc_row"], row)
    assert np.array_equal(ex["csc_eid"], eid)
    # out-degree order of the transposed view
    od = np.diff(colptr)
    ids = np.arange(n)
    assert np.array_equal(ex["perm_t"], np.lexsort((ids, -od)).astype(np.int32))
    assert g.max_in_degree == (og.deg.max() if n else 0)
    # degree buckets of both orders, from the export and from gnn_graph_info
    assert g.bucket_threshold == [2048, 512] and g.bucket_threshold_t == [2048, 2048]
    assert np.array_equal(ex["bucket_off"], og.bucket_offsets([2048, 512]))
    assert np.array_equal(ex["bucket_off_t"], og.bucket_offsets([2048, 2048], by_out=True))
    assert g.bucket_off == ex["bucket_off"].tolist() and g.bucket_off_t == ex["bucket_off_t"].tolist()
    assert g.symmetric == sym


# ---------------------------------------------------------------------------
# SpMM
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def hubg():
    s, t = hub_edges(5000, 40000, 3000, 11)
    return graph_pair(s, t, 5000, True, csc=True)


SPMM_CASES = [
    # d, weights, heads, transpose, relu, x_dt, y_dt
    (256, "gcn", 1, False, False, "f32", "f32"),
    (256, "gcn", 1, False, True, "f32", "f32"),
    (128, "gcn", 1, False, False, "f32", "f32"),
    (64, "ones", 1, False, False, "f32", "f32"),
    (41, "gcn", 1, False, False, "f32", "f32"),
    (3, "gcn", 1, False, True, "f32", "f32"),
    (1, "ones", 1, True, False, "f32", "f32"),
    (100, "gcn", 1, False, True, "bf16", "bf16"),
    (256, "gcn", 1, False, False, "bf16", "f32"),
    (47, "gcn", 1, False, False, "f32", "bf16"),
    (256, "edge", 4, False, False, "f32", "f32"),
    (256, "edge", 4, True, False, "f32", "f32"),
    (64, "edge", 2, True, False, "f32", "f32"),
    (512, "gcn", 1, False, False, "f32", "f32"),
    (256, "mean", 1, False, False, "f32", "f32"),
    (128, "mean", 1, True, False, "f32", "f32"),
    (100, "mean", 1, False, True, "bf16", "bf16"),
]


@pytest.mark.parametrize("case", SPMM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_spmm(hubg, case):
    d, wname, heads, transpose, relu, xdt, ydt = case
    g, og = hubg
    r = np.random.default_rng(d + heads)
    X = r.standard_normal((og.n, d)).astype(np.float32)
    if xdt == "bf16":
        X = bf16_values(X)
    if wname == "gcn":
        w, wt = og.gcn_norm()[1], "gcn"
    elif wname == "ones":
        w, wt = None, "ones"
    elif wname == "mean":
        w, wt = og.mean_weights(), "mean"
    else:
        w = r.random((og.nnz, heads)).astype(np.float32)
        wt = to_dev(w)
    ref = oracle.spmm(og, X, w, heads, transpose=transpose)
    mag = oracle.spmm_mag(og, X, w, heads, transpose=transpose)
    if relu:
        ref = np.maximum(ref, 0)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    Xd = to_dev(X, tdt[xdt])
    Y = torch.full((og.n, d), float("nan"), dtype=tdt[ydt], device=Xd.device)
    gnnmp.gnn_spmm(g, Xd, Y, weights=wt, heads=heads, transpose=transpose, relu=relu)
    torch.cuda.synchronize()
    check_close(from_dev(Y), ref, mag, bf16_out=ydt == "bf16", what="spmm")


# bf16 sources whose rows are a whole number of 16 bytes take eight features
# per lane: ragged widths inside padded rows, several heads, the transposed
# view (weights through the edge map), epilogues, and hub rows split in chunks
@pytest.mark.parametrize("d,ld,wname,heads,transpose,relu,ydt", [
    (256, 256, "gcn", 1, False, False, "bf16"),
    (100, 104, "gcn", 1, False, True, "bf16"),
    (200, 208, "mean", 1, False, False, "f32"),
    (256, 256, "edge", 4, False, False, "f32"),
    (256, 256, "edge", 4, True, False, "bf16"),
    (512, 512, "gcn", 1, True, True, "f32"),
    (64, 64, "ones", 1, False, False, "bf16"),
])
def test_spmm_bf16_sixteen_byte_rows(hubg, d, ld, wname, heads, transpose, relu, ydt):
    g, og = hubg
    r = np.random.default_rng(d + ld + heads)
    X = bf16_values(r.standard_normal((og.n, d)).astype(np.float32))
    if wname == "gcn":
        w, wt = og.gcn_norm()[1], "gcn"
    elif wname == "ones":
        w, wt = None, "ones"
    elif wname == "mean":
        w, wt = og.mean_weights(), "mean"
    else:
        w = r.random((og.nnz, heads)).astype(np.float32)
        wt = to_dev(w)
    ref = oracle.spmm(og, X, w, heads, transpose=transpose)
    mag = oracle.spmm_mag(og, X, w, heads, transpose=transpose)
    if relu:
        ref = np.maximum(ref, 0)
    Xb = torch.zeros((og.n, ld), dtype=torch.bfloat16, device="cuda")
    Xb[:, :d] = to_dev(X, torch.bfloat16)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    Y = torch.full((og.n, ld), float("nan"), dtype=tdt[ydt], device="cuda")
    gnnmp.gnn_spmm(g, Xb[:, :d], Y[:, :d], weights=wt, heads=heads, transpose=transpose, relu=relu)
    torch.cuda.synchronize()
    check_close(from_dev(Y[:, :d]), ref, mag, bf16_out=ydt == "bf16", what="spmm bf16 16-byte rows")
    if ld > d:  # the padding columns of Y are never written
        assert torch.isnan(Y[:, d:].float()).all()


def test_spmm_integer_exact(hubg):
    # unit weights on small-integer features: every fp32 partial sum is exact
    g, og = hubg
    r = np.random.default_rng(5)
    X = r.integers(-4, 5, (og.n, 256)).astype(np.float32)
    Y = torch.empty((og.n, 256), device="cuda")
    gnnmp.gnn_spmm(g, to_dev(X), Y, weights="ones")
    ref = oracle.spmm(og, X)
    assert np.array_equal(from_dev(Y), ref.astype(np.float32))


def test_spmm_leading_dims_and_determinism(hubg):
    g, og = hubg
    r = np.random.default_rng(6)
    Xbig = r.standard_normal((og.n, 72)).astype(np.float32)
    Xd = to_dev(Xbig)[:, :64]                       # ldx = 72
    Ybig = torch.zeros((og.n, 68), device="cuda")
    Y = Ybig[:, :64]                                 # ldy = 68
    gnnmp.gnn_spmm(g, Xd, Y)
    w = og.gcn_norm()[1]
    ref = oracle.spmm(og, Xbig[:, :64], w)
    check_close(from_dev(Y), ref, oracle.spmm_mag(og, Xbig[:, :64], w), what="spmm-ld")
    assert torch.all(Ybig[:, 64:] == 0)
    Y2 = torch.zeros_like(Ybig)
    gnnmp.gnn_spmm(g, Xd, Y2[:, :64])
    assert torch.equal(Ybig, Y2)


def test_spmm_workspace_too_small(hubg):
    g, og = hubg
    X = torch.zeros((og.n, 64), device="cuda")
    Y = torch.zeros_like(X)
    with pytest.raises(gnnmp.GnnError):
        gnnmp.gnn_spmm(g, X, Y, ws=torch.empty(16, dtype=torch.uint8, device="cuda"))


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
GEMM_CASES = [
    # M, N, K, transA, transB, a_dt, b_dt, c_dt
    (1000, 64, 64, False, False, "f32", "f32", "f32"),
    (4099, 256, 128, False, False, "f32", "f32", "f32"),
    (777, 41, 256, False, False, "f32", "f32", "f32"),
    (1000, 256, 41, False, True, "f32", "f32", "f32"),
    (3000, 100, 47, False, True, "f32", "f32", "f32"),
    (256, 256, 70001, True, False, "f32", "f32", "f32"),
    (128, 41, 9000, True, False, "f32", "f32", "f32"),
    (2500, 256, 100, False, False, "bf16", "f32", "bf16"),
    (100, 256, 30000, True, False, "bf16", "bf16", "f32"),
    (2500, 47, 256, False, False, "bf16", "f32", "f32"),
    (33, 7, 5, False, False, "f32", "f32", "f32"),
    # both operands bf16: the bf16 matrix-core path
    (1037, 130, 256, False, False, "bf16", "bf16", "f32"),
    (999, 256, 100, False, True, "bf16", "bf16", "bf16"),
    (256, 47, 70003, True, False, "bf16", "bf16", "f32"),
    (70, 50, 30, True, True, "bf16", "bf16", "f32"),
    # bf16 x bf16 weight gradients with rows of a whole 16 bytes, split over K:
    # the 16x16x32 bf16 matrix-core kernel (ragged M, N and K, bf16 output)
    (104, 256, 30000, True, False, "bf16", "bf16", "f32"),
    (256, 72, 70003, True, False, "bf16", "bf16", "f32"),
    (256, 256, 9000, True, False, "bf16", "bf16", "bf16"),
    (136, 120, 4104, True, False, "bf16", "bf16", "f32"),
    # interior 128 x 128 tiles with a K span of 256 or more: the loads go two
    # slabs ahead (weight gradients and bf16-A products); odd and even slab
    # counts end the pipelined loop differently, and a ragged M mixes in edge
    # tiles that take the checked one-slab loop
    (256, 128, 4096, True, False, "f32", "f32", "f32"),
    (128, 256, 272, True, False, "f32", "f32", "f32"),
    (256, 256, 288, True, False, "bf16", "bf16", "f32"),
    (2048, 256, 272, False, False, "bf16", "f32", "bf16"),
    (2100, 256, 288, False, False, "bf16", "f32", "f32"),
    (1024, 128, 256, False, False, "bf16", "bf16", "f32"),
    # f32 NN products with K >= 256 run the 128 x 128 tile over eight waves
    # (two slabs ahead); odd and even slab counts, a K that ends inside a slab,
    # ragged M and N, a bf16 output, and a transposed B made NN in the workspace
    (2048, 256, 272, False, False, "f32", "f32", "f32"),
    (2100, 200, 288, False, False, "f32", "f32", "f32"),
    (1040, 130, 300, False, False, "f32", "f32", "bf16"),
    (1000, 256, 300, False, True, "f32", "f32", "f32"),
]


def _mat(r, shape, dt):
    a = r.standard_normal(shape).astype(np.float32)
    return bf16_values(a) if dt == "bf16" else a


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_gemm(case):
    M, N, K, ta, tb, adt, bdt, cdt = case
    r = np.random.default_rng(M + N + K)
    A = _mat(r, (K, M) if ta else (M, K), adt)
    B = _mat(r, (N, K) if tb else (K, N), bdt)
    ref = oracle.gemm(A, B, ta, tb)
    mag = oracle.gemm(np.abs(A), np.abs(B), ta, tb)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    C = torch.full((M, N), float("nan"), dtype=tdt[cdt], device="cuda")
    gnnmp.gnn_gemm(to_dev(A, tdt[adt]), to_dev(B, tdt[bdt]), C, transA=ta, transB=tb)
    torch.cuda.synchronize()
    check_close(from_dev(C), ref, mag, bf16_out=cdt == "bf16", what="gemm")


@pytest.mark.parametrize("ta,tb,M,N", [(False, False, 515, 260), (False, True, 515, 260), (True, False, 515, 260),
                                       (True, False, 520, 264)])
def test_gemm_bf16_pair_integer_exact(ta, tb, M, N):
    # bf16 x bf16 on the bf16 matrix cores with small integers: every product
    # and partial sum is exact in binary32, so the result is exact (rows of a
    # whole 16 bytes take the 16x16x32 weight-gradient kernel)
    r = np.random.default_rng(4)
    K = 4100
    A = r.integers(-3, 4, (K, M) if ta else (M, K)).astype(np.float32)
    B = r.integers(-3, 4, (N, K) if tb else (K, N)).astype(np.float32)
    C = torch.empty((M, N), device="cuda")
    gnnmp.gnn_gemm(to_dev(A, torch.bfloat16), to_dev(B, torch.bfloat16), C, transA=ta, transB=tb)
    assert np.array_equal(from_dev(C), oracle.gemm(A, B, ta, tb).astype(np.float32))


@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False)])
def test_gemm_integer_exact(ta, tb):
    # integer inputs in [-4, 4]: all partial sums exact in binary32, any order
    r = np.random.default_rng(3)
    M, N, K = 1037, 130, 256
    A = r.integers(-4, 5, (K, M) if ta else (M, K)).astype(np.float32)
    B = r.integers(-4, 5, (N, K) if tb else (K, N)).astype(np.float32)
    C = torch.empty((M, N), device="cuda")
    gnnmp.gnn_gemm(to_dev(A), to_dev(B), C, transA=ta, transB=tb)
    assert np.array_equal(from_dev(C), oracle.gemm(A, B, ta, tb).astype(np.float32))


# ---------------------------------------------------------------------------
# SDDMM, edge softmax, edge reductions
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def dirg():
    s, t = hub_edges(4000, 30000, 2600, 21)
    return graph_pair(s, t, 4000, False, csc=True)


@pytest.mark.parametrize("heads", [1, 2, 4, 8])
def test_sddmm_add_bit_exact(dirg, heads):
    g, og = dirg
    r = np.random.default_rng(heads)
    S = r.standard_normal((og.n, heads)).astype(np.float32)
    D = r.standard_normal((og.n, heads)).astype(np.float32)
    Ep, E = oracle.sddmm_add(og, S, D, 0.2)
    out = torch.empty((og.nnz, heads), device="cuda")
    pre = torch.empty_like(out)
    gnnmp.gnn_sddmm(g, "add", to_dev(S), to_dev(D), heads, 1, out, slope=0.2, out_pre=pre)
    assert np.array_equal(from_dev(out).view(np.uint32), E.view(np.uint32))
    assert np.array_equal(from_dev(pre).view(np.uint32), Ep.view(np.uint32))
    # no activation
    gnnmp.gnn_sddmm(g, "add", to_dev(S), to_dev(D), heads, 1, out)
    assert np.array_equal(from_dev(out).view(np.uint32), Ep.view(np.uint32))


@pytest.mark.parametrize("heads,dh,dt", [(4, 64, "f32"), (2, 32, "f32"), (1, 64, "f32"), (4, 16, "f32"),
                                         (4, 64, "bf16")])
def test_sddmm_dot(dirg, heads, dh, dt):
    g, og = dirg
    r = np.random.default_rng(heads * dh)
    A = r.standard_normal((og.n, heads * dh)).astype(np.float32)   # source side (H')
    B = r.standard_normal((og.n, heads * dh)).astype(np.float32)   # destination side (dY)
    if dt == "bf16":
        A, B = bf16_values(A), bf16_values(B)
    ref = oracle.sddmm_dot(og, B, A, heads)
    mag = oracle.sddmm_dot(og, np.abs(B), np.abs(A), heads)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    out = torch.empty((og.nnz, heads), device="cuda")
    gnnmp.gnn_sddmm(g, "dot", to_dev(A, tdt), to_dev(B, tdt), heads, dh, out)
    check_close(from_dev(out), ref, mag, what="sddmm-dot")


@pytest.mark.parametrize("heads", [1, 4, 8])
def test_edge_softmax(dirg, heads):
    g, og = dirg
    r = np.random.default_rng(40 + heads)
    E = (2 * r.standard_normal((og.nnz, heads))).astype(np.float32)
    ref = oracle.edge_softmax(og, E)
    a = torch.empty((og.nnz, heads), device="cuda")
    gnnmp.gnn_edge_softmax(g, to_dev(E), a)
    check_close(from_dev(a), ref, np.abs(ref), what="edge-softmax")
    # in place
    Ed = to_dev(E)
    gnnmp.gnn_edge_softmax(g, Ed, Ed)
    assert torch.equal(Ed, a)


@pytest.mark.parametrize("heads", [1, 4])
def test_edge_softmax_long_rows_and_masked_scores(heads):
    # rows of every length class: short (kept in registers), 65..2048 edges
    # (one pass for the maximum and sum, one for alpha), over 2048 (a whole
    # workgroup); about 10% of the scores are -inf (alpha exactly 0), and one
    # long row starts with -inf in every lane before its finite scores
    r = np.random.default_rng(60 + heads)
    n = 6000
    src = [r.integers(0, n, 40000).astype(np.int32)]
    dst = [r.integers(0, n, 40000).astype(np.int32)]
    for hub, deg in ((1, 100), (2, 700), (3, 2100), (4, 5000)):
        src.append(r.choice(np.setdiff1d(np.arange(n), [hub]), deg, replace=False).astype(np.int32))
        dst.append(np.full(deg, hub, np.int32))
    g, og = graph_pair(np.concatenate(src), np.concatenate(dst), n, False, csc=False)
    E = (3 * r.standard_normal((og.nnz, heads))).astype(np.float32)
    mask = r.random((og.nnz, heads)) < 0.1
    mask[og.row_ptr[:-1]] = False  # every row keeps a finite score
    E[mask] = -np.inf
    lo, hi = og.row_ptr[2], og.row_ptr[3]  # the 700-edge row: its first 40 scores -inf
    E[lo:lo + 40] = -np.inf
    ref = oracle.edge_softmax(og, E)
    assert np.isfinite(ref).all() and hi - lo > 64
    a = torch.empty((og.nnz, heads), device="cuda")
    gnnmp.gnn_edge_softmax(g, to_dev(E), a)
    got = from_dev(a)
    check_close(got, ref, np.abs(ref), what="edge-softmax, long rows and -inf scores")
    assert np.all(got[np.isneginf(E)] == 0.0)


@pytest.mark.parametrize("with_pre", [False, True])
def test_edge_softmax_bwd(dirg, with_pre):
    g, og = dirg
    heads = 4
    r = np.random.default_rng(7)
    alpha = oracle.to_f32(oracle.edge_softmax(og, r.standard_normal((og.nnz, heads)).astype(np.float32)))
    dal = r.standard_normal((og.nnz, heads)).astype(np.float32)
    pre = r.standard_normal((og.nnz, heads)).astype(np.float32)
    ref = oracle.edge_softmax_bwd(og, alpha, dal)
    P_mag = oracle.edge_reduce(og, np.abs(alpha) * np.abs(dal))[og.dst]
    mag = np.abs(alpha) * (np.abs(dal) + P_mag)
    if with_pre:
        fac = np.where(pre > 0, 1.0, np.float64(np.float32(0.2)))
        ref, mag = ref * fac, mag * fac
    out = torch.empty((og.nnz, heads), device="cuda")
    gnnmp.gnn_edge_softmax_bwd(g, to_dev(alpha), to_dev(dal), out, lrelu_pre=to_dev(pre) if with_pre else None,
                               slope=0.2)
    check_close(from_dev(out), ref, mag, what="edge-softmax-bwd")


@pytest.mark.parametrize("by_src,heads", [(False, 4), (True, 4), (False, 1), (True, 2)])
def test_edge_reduce(dirg, by_src, heads):
    g, og = dirg
    r = np.random.default_rng(9 + heads)
    vals = r.standard_normal((og.nnz, heads)).astype(np.float32)
    ref = oracle.edge_reduce(og, vals, by_src=by_src)
    mag = oracle.edge_reduce(og, np.abs(vals), by_src=by_src)
    out = torch.empty((og.n, heads), device="cuda")
    gnnmp.gnn_edge_reduce(g, to_dev(vals), out, by_src=by_src)
    check_close(from_dev(out), ref, mag, what="edge-reduce")


# ---------------------------------------------------------------------------
# loss
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,c", [(10000, 41), (3333, 47), (5, 130), (1, 1)])
def test_softmax_xent(n, c):
    r = np.random.default_rng(n + c)
    z = (3 * r.standard_normal((n, c))).astype(np.float32)
    lab = r.integers(0, c, n).astype(np.int32)
    loss_ref, dz_ref = oracle.softmax_xent(z, lab)
    loss = torch.empty(1, device="cuda")
    dz = torch.empty((n, c), device="cuda")
    gnnmp.gnn_softmax_xent(to_dev(z), to_dev(lab), loss, dz)
    assert abs(float(loss.item()) - loss_ref) <= RTOL32 * (abs(loss_ref) + np.abs(z).max())
    mag = (np.abs(dz_ref) + 2.0 / n)
    check_close(from_dev(dz), dz_ref, mag, what="xent-grad")


# ---------------------------------------------------------------------------
# quantisation: bit-exact codes, scales, zeros and dequantised rows
# ---------------------------------------------------------------------------
QCASES = [(256, 2), (256, 4), (256, 8), (100, 4), (100, 8), (41, 8), (64, 2), (1024, 4), (6, 4), (4, 2)]


@pytest.mark.parametrize("d,bits", QCASES)
def test_quantize_dequantize_bit_exact(d, bits):
    r = np.random.default_rng(d * bits)
    n = 3000
    H = r.standard_normal((n, d)).astype(np.float32)
    H[5] = 1.25                    # constant row
    H[6, : d // 2] = 0.0           # signed zeros as extremes
    H[6, d // 2:] = -0.0
    rows = np.sort(r.choice(n, 1111, replace=False)).astype(np.int32)
    rows[:3] = [5, 6, 7]
    rows.sort()
    seed = int(r.integers(0, 2 ** 63)) | (1 << 40)
    for stream_id in (0, 7):
        pk, sc, zr = oracle.quantize(H, rows, bits, seed, stream_id)
        pkd = torch.empty(pk.shape, dtype=torch.uint8, device="cuda")
        scd = torch.empty(rows.size, device="cuda")
        zrd = torch.empty(rows.size, device="cuda")
        Hd = to_dev(H)
        rd = to_dev(rows)
        gnnmp.gnn_quantize(Hd, rd, bits, seed, pkd, scd, zrd, stream_id=stream_id)
        got = from_dev(pkd)
        if not np.array_equal(got, pk):
            cg, cr = oracle.unpack_codes(got, d, bits), oracle.unpack_codes(pk, d, bits)
            bad = np.argwhere(cg != cr)
            i, f = bad[0]
            v = rows[i]
            x = (np.float32(H[v, f]) - zr[i]) * (np.float32(2 ** bits - 1) / (H[v].max() - H[v].min()))
            u = oracle.philox_uniforms(seed, stream_id, np.array([v], np.int32), d)[0, f]
            raise AssertionError(f"{len(bad)} codes differ (stream {stream_id}); first row {i} (node {v}) "
                                 f"feature {f}: gpu {cg[i, f]} ref {cr[i, f]}; h={H[v, f]!r} Z={zr[i]!r} "
                                 f"S={sc[i]!r} gpuS={from_dev(scd)[i]!r} gpuZ={from_dev(zrd)[i]!r} x~{x!r} u={u!r}; "
                                 f"bad features {np.unique(bad[:, 1])[:16]} rows {np.unique(bad[:, 0])[:8]}")
        assert np.array_equal(from_dev(scd).view(np.uint32), sc.view(np.uint32))
        assert np.array_equal(from_dev(zrd).view(np.uint32), zr.view(np.uint32))
        out_ref = np.full_like(H, 7.0)
        oracle.dequantize(pk, sc, zr, rows, d, bits, out_ref)
        out = torch.full((n, d), 7.0, device="cuda")
        gnnmp.gnn_dequantize(pkd, scd, zrd, rd, bits, out)
        assert np.array_equal(from_dev(out).view(np.uint32), out_ref.view(np.uint32))


def test_quantize_strided_rows():
    r = np.random.default_rng(1)
    Hbig = r.standard_normal((500, 80)).astype(np.float32)
    rows = np.arange(0, 500, 7, dtype=np.int32)
    pk, sc, zr = oracle.quantize(np.ascontiguousarray(Hbig[:, :64]), rows, 4, 99)
    Hd = to_dev(Hbig)[:, :64]
    pkd = torch.empty(pk.shape, dtype=torch.uint8, device="cuda")
    scd = torch.empty(rows.size, device="cuda")
    zrd = torch.empty(rows.size, device="cuda")
    gnnmp.gnn_quantize(Hd, to_dev(rows), 4, 99, pkd, scd, zrd)
    assert np.array_equal(from_dev(pkd), pk)


@pytest.mark.parametrize("bits", [2, 4, 8, "mixed"])
def test_quantized_exchange_then_aggregate(bits):
    # AdaQP Eqn. 7 on one partition: marginal rows quantised and dequantised,
    # central rows exact, then the GCN aggregation
    s, t, n = rmat_graph(12, 24, True, 77)
    g, og = graph_pair(s, t, n, True, csc=False)
    r = np.random.default_rng(3)
    H = r.standard_normal((n, 256)).astype(np.float32)
    rows = synth.marginal_rows(n, 0.3, 5)
    b = bits if bits != "mixed" else synth.random_bits(rows.size, (2, 4, 8), 6)
    Hmix_ref, Y_ref, parts = oracle.quantized_aggregate(og, H, rows, b, seed=1234)
    Hd = to_dev(H)
    Hmix = Hd.clone()
    for bb, (sel, pk, sc, zr) in parts.items():
        pkd = torch.empty(pk.shape, dtype=torch.uint8, device="cuda")
        scd = torch.empty(sel.size, device="cuda")
        zrd = torch.empty(sel.size, device="cuda")
        sd = to_dev(sel)
        gnnmp.gnn_quantize(Hd, sd, bb, 1234, pkd, scd, zrd)
        gnnmp.gnn_dequantize(pkd, scd, zrd, sd, bb, Hmix)
    assert np.array_equal(from_dev(Hmix).view(np.uint32), Hmix_ref.view(np.uint32))
    Y = torch.empty_like(Hmix)
    gnnmp.gnn_spmm(g, Hmix, Y)
    w = og.gcn_norm()[1]
    check_close(from_dev(Y), Y_ref, oracle.spmm_mag(og, Hmix_ref, w), what="mixed aggregate")


# ---------------------------------------------------------------------------
# dequantise-in-gather aggregation (marginal rows read straight from codes)
# ---------------------------------------------------------------------------
def _gpu_groups(Hd, parts, seed, stream_id):
    """Quantise each bit-width group on the GPU (codes checked against the
    oracle's) and return the group descriptors and row lists."""
    groups, rows_list = [], []
    for bb, (sel, pk, sc, zr) in parts.items():
        sd = to_dev(sel)
        pkd = torch.empty(pk.shape, dtype=torch.uint8, device="cuda")
        scd = torch.empty(sel.size, device="cuda")
        zrd = torch.empty(sel.size, device="cuda")
        gnnmp.gnn_quantize(Hd, sd, bb, seed, pkd, scd, zrd, stream_id=stream_id)
        assert np.array_equal(from_dev(pkd), pk)
        groups.append((pkd, scd, zrd, bb))
        rows_list.append(sd)
    return groups, rows_list


@pytest.mark.parametrize("bits,d", [(2, 256), (4, 64), (8, 256), ("mixed", 256), ("mixed", 4)])
def test_spmm_dequant_in_gather(bits, d):
    # AdaQP Eqn. 5 and 7 with the dequantisation moved into the gather: against
    # the oracle's dequantise-then-aggregate composition element by element,
    # and bitwise against the GPU's two-kernel path (same values, same order).
    s, t, n = rmat_graph(12, 24, True, 78)
    g, og = graph_pair(s, t, n, True, csc=False)
    r = np.random.default_rng(d)
    H = r.standard_normal((n, d)).astype(np.float32)
    rows = synth.marginal_rows(n, 0.3, 7)
    H[rows[:5]] = 1.5                      # constant rows: scale 0, every value the zero point
    b = bits if bits != "mixed" else synth.random_bits(rows.size, (2, 4, 8), 8)
    seed, sid = 4321, 1
    Hmix_ref, Y_ref, parts = oracle.quantized_aggregate(og, H, rows, b, seed=seed, stream=sid)
    Hd = to_dev(H)
    groups, rows_list = _gpu_groups(Hd, parts, seed, sid)
    qslot = torch.empty(n, dtype=torch.int32, device="cuda")
    gnnmp.gnn_quant_slots(n, rows_list, qslot)
    want = np.full(n, -1, np.int64)
    for gi, (bb, (sel, *_)) in enumerate(parts.items()):
        want[sel] = (gi << 27) | np.arange(sel.size)
    assert np.array_equal(from_dev(qslot).astype(np.int64), want)
    Y = torch.empty((n, d), device="cuda")
    gnnmp.gnn_spmm_dequant(g, Hd, qslot, groups, Y)
    w = og.gcn_norm()[1]
    check_close(from_dev(Y), Y_ref, oracle.spmm_mag(og, Hmix_ref, w), what=f"dequant-in-gather b={bits} d={d}")
    Hmix = Hd.clone()
    for (pkd, scd, zrd, bb), sd in zip(groups, rows_list):
        gnnmp.gnn_dequantize(pkd, scd, zrd, sd, bb, Hmix)
    Y2 = torch.empty_like(Y)
    gnnmp.gnn_spmm(g, Hmix, Y2)
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
    # fused ReLU
    gnnmp.gnn_spmm_dequant(g, Hd, qslot, groups, Y, relu=True)
    gnnmp.gnn_spmm(g, Hmix, Y2, relu=True)
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))


def test_spmm_dequant_without_quantised_rows():
    # no groups, every slot -1: the plain aggregation, bitwise
    s, t = hub_edges(2000, 12000, 700, 5)
    g, og = graph_pair(s, t, 2000, True, csc=False)
    X = to_dev(np.random.default_rng(2).standard_normal((2000, 128)).astype(np.float32))
    qslot = torch.empty(2000, dtype=torch.int32, device="cuda")
    gnnmp.gnn_quant_slots(2000, [], qslot)
    assert bool((qslot == -1).all())
    Y = torch.empty_like(X)
    Y2 = torch.empty_like(X)
    gnnmp.gnn_spmm_dequant(g, X, qslot, [], Y)
    gnnmp.gnn_spmm(g, X, Y2)
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))


def test_spmm_dequant_rejects_bad_shapes():
    s, t = hub_edges(100, 400, 10, 6)
    g, _ = graph_pair(s, t, 100, True, csc=False)
    qslot = torch.full((100,), -1, dtype=torch.int32, device="cuda")
    X = torch.zeros((100, 42), device="cuda")
    with pytest.raises(gnnmp.GnnError, match="multiple of 4"):
        gnnmp.gnn_spmm_dequant(g, X, qslot, [], torch.empty_like(X))
    X = torch.zeros((100, 64), device="cuda")
    pk = torch.zeros((1, 16), dtype=torch.uint8, device="cuda")
    sc = torch.zeros(1, device="cuda")
    with pytest.raises(gnnmp.GnnError, match="bits"):
        gnnmp.gnn_spmm_dequant(g, X, qslot, [(pk, sc, sc, 3)], torch.empty_like(X))


def test_quantized_exchange_step_fused_and_backward():
    # the step object: the fused forward equals the two-kernel forward bitwise;
    # the backward exchanges the gradient rows quantised (Philox stream + 1)
    from sparse_message_passing_amd.step import QuantExchange
    s, t, n = rmat_graph(11, 24, True, 79)
    g, og = graph_pair(s, t, n, True, csc=False)
    r = np.random.default_rng(11)
    H = r.standard_normal((n, 128)).astype(np.float32)
    dY = r.standard_normal((n, 128)).astype(np.float32)
    rows = synth.marginal_rows(n, 0.3, 12)
    b = synth.random_bits(rows.size, (2, 4, 8), 13)
    plain = QuantExchange(g, to_dev(H), rows, b, 77, stream_id=2)
    fused = QuantExchange(g, to_dev(H), rows, b, 77, stream_id=2, fused=True)
    Y1 = plain.step().clone()
    Y2 = fused.step().clone()
    assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))
    mix_ref, Y_ref, _ = oracle.quantized_aggregate(og, H, rows, b, seed=77, stream=2)
    w = og.gcn_norm()[1]
    check_close(from_dev(Y2), Y_ref, oracle.spmm_mag(og, mix_ref, w), what="exchange forward")
    dH = fused.backward(to_dev(dY))
    dmix_ref, dH_ref, _ = oracle.quantized_aggregate(og, dY, rows, b, seed=77, stream=3)
    check_close(from_dev(dH), dH_ref, oracle.spmm_mag(og, dmix_ref, w), what="exchange backward")


# ---------------------------------------------------------------------------
# AdaQP Eqn. 7 split and the overlapped exchange
# ---------------------------------------------------------------------------
def test_graph_split_matches_oracle():
    s, t = hub_edges(3000, 20000, 800, 21)
    g, og = graph_pair(s, t, 3000, True, csc=False)
    marginal = np.random.default_rng(22).random(3000) < 0.3
    lo, hi = gnnmp.gnn_graph_split(g, marginal)
    lg, rg, lw, rw = og.split_by_source(marginal)
    for gg, ref, wref in ((lo, lg, lw), (hi, rg, rw)):
        ex = gnnmp.gnn_graph_export(gg)
        assert np.array_equal(ex["row_ptr"], ref.row_ptr) and np.array_equal(ex["col"], ref.col)
        assert np.array_equal(ex["w"].view(np.uint32), wref.view(np.uint32))
        assert np.array_equal(ex["perm"], ref.degree_perm())


@pytest.mark.parametrize("bits", [4, "mixed"])
def test_overlap_exchange_schedules(bits):
    # the central/marginal split on two streams: the three schedules run the
    # same kernels in the same order per element, so agree bitwise; the result
    # is Eqn. 7's local sum plus remote sum
    from sparse_message_passing_amd.step import OverlapExchange
    s, t, n = rmat_graph(12, 24, True, 80)
    g, og = graph_pair(s, t, n, True, csc=False)
    r = np.random.default_rng(23)
    H = r.standard_normal((n, 256)).astype(np.float32)
    rows = synth.marginal_rows(n, 0.3, 24)
    b = bits if bits != "mixed" else synth.random_bits(rows.size, (2, 4, 8), 25)
    ex = OverlapExchange(g, to_dev(H), rows, b, 555)
    outs = []
    for step in (ex.step_sequential, ex.step_free, ex.step_staged):
        ex.Y.fill_(float("nan"))
        outs.append(step().clone())
        torch.cuda.synchronize()
        tl = ex.timeline()
        assert tl["end"] >= max(tl["central"], tl["transferred"]) >= 0.0
    assert all(torch.equal(outs[0].view(torch.int32), o.view(torch.int32)) for o in outs[1:])
    yl, yr, ref, Hmix = oracle.split_aggregate(og, H, rows, b, 555)
    check_close(from_dev(outs[0]), ref, oracle.spmm_mag(og, Hmix, og.gcn_norm()[1]) + 1e-30,
                what=f"overlapped exchange b={bits}")


# ---------------------------------------------------------------------------
# bit-width statistics (AdaQP Sec. 3.2) and the adaptive assignment
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("directed", [False, True])
def test_quant_stats_matches_oracle(directed):
    s, t = hub_edges(5000, 30000, 1500, 26)
    g, og = graph_pair(s, t, 5000, not directed, csc=directed)
    r = np.random.default_rng(27)
    H = (r.standard_normal((5000, 96)) * r.uniform(0.1, 4, (5000, 1))).astype(np.float32)
    rows = synth.marginal_rows(5000, 0.3, 28)
    rows = np.concatenate([rows, [0]]).astype(np.int32)   # the hub (node 0 has hub_in in-edges)
    H[rows[3]] = -2.5                                      # a constant row: range 0, beta 0
    w = None if not directed else r.random(og.nnz).astype(np.float32)
    beta_ref, rng_ref = oracle.quant_stats(og, H, rows, w)
    beta = torch.empty(rows.size, device="cuda")
    rngd = torch.empty(rows.size, device="cuda")
    gnnmp.gnn_quant_stats(g, to_dev(H), to_dev(rows), beta, rngd, edge_w=None if w is None else to_dev(w))
    assert np.array_equal(from_dev(rngd).view(np.uint32), rng_ref.view(np.uint32))
    np.testing.assert_allclose(from_dev(beta), beta_ref, rtol=2e-6, atol=0)


def test_adaptive_assignment_lowers_variance():
    # statistics on the GPU, greedy assignment on the host, at the average
    # width of uniform sampling from {2, 4, 8}: lower variance than the
    # uniform draw (AdaQP Table 6's comparison, in variance terms)
    from sparse_message_passing_amd.step import adaptive_bits
    s, t, n = rmat_graph(12, 24, True, 81)
    g, og = graph_pair(s, t, n, True, csc=False)
    r = np.random.default_rng(29)
    H = (r.standard_normal((n, 128)) * r.lognormal(0, 1, (n, 1))).astype(np.float32)
    rows = synth.marginal_rows(n, 0.3, 30)
    uniform = synth.random_bits(rows.size, (2, 4, 8), 31)
    avg = float(uniform.mean())
    bits, beta = adaptive_bits(g, to_dev(H), rows, avg)
    beta_ref, _ = oracle.quant_stats(og, H, rows)
    np.testing.assert_allclose(beta, beta_ref, rtol=2e-6)
    assert np.array_equal(bits, oracle.assign_bits_greedy(beta.astype(np.float64), 128, avg))
    assert bits.sum() <= uniform.sum()                          # no more bytes than the uniform draw
    assert oracle.quant_variance(beta, bits) < oracle.quant_variance(beta, uniform)


# ---------------------------------------------------------------------------
# Tango's quantisation-aware GEMM on the int8 matrix cores
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K", [(1000, 256, 128), (777, 41, 256), (4099, 100, 70), (33, 7, 5), (300, 130, 3000)])
def test_gemm_q8_bit_exact(M, N, K):
    # codes, int32 sums and the binary32 dequantisation are all fixed by the
    # definition: the result matches the oracle bit for bit
    r = np.random.default_rng(M + N + K)
    A = (r.standard_normal((M, K)) * r.uniform(0.5, 2, (M, 1))).astype(np.float32)
    B = r.standard_normal((K, N)).astype(np.float32)
    ref, *_ = oracle.gemm_q8(A, B, seed=606, stream=3)
    C = torch.full((M, N), float("nan"), device="cuda")
    gnnmp.gnn_gemm_q8(to_dev(A), to_dev(B), C, seed=606, stream_id=3)
    assert np.array_equal(from_dev(C).view(np.uint32), ref.view(np.uint32))


def test_gemm_q8_zero_and_strided():
    r = np.random.default_rng(7)
    A = np.zeros((50, 64), np.float32)
    B = r.standard_normal((64, 20)).astype(np.float32)
    C = torch.full((50, 20), float("nan"), device="cuda")
    gnnmp.gnn_gemm_q8(to_dev(A), to_dev(B), C, seed=1)
    assert not from_dev(C).any()
    # row-strided operands and output
    A = r.standard_normal((90, 40)).astype(np.float32)
    Ab = torch.zeros((90, 48), device="cuda")
    Ab[:, :40] = to_dev(A)
    Bb = torch.zeros((40, 24), device="cuda")
    Bb[:, :20] = to_dev(B[:40])
    Cb = torch.zeros((90, 28), device="cuda")
    gnnmp.gnn_gemm_q8(Ab[:, :40], Bb[:, :20], Cb[:, :20], seed=2)
    ref, *_ = oracle.gemm_q8(A, B[:40], seed=2)
    assert np.array_equal(from_dev(Cb[:, :20]).view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------------------
# Tango's SDDMM dot on 8-bit codes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("heads,dh", [(4, 64), (1, 16), (3, 16), (2, 128), (8, 32), (1, 256), (4, 256)])
def test_sddmm_q8_bit_exact(heads, dh):
    # codes, int32 sums and the binary32 dequantisation are fixed by the
    # definition: every edge matches the oracle bit for bit (a hub with 2300
    # in-edges exercises the chunked rows)
    s, t = hub_edges(3000, 30000, 2300, heads * dh)
    g, og = graph_pair(s, t, 3000, False, csc=False)
    r = np.random.default_rng(heads + dh)
    S = (r.standard_normal((og.n, heads * dh)) * r.uniform(0.5, 2, (og.n, 1))).astype(np.float32)
    D = r.standard_normal((og.n, heads * dh)).astype(np.float32)
    ref, *_ = oracle.sddmm_q8(og, S, D, heads, seed=77, stream=2)
    out = torch.full((og.nnz, heads), float("nan"), device="cuda")
    gnnmp.gnn_sddmm_q8(g, to_dev(S), to_dev(D), heads, dh, out, seed=77, stream_id=2)
    assert np.array_equal(from_dev(out).view(np.uint32), ref.view(np.uint32))


def test_sddmm_q8_strided_zero_and_unsupported():
    s, t = hub_edges(500, 4000, 300, 5)
    g, og = graph_pair(s, t, 500, False, csc=False)
    r = np.random.default_rng(8)
    S = r.standard_normal((og.n, 64)).astype(np.float32)
    D = r.standard_normal((og.n, 64)).astype(np.float32)
    Sb = torch.zeros((og.n, 80), device="cuda")
    Sb[:, :64] = to_dev(S)
    Db = torch.zeros((og.n, 72), device="cuda")
    Db[:, :64] = to_dev(D)
    out = torch.empty((og.nnz, 2), device="cuda")
    gnnmp.gnn_sddmm_q8(g, Sb[:, :64], Db[:, :64], 2, 32, out, seed=3)
    ref, *_ = oracle.sddmm_q8(og, S, D, 2, seed=3)
    assert np.array_equal(from_dev(out).view(np.uint32), ref.view(np.uint32))
    gnnmp.gnn_sddmm_q8(g, torch.zeros((og.n, 64), device="cuda"), Db[:, :64], 2, 32, out, seed=3)
    assert not from_dev(out).any()
    with pytest.raises(gnnmp.GnnError, match="d_head"):
        gnnmp.gnn_sddmm_q8(g, Sb[:, :48], Db[:, :48], 2, 24, out, seed=3)
