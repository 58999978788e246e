"""Pins of the oracle's primitives: dense products on tiny graphs, brute force
over edge lists, the Tango worked example, finite differences and closed forms."""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from oracle.graph import OracleGraph, build_graph

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def tiny_graph(seed, n=24, m=90, symmetrize=False):
    g0 = np.random.default_rng(seed)
    src = g0.integers(0, n, m).astype(np.int32)
    dst = g0.integers(0, n, m).astype(np.int32)
    return build_graph(src, dst, n, symmetrize), src, dst


def edge_list(g):
    """(u, v) per CSR slot, taken straight from the brute-force structure."""
    return [(int(g.col[e]), int(g.dst[e])) for e in range(g.nnz)]


# ---------------------------------------------------------------------------
# SpMM
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("heads", [1, 2, 4])
@pytest.mark.parametrize("seed", [0, 1])
def test_spmm_dense(heads, seed):
    g, _, _ = tiny_graph(seed)
    r = np.random.default_rng(10 + seed)
    d = 8 * heads
    X = r.standard_normal((g.n, d)).astype(np.float32)
    w = r.standard_normal((g.nnz, heads)).astype(np.float32)
    Y = oracle.spmm(g, X, w, heads)
    dh = d // heads
    for k in range(heads):
        A = g.dense(w[:, k])
        assert np.allclose(Y[:, k * dh:(k + 1) * dh], A @ X[:, k * dh:(k + 1) * dh].astype(np.float64), rtol=1e-12, atol=1e-12)
    Yt = oracle.spmm(g, X, w, heads, transpose=True)
    for k in range(heads):
        A = g.dense(w[:, k])
        assert np.allclose(Yt[:, k * dh:(k + 1) * dh], A.T @ X[:, k * dh:(k + 1) * dh].astype(np.float64), rtol=1e-12, atol=1e-12)
    # ones
    assert np.allclose(oracle.spmm(g, X), g.dense() @ X.astype(np.float64))


def test_spmm_linearity_and_mag():
    g, _, _ = tiny_graph(3)
    r = np.random.default_rng(3)
    X1 = r.standard_normal((g.n, 5)).astype(np.float32)
    X2 = r.standard_normal((g.n, 5)).astype(np.float32)
    _, w = build_graph(g.col, g.dst, g.n, False).gcn_norm()
    Y = oracle.spmm(g, X1, w) + oracle.spmm(g, X2, w)
    assert np.allclose(Y, oracle.spmm(g, (X1.astype(np.float64) + X2).astype(np.float32), w), atol=1e-6)
    M = oracle.spmm_mag(g, X1, w)
    assert np.all(M >= np.abs(oracle.spmm(g, X1, w)) - 1e-12)


# ---------------------------------------------------------------------------
# SDDMM, edge softmax, edge reductions
# ---------------------------------------------------------------------------
def test_sddmm_add_leaky_brute_force():
    g, _, _ = tiny_graph(4)
    r = np.random.default_rng(4)
    S = r.standard_normal((g.n, 3)).astype(np.float32)
    D = r.standard_normal((g.n, 3)).astype(np.float32)
    E_pre, E = oracle.sddmm_add(g, S, D, 0.2)
    for e, (u, v) in enumerate(edge_list(g)):
        for k in range(3):
            p = np.float32(S[u, k]) + np.float32(D[v, k])
            assert E_pre[e, k] == p
            assert E[e, k] == (p if p > 0 else np.float32(0.2) * p)


def test_sddmm_dot_brute_force():
    g, _, _ = tiny_graph(5)
    r = np.random.default_rng(5)
    A = r.standard_normal((g.n, 12)).astype(np.float32)
    B = r.standard_normal((g.n, 12)).astype(np.float32)
    out = oracle.sddmm_dot(g, A, B, 3)
    for e, (u, v) in enumerate(edge_list(g)):
        for k in range(3):
            ref = float(np.dot(A[v, 4 * k:4 * k + 4].astype(np.float64), B[u, 4 * k:4 * k + 4]))
            assert abs(out[e, k] - ref) < 1e-12


def test_edge_softmax_brute_force():
    g, _, _ = tiny_graph(6)
    r = np.random.default_rng(6)
    E = (3 * r.standard_normal((g.nnz, 2))).astype(np.float32)
    a = oracle.edge_softmax(g, E)
    el = edge_list(g)
    for v in range(g.n):
        es = [e for e, (u, vv) in enumerate(el) if vv == v]
        for k in range(2):
            assert np.allclose(a[es, k], sp_softmax(E[es, k].astype(np.float64)), rtol=1e-12)
    s = oracle.edge_reduce(g, a.astype(np.float32))
    assert np.allclose(s, 1.0, atol=1e-6)
    # uniform scores: alpha = 1 / in-degree
    a1 = oracle.edge_softmax(g, np.full((g.nnz, 1), 0.7, np.float32))
    assert np.allclose(a1[:, 0], 1.0 / g.deg[g.dst])


def test_edge_reduce_brute_force():
    g, _, _ = tiny_graph(7)
    r = np.random.default_rng(7)
    vals = r.standard_normal((g.nnz, 3)).astype(np.float32)
    by_dst = oracle.edge_reduce(g, vals, by_src=False)
    by_src = oracle.edge_reduce(g, vals, by_src=True)
    rd = np.zeros((g.n, 3))
    rs = np.zeros((g.n, 3))
    for e, (u, v) in enumerate(edge_list(g)):
        rd[v] += vals[e]
        rs[u] += vals[e]
    assert np.allclose(by_dst, rd) and np.allclose(by_src, rs)


def test_edge_softmax_bwd_finite_difference_and_zero_sum():
    g, _, _ = tiny_graph(8)
    r = np.random.default_rng(8)
    E = r.standard_normal((g.nnz, 2))
    R = r.standard_normal((g.nnz, 2))            # loss = <alpha(E), R>

    def loss(E64):
        return float(np.sum(oracle.edge_softmax(g, E64.astype(np.float32)) * R))
    a = oracle.edge_softmax(g, E.astype(np.float32)).astype(np.float32)
    dE = oracle.edge_softmax_bwd(g, a, R.astype(np.float32))
    # sum of dE over the in-edges of each destination vanishes
    assert np.allclose(oracle.edge_reduce(g, dE.astype(np.float32)), 0.0, atol=1e-6)
    dirn = r.standard_normal(E.shape)
    eps = 1e-3
    fd = (loss(E + eps * dirn) - loss(E - eps * dirn)) / (2 * eps)
    assert abs(fd - np.sum(dE * dirn)) < 2e-3 * (1 + abs(fd))


# ---------------------------------------------------------------------------
# Tango worked example (GAT running example, Fig. 1a / 1b)
# ---------------------------------------------------------------------------
def test_tango_fragment():
    fx = json.load(open(os.path.join(GOLD, "tango_gat_fragment.json")))
    tol = fx["tolerance"]
    # in-star v0 -> v3 (e3), v2 -> v3 (e4); no self-loops in the figure's fragment
    g = OracleGraph(4, np.array([0, 0, 0, 0, 2], np.int64), np.array([0, 2], np.int32), np.array([3, 3], np.int32))
    S0 = oracle.gat_scores(np.array([fx["Hp_v0"]], np.float32), np.array(fx["a_src"], np.float32), 2)[0]
    assert np.allclose(S0, fx["S_v0"], atol=tol)
    S = np.zeros((4, 2), np.float32)
    D = np.zeros((4, 2), np.float32)
    S[0] = fx["S_v0"]
    D[3] = fx["D_v3"]
    # e4's pre-activation is positive, so its printed post-activation value fixes S[v2]
    S[2] = np.array(fx["E_e4_after_activation"], np.float32) - D[3]
    E_pre, E = oracle.sddmm_add(g, S, D, 0.0)
    assert np.allclose(E_pre[0], fx["E_pre_e3"], atol=tol)
    assert np.allclose(E[0], fx["E_e3_after_activation"], atol=tol)
    alpha = oracle.edge_softmax(g, E)
    assert np.allclose(alpha[0], fx["alpha_e3"], atol=tol)
    assert np.allclose(alpha[1], fx["alpha_e4"], atol=tol)
    a_page = np.array([fx["alpha_e3"], fx["alpha_e4"]], np.float32)
    dal = np.array([[fx["dalpha_head0"]["e3"], 0.3], [fx["dalpha_head0"]["e4"], -0.2]], np.float32)
    dE = oracle.edge_softmax_bwd(g, a_page, dal)
    assert abs(dE[0, 0] - fx["dE_e3_head0"]) <= tol
    P = dal[0, 0] - dE[0, 0] / a_page[0, 0]
    assert abs(P - fx["P_v3_head0"]) <= tol
    dD = oracle.edge_reduce(g, dE.astype(np.float32))
    assert abs(dD[3, 0] - fx["dD_v3"][0]) <= tol


# ---------------------------------------------------------------------------
# GEMM wrapper and loss
# ---------------------------------------------------------------------------
def test_gemm_transposes_loops():
    r = np.random.default_rng(9)
    A = r.standard_normal((5, 3))
    B = r.standard_normal((3, 4))
    ref = np.zeros((5, 4))
    for i in range(5):
        for j in range(4):
            for k in range(3):
                ref[i, j] += A[i, k] * B[k, j]
    assert np.allclose(oracle.gemm(A, B), ref)
    assert np.allclose(oracle.gemm(A.T.copy(), B, transA=True), ref)
    assert np.allclose(oracle.gemm(A, B.T.copy(), transB=True), ref)


def test_xent_zero_logits_closed_form():
    n, c = 7, 41
    lab = np.arange(n) % c
    loss, dz = oracle.softmax_xent(np.zeros((n, c)), lab)
    assert abs(loss - np.log(c)) < 1e-15
    ref = np.full((n, c), 1.0 / c)
    ref[np.arange(n), lab] -= 1.0
    assert np.allclose(dz, ref / n, atol=1e-16)


def test_xent_finite_difference():
    r = np.random.default_rng(11)
    z = r.standard_normal((6, 5))
    lab = r.integers(0, 5, 6)
    _, dz = oracle.softmax_xent(z, lab)
    dirn = r.standard_normal(z.shape)
    eps = 1e-5
    fd = (oracle.softmax_xent(z + eps * dirn, lab)[0] - oracle.softmax_xent(z - eps * dirn, lab)[0]) / (2 * eps)
    assert abs(fd - np.sum(dz * dirn)) < 1e-8
