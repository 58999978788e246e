"""Pins of the oracle's graph layer against brute force on tiny graphs and
against closed forms of the GCN operator (Sancus, Sec. 2 Preliminaries)."""
import numpy as np
import pytest

import oracle
from oracle.graph import OracleGraph, build_graph


def brute_in_sets(src, dst, n, symmetrize):
    """Adjacency by Python sets: the in-neighbour set of every node, self included."""
    ins = [set([v]) for v in range(n)]
    for u, v in zip(src.tolist(), dst.tolist()):
        if u == v:
            continue
        ins[v].add(u)
        if symmetrize:
            ins[u].add(v)
    return ins


@pytest.mark.parametrize("symmetrize", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_csr_matches_brute_force(symmetrize, seed):
    g0 = np.random.default_rng(seed)
    n = int(g0.integers(1, 40))
    m = int(g0.integers(0, 4 * n))
    src = g0.integers(0, n, m).astype(np.int32)
    dst = g0.integers(0, n, m).astype(np.int32)
    # plant self-loops and repeats
    if m:
        src[: m // 5] = dst[: m // 5]
        src = np.concatenate([src, src[: m // 3]])
        dst = np.concatenate([dst, dst[: m // 3]])
    g = build_graph(src, dst, n, symmetrize)
    ins = brute_in_sets(src, dst, n, symmetrize)
    assert g.row_ptr[0] == 0 and g.row_ptr[-1] == g.nnz
    for v in range(n):
        row = g.col[g.row_ptr[v]:g.row_ptr[v + 1]].tolist()
        assert row == sorted(ins[v]), v
        assert np.all(g.dst[g.row_ptr[v]:g.row_ptr[v + 1]] == v)


def test_empty_and_isolated():
    g = build_graph(np.zeros(0, np.int32), np.zeros(0, np.int32), 5, True)
    assert g.nnz == 5
    assert g.col.tolist() == [0, 1, 2, 3, 4]
    dinv, w = g.gcn_norm()
    assert np.all(dinv == 1.0) and np.all(w == 1.0)


def test_bad_ids_rejected():
    with pytest.raises(ValueError):
        build_graph(np.array([0, 5], np.int32), np.array([1, 1], np.int32), 5, False)


@pytest.mark.parametrize("seed", [3, 4])
def test_csc_is_exact_transpose(seed):
    g0 = np.random.default_rng(seed)
    n = 50
    src = g0.integers(0, n, 300).astype(np.int32)
    dst = g0.integers(0, n, 300).astype(np.int32)
    g = build_graph(src, dst, n, False)
    colptr, row, eid = g.csc()
    assert sorted(eid.tolist()) == list(range(g.nnz))
    for u in range(n):
        rows = row[colptr[u]:colptr[u + 1]]
        assert np.all(np.diff(rows) > 0)
        for i in range(colptr[u], colptr[u + 1]):
            e = eid[i]
            assert g.col[e] == u and g.dst[e] == row[i]


def test_degree_perm_and_buckets():
    g0 = np.random.default_rng(7)
    n = 200
    src = g0.integers(0, n, 1500).astype(np.int32)
    dst = (g0.integers(0, n, 1500) % 37).astype(np.int32)  # skew in-degrees
    g = build_graph(src, dst, n, False)
    perm = g.degree_perm()
    assert sorted(perm.tolist()) == list(range(n))
    d = g.deg[perm]
    assert np.all(np.diff(d) <= 0)
    for i in range(n - 1):
        if d[i] == d[i + 1]:
            assert perm[i] < perm[i + 1]
    off = g.bucket_offsets([32, 8, 2])
    assert off[0] == 0 and off[-1] == n and np.all(np.diff(off) >= 0)
    for b, (lo, hi) in enumerate(zip(off[:-1], off[1:])):
        upper = np.inf if b == 0 else [32, 8, 2][b - 1]
        lower = [32, 8, 2][b] if b < 3 else -1
        assert np.all((d[lo:hi] <= upper) & (d[lo:hi] > lower))


def test_out_degree_buckets_brute_force():
    # out-degree buckets of the transposed view, counted edge by edge
    g0 = np.random.default_rng(8)
    n = 150
    src = (g0.integers(0, n, 2000) % 23).astype(np.int32)  # skew out-degrees
    dst = g0.integers(0, n, 2000).astype(np.int32)
    g = build_graph(src, dst, n, False)
    outdeg = [0] * n
    for u in g.col.tolist():
        outdeg[u] += 1
    th = [60, 20, 1]
    want = [0] + [sum(1 for x in outdeg if x > t) for t in th] + [n]
    assert g.bucket_offsets(th, by_out=True).tolist() == want
    assert g.bucket_offsets(th).tolist() == [0] + [int(np.sum(g.deg > t)) for t in th] + [n]


def _ring(n):
    s = np.arange(n, dtype=np.int32)
    return s, (s + 1) % n


@pytest.mark.parametrize("n", [3, 10, 17])
def test_gcn_norm_regular_graphs_row_sums(n):
    # ring: every node has 2 neighbours + self -> dbar = 3, A_hat rows sum to 1
    s, t = _ring(n)
    g = build_graph(s, t, n, True)
    dinv, w = g.gcn_norm()
    assert np.all(g.deg == 3)
    rs = oracle.spmm(g, np.ones((n, 1), np.float32), w)
    assert np.allclose(rs, 1.0, rtol=0, atol=1e-6)
    # complete graph K_n: dbar = n
    uu, vv = np.triu_indices(n, 1)
    g = build_graph(uu.astype(np.int32), vv.astype(np.int32), n, True)
    dinv, w = g.gcn_norm()
    assert np.all(g.deg == n)
    rs = oracle.spmm(g, np.ones((n, 1), np.float32), w)
    assert np.allclose(rs, 1.0, rtol=0, atol=1e-6)


@pytest.mark.parametrize("seed", [0, 1])
def test_gcn_norm_eigenvector(seed):
    # A_hat sqrt(dbar) = Dbar^-1/2 Abar 1 = Dbar^-1/2 dbar = sqrt(dbar)
    g0 = np.random.default_rng(seed)
    n = 300
    g = build_graph(g0.integers(0, n, 2000).astype(np.int32), g0.integers(0, n, 2000).astype(np.int32), n, True)
    _, w = g.gcn_norm()
    sq = np.sqrt(g.deg.astype(np.float64))
    y = oracle.spmm(g, sq[:, None].astype(np.float32), w)[:, 0]
    assert np.allclose(y, sq, rtol=2e-6)


def test_gcn_norm_dense_matches_definition():
    # Dbar^-1/2 Abar Dbar^-1/2 built densely from the brute-force adjacency
    g0 = np.random.default_rng(5)
    n = 30
    src = g0.integers(0, n, 80).astype(np.int32)
    dst = g0.integers(0, n, 80).astype(np.int32)
    g = build_graph(src, dst, n, True)
    ins = brute_in_sets(src, dst, n, True)
    Abar = np.zeros((n, n))
    for v in range(n):
        for u in ins[v]:
            Abar[v, u] = 1.0
    Dm = np.diag(Abar.sum(1) ** -0.5)
    Ahat = Dm @ Abar @ Dm
    _, w = g.gcn_norm()
    assert np.allclose(g.dense(w), Ahat, rtol=1e-6, atol=0)


@pytest.mark.parametrize("frac", [0.0, 0.3, 1.0])
def test_split_by_source_partitions_the_edges(frac):
    # AdaQP Eqn. 7: every in-edge is local or remote by its source, each keeps
    # its weight in A_hat, and the two sums add up to the whole aggregation
    r = np.random.default_rng(31)
    n = 400
    src, dst = r.integers(0, n, 3000), r.integers(0, n, 3000)
    g = build_graph(src, dst, n, True)
    marginal = r.random(n) < frac
    lg, rg, lw, rw = g.split_by_source(marginal)
    assert lg.nnz + rg.nnz == g.nnz
    assert not marginal[lg.col].any() and marginal[rg.col].all()
    # the parent's edges, regrouped: same (dst, src, weight) triples per row, order kept
    _, w = g.gcn_norm()
    for v in range(0, n, 7):
        row = g.col[g.row_ptr[v]:g.row_ptr[v + 1]]
        wv = w[g.row_ptr[v]:g.row_ptr[v + 1]]
        m = marginal[row]
        assert np.array_equal(lg.col[lg.row_ptr[v]:lg.row_ptr[v + 1]], row[~m])
        assert np.array_equal(rg.col[rg.row_ptr[v]:rg.row_ptr[v + 1]], row[m])
        assert np.array_equal(lw[lg.row_ptr[v]:lg.row_ptr[v + 1]], wv[~m])
        assert np.array_equal(rw[rg.row_ptr[v]:rg.row_ptr[v + 1]], wv[m])
    # linearity against the dense operator
    X = r.standard_normal((n, 5))
    A = g.dense(w).astype(np.float64)
    Y = oracle.spmm(lg, X, lw) + oracle.spmm(rg, X, rw)
    assert np.allclose(Y, A @ X, rtol=1e-12, atol=1e-12)


def test_mean_weights_against_brute_force():
    # GraphSAGE mean: row v of the aggregation is the average of the rows of
    # {v} u N(v), by Python sets on a tiny directed graph
    r = np.random.default_rng(41)
    n = 60
    src, dst = r.integers(0, n, 400), r.integers(0, n, 400)
    g = build_graph(src, dst, n, False)
    ins = brute_in_sets(src, dst, n, False)
    X = r.standard_normal((n, 3))
    Y = oracle.spmm(g, X, g.mean_weights())
    for v in range(n):
        nb = sorted(ins[v])
        assert np.allclose(Y[v], X[nb].mean(axis=0), rtol=1e-6, atol=1e-7)
    # every row's weights sum to 1 within the rounding of 1/len
    sums = np.add.reduceat(g.mean_weights().astype(np.float64), g.row_ptr[:-1])
    assert np.all(np.abs(sums - 1.0) <= g.deg * 2.0 ** -24)
