"""Pins of the oracle's layer compositions: dense closed forms for the
forward passes and central finite differences for every backward formula."""
import numpy as np
import pytest

import oracle
from oracle.graph import build_graph


def graph(seed, n=20, m=60, sym=True):
    r = np.random.default_rng(seed)
    return build_graph(r.integers(0, n, m).astype(np.int32), r.integers(0, n, m).astype(np.int32), n, sym)


def fd_check(f, x, grad, seed, eps=1e-6, rtol=1e-6):
    """Directional derivative of scalar f at x along a random unit direction vs
    <grad, dir>, in the oracle's unrounded float64 mode (a step this small
    crosses no ReLU / LeakyReLU kink for these seeds)."""
    r = np.random.default_rng(seed)
    d = r.standard_normal(x.shape)
    d /= np.linalg.norm(d)
    fd = (f(x + eps * d) - f(x - eps * d)) / (2 * eps)
    an = float(np.sum(np.asarray(grad, np.float64) * d))
    assert abs(fd - an) <= rtol * (abs(an) + np.linalg.norm(grad) * 1e-2), (fd, an)


@pytest.mark.parametrize("d_in,d_out", [(8, 8), (6, 10), (10, 3)])
def test_gcn_fwd_dense(d_in, d_out):
    g = graph(0)
    r = np.random.default_rng(1)
    X = r.standard_normal((g.n, d_in)).astype(np.float32)
    W = r.standard_normal((d_in, d_out)).astype(np.float32)
    _, w = g.gcn_norm()
    Ah = g.dense(w)
    Y, _ = oracle.gcn_layer_fwd(g, X, W, relu=True)
    ref = np.maximum(Ah @ X.astype(np.float64) @ W, 0)
    assert np.allclose(Y, ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("sym", [True, False], ids=["symmetrised", "directed"])
@pytest.mark.parametrize("d_in,d_out,relu", [(8, 8, True), (6, 10, True), (10, 3, False), (5, 9, False)])
def test_gcn_bwd_finite_difference(d_in, d_out, relu, sym):
    # on a directed graph A_hat is not symmetric: the backward must apply A_hat^T
    g = graph(2, sym=sym)
    r = np.random.default_rng(3)
    X = r.standard_normal((g.n, d_in))
    W = r.standard_normal((d_in, d_out))
    R = r.standard_normal((g.n, d_out))

    def fX(Xv):
        return float(np.sum(oracle.gcn_layer_fwd(g, Xv, W, relu, dt="f64")[0] * R))

    def fW(Wv):
        return float(np.sum(oracle.gcn_layer_fwd(g, X, Wv, relu, dt="f64")[0] * R))
    Y, saved = oracle.gcn_layer_fwd(g, X, W, relu, dt="f64")
    dX, dW = oracle.gcn_layer_bwd(g, X, saved, Y, R, W, relu, dt="f64")
    fd_check(fX, X, dX, 4)
    fd_check(fW, W, dW, 5)


def test_gcn_three_layer_step_finite_difference():
    g = graph(6, n=30, m=90)
    r = np.random.default_rng(7)
    X = r.standard_normal((g.n, 6))
    Ws = [r.standard_normal(s) * 0.5 for s in [(6, 8), (8, 8), (8, 4)]]
    lab = r.integers(0, 4, g.n)
    out = oracle.gcn_forward_backward(g, X, Ws, lab, dt="f64")
    for li in range(3):
        def f(Wl, li=li):
            Wc = list(Ws)
            Wc[li] = Wl
            return oracle.gcn_forward_backward(g, X, Wc, lab, dt="f64")["loss"]
        fd_check(f, Ws[li], out["dW"][li], 10 + li)


def test_gat_fwd_dense_and_mean_special_case():
    g = graph(8, n=16, m=50, sym=False)
    r = np.random.default_rng(9)
    h, dh = 2, 4
    X = r.standard_normal((g.n, 6)).astype(np.float32)
    W = r.standard_normal((6, h * dh)).astype(np.float32)
    a_s = r.standard_normal((h, dh)).astype(np.float32)
    a_d = r.standard_normal((h, dh)).astype(np.float32)
    fw = oracle.gat_layer_fwd(g, X, W, a_s, a_d, h, 0.2)
    Hp = X.astype(np.float64) @ W
    for k in range(h):
        S = Hp[:, k * dh:(k + 1) * dh] @ a_s[k]
        D = Hp[:, k * dh:(k + 1) * dh] @ a_d[k]
        logits = np.full((g.n, g.n), -np.inf)
        A = g.dense() > 0
        pre = D[:, None] + S[None, :]               # [dst, src]
        logits[A] = np.where(pre > 0, pre, 0.2 * pre)[A]
        att = np.exp(logits - logits.max(1, keepdims=True))
        att /= att.sum(1, keepdims=True)
        assert np.allclose(fw["Y"][:, k * dh:(k + 1) * dh], att @ Hp[:, k * dh:(k + 1) * dh], rtol=1e-4, atol=1e-5)
    # a_src = a_dst = 0 -> alpha = 1/indeg -> mean aggregation
    z = np.zeros((h, dh), np.float32)
    fw0 = oracle.gat_layer_fwd(g, X, W, z, z, h, 0.2)
    mean = (g.dense() @ Hp) / g.deg[:, None]
    assert np.allclose(fw0["Y"], mean, rtol=1e-5, atol=1e-5)


def test_gat_bwd_finite_difference():
    g = graph(10, n=14, m=40, sym=False)
    r = np.random.default_rng(11)
    h, dh, din = 2, 3, 5
    X = r.standard_normal((g.n, din))
    W = r.standard_normal((din, h * dh))
    a_s = r.standard_normal((h, dh))
    a_d = r.standard_normal((h, dh))
    dY = r.standard_normal((g.n, h * dh))
    def L(Xv=X, Wv=W, asv=a_s, adv=a_d):
        return float(np.sum(oracle.gat_layer_fwd(g, Xv, Wv, asv, adv, h, 0.2, dt="f64")["Y"] * dY))
    fw = oracle.gat_layer_fwd(g, X, W, a_s, a_d, h, 0.2, dt="f64")
    bw = oracle.gat_layer_bwd(g, fw, X, W, a_s, a_d, dY, h, 0.2, dt="f64")
    fd_check(lambda v: L(Xv=v), X, bw["dX"], 1)
    fd_check(lambda v: L(Wv=v), W, bw["dW"], 2)
    fd_check(lambda v: L(asv=v), a_s, bw["da_src"], 3)
    fd_check(lambda v: L(adv=v), a_d, bw["da_dst"], 4)
    # the softmax gradient sums to zero over each destination's in-edges
    assert np.allclose(oracle.edge_reduce(g, bw["dE"]), 0.0, atol=1e-12)


def test_gat_softmax_term_is_row_product_and_row_stats_rebuild_alpha():
    # The GPU backward takes the softmax backward's per-destination term
    # P[v] = sum_in alpha dalpha as <dY[v], Y[v]> per head (Y[v] = sum_in
    # alpha H'[u]) and forms alpha again from each row's maximum and 1/sum;
    # both against the oracle's edge-sum order, in float64.
    from parity import softmax_row_stats
    g = graph(12, n=30, m=120, sym=False)
    r = np.random.default_rng(13)
    h, dh, din = 4, 3, 5
    X = r.standard_normal((g.n, din))
    W = r.standard_normal((din, h * dh))
    a_s = r.standard_normal((h, dh))
    a_d = r.standard_normal((h, dh))
    dY = r.standard_normal((g.n, h * dh))
    fw = oracle.gat_layer_fwd(g, X, W, a_s, a_d, h, 0.2, dt="f64")
    bw = oracle.gat_layer_bwd(g, fw, X, W, a_s, a_d, dY, h, 0.2, dt="f64")
    P_edges = oracle.edge_reduce(g, fw["alpha"] * bw["dalpha"])
    P_rows = np.einsum("nkj,nkj->nk", dY.reshape(g.n, h, dh), fw["Y"].reshape(g.n, h, dh))
    assert np.allclose(P_rows, P_edges, rtol=1e-12, atol=1e-12)
    M, Z = softmax_row_stats(g, fw["E"])
    assert np.array_equal(M[g.dst], np.maximum(M[g.dst], fw["E"]))  # M bounds every in-edge score
    assert np.allclose(np.exp(fw["E"] - M[g.dst]) * Z[g.dst], fw["alpha"], rtol=1e-12, atol=0)


def test_bf16_rounding_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9, -2.5, 0.0], np.float32)
    y = oracle.to_bf16(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-9 rounds up
    assert y.tolist() == [1.0, 1.0, 1.0 + 2 ** -7, 1.0, -2.5, 0.0]


def test_bf16_rounding_against_torch_and_nan():
    """The store rounding against torch's CPU conversion to bfloat16 (a
    library round-to-nearest-even) on random bit patterns of every exponent,
    ties, the largest finite values and infinities; NaNs (which torch turns
    into one canonical NaN) must stay NaNs of their sign, also those whose
    payload lies only in the low 16 bits."""
    import torch
    r = np.random.default_rng(31)
    bits = r.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000, 0x3F808000, 0x3F818000,
                        0x3F80FFFF, 0x7F7FFFFF, 0x7F7F7FFF, 0x7F7F8000, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
                        0x7F800001, 0xFF800001, 0x7F80FFFF, 0x7FC00000, 0xFFFFFFFF, 0x7F807FFF], np.uint32)
    bits = np.concatenate([special, bits])
    x = bits.view(np.float32)
    got = oracle.to_bf16(x)
    nan = np.isnan(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(np.signbit(got[nan]), np.signbit(x[nan]))
    assert np.all(got.view(np.uint32) & 0xFFFF == 0)
    assert oracle.to_bf16(np.array([0x7F800001], np.uint32).view(np.float32)).view(np.uint32)[0] == 0x7FC00000


@pytest.mark.parametrize("d_in,d_out,relu", [(8, 8, True), (6, 10, True), (10, 3, False)])
def test_sage_fwd_dense_and_bwd_finite_difference(d_in, d_out, relu):
    # forward against D^-1 A dense on a directed graph (M is not symmetric),
    # backward against finite differences
    g = graph(12, sym=False)
    r = np.random.default_rng(13)
    X = r.standard_normal((g.n, d_in))
    W = r.standard_normal((d_in, d_out))
    R = r.standard_normal((g.n, d_out))
    M = g.dense(g.mean_weights())
    Y, saved = oracle.sage_layer_fwd(g, X, W, relu, dt="f64")
    P = M @ X @ W
    assert np.allclose(Y, np.maximum(P, 0) if relu else P, rtol=1e-6, atol=1e-6)

    def fX(Xv):
        return float(np.sum(oracle.sage_layer_fwd(g, Xv, W, relu, dt="f64")[0] * R))

    def fW(Wv):
        return float(np.sum(oracle.sage_layer_fwd(g, X, Wv, relu, dt="f64")[0] * R))
    dX, dW = oracle.sage_layer_bwd(g, X, saved, Y, R, W, relu, dt="f64")
    fd_check(fX, X, dX, 14)
    fd_check(fW, W, dW, 15)
