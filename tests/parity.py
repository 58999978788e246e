"""Shared helpers of the GPU parity tests: seeded graphs, transfers and the
tolerance rule.

Tolerance (floating point): a reduction output r (a sum of terms t_i) is
accepted when |gpu - r| <= rtol * M with M = sum |t_i| computed by the
oracle on absolute values; binary32 accumulation gives rtol = 1e-4 (an
error of that size needs ~1000 ulps of cancellation-free drift).  A
bfloat16 store adds at most half an ulp of bf16: with 8 significant bits
that is at most 2^-8 |r| (the bound at r just above a power of two), which
the check allows on top (2e-2 * M is the bf16 bar; the accumulation is still
binary32).
Integer, index and code outputs are compared for equality.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.graph import build_graph
from sparse_message_passing_amd import gnnmp, synth

RTOL32 = 1e-4
RTOL16 = 2e-2


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def from_dev(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def graph_pair(src, dst, n, symmetrize, csc=True):
    """(library graph, oracle graph) from one raw edge list."""
    g = gnnmp.gnn_graph_create(n, src, dst, symmetrize=symmetrize, csc=csc)
    og = build_graph(src, dst, n, symmetrize)
    return g, og


def hub_edges(n, m, hub_in, seed, hub=0):
    """Uniform random edges plus one hub with `hub_in` distinct in-neighbours
    (and, once symmetrised, as many out-neighbours)."""
    r = np.random.default_rng(seed)
    src = r.integers(0, n, m).astype(np.int32)
    dst = r.integers(0, n, m).astype(np.int32)
    hs = r.choice(np.setdiff1d(np.arange(n), [hub]), size=hub_in, replace=False).astype(np.int32)
    return np.concatenate([src, hs]), np.concatenate([dst, np.full(hub_in, hub, np.int32)])


def rmat_graph(scale, avg_deg, symmetric, seed):
    n = 1 << scale
    m = avg_deg * n // (2 if symmetric else 1)
    s, d = synth.rmat_edges(scale, m, seed)
    return s, d, n


def check_close(gpu, ref, mag, rtol=RTOL32, bf16_out=False, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    mag = np.asarray(mag, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    tol = rtol * mag + (2.0 ** -8) * np.abs(ref) * (1 if bf16_out else 0) + 1e-30
    err = np.abs(gpu - ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r} mag={mag[i]!r} tol={tol[i]!r}")


def bf16_values(a):
    """float32 array holding the bfloat16 rounding of a (what a bf16 tensor stores)."""
    return oracle.to_bf16(a)


def sub_rows(og, rows):
    """Oracle graph restricted to the listed destination rows (same column ids)
    and the CSR slots of its edges in the full graph."""
    rows = np.asarray(rows, np.int64)
    lens = og.row_ptr[rows + 1] - og.row_ptr[rows]
    rp = np.zeros(rows.size + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    eids = np.concatenate([np.arange(og.row_ptr[v], og.row_ptr[v + 1]) for v in rows]) if rows.size else np.zeros(0, np.int64)
    dst = np.repeat(rows.astype(np.int32), lens)
    return oracle.OracleGraph(rows.size, rp, og.col[eids].astype(np.int32), dst), eids


def saved_alpha(og, S, D, M, Z, slope, eids=None):
    """The attention weights a GAT forward leaves implied by its saved per-node
    S, D and per-destination M, Z (device tensors): alpha[e] =
    exp(LReLU(S[src] + D[dst]) - M[dst]) * Z[dst] in float64 from the binary32
    score sum (the edges eids of og, or all of them)."""
    S, D, M, Z = (from_dev(t) for t in (S, D, M, Z))
    col, dst = (og.col, og.dst) if eids is None else (og.col[eids], og.dst[eids])
    E = S[col] + D[dst]                       # one binary32 add, as the kernels
    E = np.where(E > 0, E, np.float32(slope) * E).astype(np.float64)
    return np.exp(E - M[dst].astype(np.float64)) * Z[dst].astype(np.float64)


def softmax_row_stats(og, E):
    """Per destination row and head, the maximum M of the scores E over the
    row's in-edges and Z = 1 / sum exp(E - M) (float64; rows without in-edges
    get M = -inf, Z = inf), so that alpha = exp(E - M[dst]) * Z[dst]."""
    E = np.asarray(E, np.float64)
    n, h = og.n, E.shape[1]
    deg = np.diff(og.row_ptr)
    M = np.full((n, h), -np.inf)
    has = deg > 0
    if og.nnz:
        M[has] = np.maximum.reduceat(E, og.row_ptr[:-1][has], axis=0)
    row = np.repeat(np.arange(n), deg)  # CSR row of each edge slot
    ex = np.exp(E - M[row])
    s = np.zeros((n, h))
    np.add.at(s, row, ex)
    with np.errstate(divide="ignore"):
        Z = 1.0 / s
    return M, Z



def check_gcn_stack_step(og, st, Ws, labels, dt, rows=None, log=print):
    """Element-by-element parity of one GcnStack step (forward, loss, backward)
    the way the library chains it, layer by layer: each layer's outputs are
    compared with the oracle's layer applied to the GPU's own inputs of that
    layer (the activation, the saved aggregate, the upstream gradient), so
    every ReLU decision is shared and every check covers one layer's
    rounding.  The backward of layer i > 0 returns its input gradient times
    [H_i > 0] (the previous layer's ReLU derivative, fused).  rows: check the
    row-valued outputs on these rows only (None: every row), with the graph
    symmetrised (A_hat^T restricted to rows is then A_hat's rows); the weight
    gradients and the loss are always checked in full."""
    rtol = RTOL16 if dt == "bf16" else RTOL32
    bf = dt == "bf16"
    L = len(Ws)
    H = [from_dev(h) for h in st.H]
    w = og.gcn_norm()[1]
    wa = np.abs(w)
    if rows is None:
        sel = lambda a: a
        loc, need, wl = og, np.arange(og.n), w          # the rows' in-edge graph and the sources it reads
        aggT_mag = lambda M: oracle.spmm(og, M, wa, transpose=True)
    else:
        sg, eids = sub_rows(og, rows)
        need = np.unique(sg.col).astype(np.int64)
        loc = oracle.OracleGraph(sg.n, sg.row_ptr, np.searchsorted(need, sg.col).astype(np.int32), sg.dst)
        wl = w[eids]
        sel = lambda a: a[rows]
        aggT_mag = lambda M: oracle.spmm(loc, M[need], np.abs(wl))
    for i in range(L):
        last = i == L - 1
        out_dt = "f32" if last else dt
        W = np.asarray(Ws[i], np.float64)
        d_in, d_out = W.shape
        Xn = H[i][need].astype(np.float64)
        if d_out <= d_in:                            # Z = X W (stored), Y = sigma(A_hat Z)
            A = oracle.spmm(loc, oracle.store(Xn @ W, dt), wl)
        else:                                        # saved = A_hat X (stored), Y = sigma(saved W)
            saved_ref = oracle.store(oracle.spmm(loc, Xn, wl), dt)
            sv = sel(from_dev(st.saved[i]))
            check_close(sv, saved_ref, oracle.spmm(loc, np.abs(Xn), np.abs(wl)), rtol=rtol, bf16_out=bf,
                        what=f"step layer {i} saved A_hat X")
            A = sv.astype(np.float64) @ W            # the GEMM reads the GPU's own saved aggregate
        Y_ref = oracle.store(A if last else np.maximum(A, 0.0), out_dt)
        check_close(sel(H[i + 1]), Y_ref, oracle.spmm(loc, np.abs(Xn) @ np.abs(W), np.abs(wl)), rtol=rtol,
                    bf16_out=bf and not last, what=f"step layer {i} forward")
        log(f"step layer {i} forward checked")
    loss_ref, dz_ref = oracle.softmax_xent(H[L], labels)
    n = og.n
    assert abs(float(st.loss.item()) - loss_ref) <= RTOL32 * (abs(loss_ref) + np.abs(H[L]).max()), "step loss"
    check_close(from_dev(st.dlogits), dz_ref, np.abs(dz_ref) + 2.0 / n, what="step loss gradient")
    U = from_dev(st.dlogits)
    for i in reversed(range(L)):
        W = np.asarray(Ws[i], np.float64)
        d_in, d_out = W.shape
        saved = from_dev(st.saved[i]) if st.saved[i] is not None else None
        dX_ref, dW_ref = oracle.gcn_layer_bwd(og, H[i], saved, H[i + 1], U, Ws[i], relu=False, need_dX=i > 0,
                                              dt=dt)
        Ga = np.abs(U).astype(np.float64)
        if d_out <= d_in:                            # dZ = A_hat^T G, dW = X^T dZ, dX = dZ W^T
            MdZ = oracle.spmm(og, Ga, wa, transpose=True)
            m_dW = np.abs(H[i]).T.astype(np.float64) @ MdZ
            m_dX = lambda: sel(MdZ) @ np.abs(W).T
        else:                                        # dW = (A_hat X)^T G, dX = A_hat^T (G W^T)
            m_dW = np.abs(saved).T.astype(np.float64) @ Ga
            m_dX = lambda: aggT_mag(Ga @ np.abs(W).T)
        check_close(from_dev(st.dW[i]), dW_ref, m_dW, rtol=rtol, what=f"step layer {i} dW")
        if i > 0:
            keep = sel(H[i] > 0)
            check_close(sel(from_dev(st.dH[i])), np.where(keep, sel(dX_ref), 0.0), np.where(keep, m_dX(), 0.0),
                        rtol=rtol, bf16_out=bf, what=f"step layer {i} dX (times the ReLU derivative)")
            U = from_dev(st.dH[i])
        log(f"step layer {i} backward checked")
