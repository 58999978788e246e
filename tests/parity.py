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
