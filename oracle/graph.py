"""Oracle graph layer (numpy): edge list -> CSR by destination, CSC view,
GCN normalisation, degree ordering.

TEST INFRASTRUCTURE: used only by the tests, the smoke check and the CPU
baseline leg of the benchmark.  Independent of the library's graph builder.

Definitions followed
  * Sancus (IJCAI'23 extended abstract), Sec. 2 Preliminaries: the GCN
    operator is A_hat = Dbar^-1/2 Abar Dbar^-1/2 with Abar = A + I and
    Dbar = D + I, i.e. every node has one self-connection and its degree
    counts it.
  * Tango (SC'23), Evaluation, datasets paragraph: reverse edges and
    self-loops are added so that the aggregation reaches every node.
  * AdaQP (arXiv 2306.01381), Thm. 3 text: the aggregation of v includes v.
Reading: existing self-loops and repeated edges are dropped first, then one
self-loop per node is added, so Dbar_vv is exactly the row length.
"""
from __future__ import annotations

import numpy as np


class OracleGraph:
    """CSR by destination: row v holds the sources u of edges u -> v, ascending."""

    def __init__(self, n, row_ptr, col, dst_of_edge):
        self.n = int(n)
        self.row_ptr = row_ptr          # int64 [n+1]
        self.col = col                  # int32 [nnz]
        self.dst = dst_of_edge          # int32 [nnz] (row id of each CSR slot)
        self.nnz = int(col.size)
        self._csc = None
        self._norm = None

    # -- degree --------------------------------------------------------------
    @property
    def deg(self):
        return np.diff(self.row_ptr)

    # -- Sancus Sec. 2: symmetric normalisation ------------------------------
    def gcn_norm(self):
        """dinv[v] = 1/sqrt(dbar_v) and w[e] = dinv[src] * dinv[dst], binary32."""
        if self._norm is None:
            dbar = self.deg.astype(np.float32)
            dinv = (np.float32(1.0) / np.sqrt(dbar)).astype(np.float32)
            w = (dinv[self.col] * dinv[self.dst]).astype(np.float32)
            self._norm = (dinv, w)
        return self._norm

    # -- mean aggregation (GraphSAGE in AdaQP's weighted-sum form, Eqn. 1) ---
    def mean_weights(self):
        """w[e] = 1 / (row length of the edge's destination), binary32: the
        aggregation of v is the mean over {v} u N(v)."""
        inv = (np.float32(1.0) / self.deg.astype(np.float32)).astype(np.float32)
        return inv[self.dst]

    # -- transposed view -----------------------------------------------------
    def csc(self):
        """(colptr int64[n+1], row int32[nnz], eid int32[nnz]): column u lists the
        destinations v of u's out-edges ascending; eid is the CSR slot of each entry."""
        if self._csc is None:
            key = self.col.astype(np.int64) * self.n + self.dst.astype(np.int64)
            eid = np.argsort(key, kind="stable").astype(np.int32)
            row = self.dst[eid].astype(np.int32)
            colptr = np.zeros(self.n + 1, dtype=np.int64)
            colptr[1:] = np.cumsum(np.bincount(self.col, minlength=self.n))
            self._csc = (colptr, row, eid)
        return self._csc

    # -- AdaQP Eqn. 7: local and remote in-neighbour sums ------------------
    def split_by_source(self, marginal):
        """(local, remote, w_local, w_remote): the in-edges of every row whose
        source is not / is marginal, each in its CSR order, with the GCN weight
        it has in this graph (the sub-graphs' own degrees play no part)."""
        marginal = np.asarray(marginal, dtype=bool)
        _, w = self.gcn_norm()
        parts = []
        for want in (False, True):
            keep = marginal[self.col] == want
            counts = np.bincount(self.dst[keep], minlength=self.n)
            row_ptr = np.zeros(self.n + 1, dtype=np.int64)
            row_ptr[1:] = np.cumsum(counts)
            parts.append((OracleGraph(self.n, row_ptr, self.col[keep].astype(np.int32),
                                      self.dst[keep].astype(np.int32)), w[keep]))
        (lg, lw), (rg, rw) = parts
        return lg, rg, lw, rw

    # -- degree ordering -----------------------------------------------------
    def degree_perm(self):
        """Rows by in-degree descending, ties by id ascending."""
        ids = np.arange(self.n, dtype=np.int64)
        return np.lexsort((ids, -self.deg)).astype(np.int32)

    def bucket_offsets(self, thresholds, by_out=False):
        """Given descending degree thresholds t_0 > t_1 > ..., offsets into the
        degree-ordered row list where the degree first drops to <= t_i (by_out:
        the columns of the transposed view ordered by out-degree)."""
        if by_out:
            deg = np.bincount(self.col, minlength=self.n).astype(np.int64)
            ids = np.arange(self.n, dtype=np.int64)
            d_sorted = deg[np.lexsort((ids, -deg))]
        else:
            d_sorted = self.deg[self.degree_perm()]
        # d_sorted is non-increasing; count rows with degree > t
        off = [0]
        for t in thresholds:
            off.append(int(np.count_nonzero(d_sorted > t)))
        off.append(self.n)
        return np.asarray(off, dtype=np.int64)

    def dense(self, weights=None):
        """Dense [n, n] matrix with entry [v, u] = weight of edge u -> v (tiny graphs)."""
        A = np.zeros((self.n, self.n), dtype=np.float64)
        w = np.ones(self.nnz) if weights is None else np.asarray(weights, dtype=np.float64)
        A[self.dst, self.col] = w
        return A


def build_graph(src, dst, n, symmetrize: bool) -> OracleGraph:
    """Drop self-loops and repeats, optionally add every reverse edge, then add
    one self-loop per node; sort by (destination, source)."""
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    if src.size and (src.min() < 0 or dst.min() < 0 or src.max() >= n or dst.max() >= n):
        raise ValueError("node id out of range")
    keep = src != dst
    s, t = src[keep], dst[keep]
    if symmetrize:
        s, t = np.concatenate([s, t]), np.concatenate([t, s])
    loops = np.arange(n, dtype=np.int64)
    s = np.concatenate([s, loops])
    t = np.concatenate([t, loops])
    key = np.unique(t * n + s)           # sorted by destination, then source; repeats gone
    d_of_e = (key // n).astype(np.int32)
    col = (key % n).astype(np.int32)
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(np.bincount(d_of_e, minlength=n))
    return OracleGraph(n, row_ptr, col, d_of_e)
