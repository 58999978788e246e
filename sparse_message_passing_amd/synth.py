"""Seeded synthetic inputs shaped like the workloads of the GNN pages.

This module only draws random numbers: edge lists, dense feature matrices,
weights, labels and index lists.  It holds none of the message-passing
arithmetic (no graph build, no normalisation, no aggregation): the library and
the CPU oracle each turn these raw inputs into their own data structures.

Recipes (all numpy ``Generator(PCG64(seed))``):

* ``gnm_pairs``    -- G(n, m): m distinct unordered non-loop pairs, uniform.
* ``rmat_edges``   -- R-MAT (Chakrabarti et al. 2004) with quadrant
  probabilities (a, b, c, d); one quadrant choice per bit level, no noise and
  no vertex relabelling.  Each level draws a 16-bit uniform, so the quadrant
  probabilities are quantised to multiples of 2^-16.
* ``chung_lu_pairs`` -- Chung-Lu: endpoints drawn independently with
  probability proportional to w_i = (i+1)^-eta, eta solved so that the
  expected degree of node 0 over the mean expected degree hits a target
  (a heavy-tailed graph with a single ~17K hub, like ogbn-products).
* features ~ N(0, 1) (float32), Glorot-uniform weights, uniform labels.

Workload k uses seed 1000*k + {1 graph, 2 features, 3 weights, 4 labels or
upstream gradient, 5 marginal rows}; the Philox seed of the quantiser is
1000*k + 6.
"""
from __future__ import annotations

import os
import numpy as np

__all__ = [
    "rng", "gnm_pairs", "rmat_edges", "chung_lu_pairs", "normal", "glorot",
    "labels", "marginal_rows", "random_bits", "WORKLOADS", "workload_inputs",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def gnm_pairs(n: int, m: int, seed: int):
    """m distinct unordered pairs {u, v}, u != v, uniform over all such pairs."""
    g = rng(seed)
    have = np.empty(0, dtype=np.int64)
    while have.size < m:
        need = (m - have.size) * 2 + 16
        u = g.integers(0, n, need, dtype=np.int64)
        v = g.integers(0, n, need, dtype=np.int64)
        keep = u != v
        lo = np.minimum(u, v)[keep]
        hi = np.maximum(u, v)[keep]
        key = lo * n + hi
        # keep first occurrences in draw order so the result is a pure function of the seed
        allk = np.concatenate([have, key])
        _, first = np.unique(allk, return_index=True)
        have = allk[np.sort(first)]
    have = have[:m]
    return (have // n).astype(np.int32), (have % n).astype(np.int32)


def _uniform16(g: np.random.Generator, size: int) -> np.ndarray:
    return np.frombuffer(g.bytes(2 * size), dtype=np.uint16)


def rmat_edges(scale: int, n_edges: int, seed: int, a=0.57, b=0.19, c=0.19):
    """R-MAT edge list (src, dst) over 2**scale nodes; may contain loops and repeats."""
    g = rng(seed)
    ta = int(round(a * 65536))
    tb = int(round((a + b) * 65536))
    tc = int(round((a + b + c) * 65536))
    src = np.zeros(n_edges, dtype=np.int32)
    dst = np.zeros(n_edges, dtype=np.int32)
    for _ in range(scale):
        r = _uniform16(g, n_edges)
        src_bit = r >= tb
        dst_bit = ((r >= ta) & (r < tb)) | (r >= tc)
        src <<= 1
        dst <<= 1
        src |= src_bit
        dst |= dst_bit
    return src, dst


def _chung_lu_eta(n: int, max_over_mean: float) -> float:
    i = np.arange(1, n + 1, dtype=np.float64)
    lo, hi = 0.0, 1.5
    for _ in range(80):
        eta = 0.5 * (lo + hi)
        ratio = 1.0 / np.mean(i ** -eta)  # w_0 / mean(w) with w_i = (i+1)^-eta
        if ratio < max_over_mean:
            lo = eta
        else:
            hi = eta
    return 0.5 * (lo + hi)


def chung_lu_pairs(n: int, n_pairs: int, max_deg: float, mean_deg: float, seed: int,
                   chunk: int = 1 << 24):
    """n_pairs endpoint pairs drawn independently, each endpoint ~ w_i = (i+1)^-eta."""
    eta = _chung_lu_eta(n, max_deg / mean_deg)
    w = np.arange(1, n + 1, dtype=np.float64) ** -eta
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    g = rng(seed)
    src = np.empty(n_pairs, dtype=np.int32)
    dst = np.empty(n_pairs, dtype=np.int32)
    for s in range(0, n_pairs, chunk):
        e = min(n_pairs, s + chunk)
        src[s:e] = np.minimum(np.searchsorted(cdf, g.random(e - s), side="right"), n - 1)
        dst[s:e] = np.minimum(np.searchsorted(cdf, g.random(e - s), side="right"), n - 1)
    return src, dst


def normal(shape, seed: int) -> np.ndarray:
    return rng(seed).standard_normal(shape, dtype=np.float32)


def glorot(fan_in: int, fan_out: int, seed: int, shape=None) -> np.ndarray:
    lim = np.sqrt(6.0 / (fan_in + fan_out))
    shape = (fan_in, fan_out) if shape is None else shape
    return rng(seed).uniform(-lim, lim, shape).astype(np.float32)


def labels(n: int, c: int, seed: int) -> np.ndarray:
    return rng(seed).integers(0, c, n, dtype=np.int32)


def marginal_rows(n: int, frac: float, seed: int) -> np.ndarray:
    """round(frac*n) distinct node ids, ascending."""
    m = int(round(frac * n))
    return np.sort(rng(seed).permutation(n)[:m]).astype(np.int32)


def random_bits(m: int, choices, seed: int) -> np.ndarray:
    """Per-row bit-width drawn uniformly from ``choices`` (uniform bit-width sampling)."""
    return np.asarray(choices, dtype=np.int32)[rng(seed).integers(0, len(choices), m)]


# ---------------------------------------------------------------------------
# The five workloads.  ``scale_down`` shrinks node and edge counts (same
# generator, same degree) for parity tests the oracle finishes in seconds.
# ---------------------------------------------------------------------------
WORKLOADS = {
    1: dict(name="gcn1-gnm1k", kind="gcn", graph="gnm", n=1000, pairs=5000,
            symmetric=True, widths=[64, 64], relu_last=True, dtype="f32"),
    2: dict(name="gcn3-rmat20", kind="gcn", graph="rmat", scale=20, avg_deg=16,
            symmetric=True, widths=[128, 256, 256, 41], dtype="f32"),
    3: dict(name="gat1-rmat21", kind="gat", graph="rmat", scale=21, avg_deg=20,
            symmetric=False, d_in=256, heads=4, d_head=64, slope=0.2, dtype="f32"),
    4: dict(name="gcn3-chunglu2.45m-bf16", kind="gcn", graph="chunglu", n=2_450_000,
            pairs=62_000_000, max_deg=17_000, symmetric=True,
            widths=[100, 256, 256, 47], dtype="bf16"),
    5: dict(name="quant-rmat20", kind="quant", graph="rmat", scale=20, avg_deg=24,
            symmetric=True, d=256, marginal_frac=0.3, dtype="f32"),
}


def workload_graph(k: int, scale_down: int = 0):
    """Raw edge list (src, dst, n) of workload k.  ``scale_down`` halves the node
    count that many times, keeping the average degree."""
    cfg = WORKLOADS[k]
    seed = 1000 * k + 1
    if cfg["graph"] == "gnm":
        n = cfg["n"] >> scale_down
        m = cfg["pairs"] >> scale_down
        s, d = gnm_pairs(n, m, seed)
    elif cfg["graph"] == "rmat":
        sc = cfg["scale"] - scale_down
        n = 1 << sc
        # undirected configs draw avg_deg*n/2 pairs (each becomes two directed edges)
        m = cfg["avg_deg"] * n // (2 if cfg["symmetric"] else 1)
        s, d = rmat_edges(sc, m, seed)
    else:
        n = cfg["n"] >> scale_down
        m = cfg["pairs"] >> scale_down
        mean_deg = 2.0 * cfg["pairs"] / cfg["n"]
        s, d = chung_lu_pairs(n, m, cfg["max_deg"] / (1 << scale_down) if scale_down else cfg["max_deg"],
                              mean_deg, seed)
    return s, d, n


def workload_inputs(k: int, scale_down: int = 0, cache: bool = True):
    """All seeded inputs of workload k as a dict of numpy arrays (cached on disk)."""
    cfg = WORKLOADS[k]
    cdir = os.environ.get("GNNMP_INPUT_CACHE", os.path.join(os.environ.get("TMPDIR", "/tmp"), "gnnmp_inputs"))
    path = os.path.join(cdir, f"cfg{k}_sd{scale_down}.npz")
    if cache and os.path.exists(path):
        with np.load(path, allow_pickle=False) as z:
            return {key: z[key] for key in z.files}
    src, dst, n = workload_graph(k, scale_down)
    out = dict(src=src, dst=dst, n=np.int64(n))
    base = 1000 * k
    if cfg["kind"] == "gcn":
        w = cfg["widths"]
        out["X"] = normal((n, w[0]), base + 2)
        for li in range(len(w) - 1):
            out[f"W{li}"] = glorot(w[li], w[li + 1], base + 3 + 100 * li)
        if len(w) > 2:
            out["labels"] = labels(n, w[-1], base + 4)
    elif cfg["kind"] == "gat":
        h, dh = cfg["heads"], cfg["d_head"]
        out["X"] = normal((n, cfg["d_in"]), base + 2)
        out["W"] = glorot(cfg["d_in"], h * dh, base + 3)
        out["a_src"] = glorot(dh, 1, base + 103, shape=(h, dh))
        out["a_dst"] = glorot(dh, 1, base + 203, shape=(h, dh))
        out["dY"] = normal((n, h * dh), base + 4)
    else:
        out["H"] = normal((n, cfg["d"]), base + 2)
        out["rows"] = marginal_rows(n, cfg["marginal_frac"], base + 5)
        out["mixed_bits"] = random_bits(out["rows"].size, (2, 4, 8), base + 7)
        out["philox_seed"] = np.uint64(base + 6)
    if cache:
        os.makedirs(cdir, exist_ok=True)
        tmp = path + f".tmp{os.getpid()}.npz"
        np.savez(tmp, **out)
        os.replace(tmp, path)
    return out
