"""The allocation-free aggregation (gnn_spmm_noalloc): the hub-row partials
in the library's fixed device scratch instead of a caller workspace.  Its
output must equal gnn_spmm's bit for bit (the same kernels) and the oracle's
to the binary32 bar, on consecutive calls that reuse the scratch (the second
smaller than the first), and a call whose partials exceed the scratch is
refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
from parity import check_close, from_dev, graph_pair, hub_edges, to_dev
from sparse_message_passing_amd import gnnmp

pytestmark = pytest.mark.gpu


def _agg_check(g, og, d, seed, transpose=False, weights="gcn"):
    r = np.random.default_rng(seed)
    X = r.standard_normal((og.n, d)).astype(np.float32)
    Xd = to_dev(X)
    Y_ws = torch.empty((og.n, d), device="cuda")
    Y_na = torch.full((og.n, d), 7.0, device="cuda")
    gnnmp.gnn_spmm(g, Xd, Y_ws, weights=weights, transpose=transpose)
    gnnmp.gnn_spmm_noalloc(g, Xd, Y_na, weights=weights, transpose=transpose)
    torch.cuda.synchronize()
    assert torch.equal(Y_ws, Y_na), "gnn_spmm_noalloc differs from gnn_spmm"
    w = og.gcn_norm()[1] if weights == "gcn" else og.mean_weights()
    ref = oracle.spmm(og, X, w, transpose=transpose)
    mag = oracle.spmm(og, np.abs(X), np.abs(w), transpose=transpose)
    check_close(from_dev(Y_na), ref, mag, what=f"noalloc aggregation d={d}")


def test_noalloc_matches_workspace_path_on_consecutive_calls():
    # hub rows (2,500 and 1,200 in-edges) so the chunked partial path runs
    s, t = hub_edges(6000, 40000, 2500, 51)
    g, og = graph_pair(s, t, 6000, True, csc=True)
    assert gnnmp.lib().gnn_spmm_workspace_size(g.h, 0, 256) > 0
    _agg_check(g, og, 256, 1)
    # second call: a smaller graph and width, on the scratch the first call left
    s2, t2 = hub_edges(3000, 15000, 1200, 52)
    g2, og2 = graph_pair(s2, t2, 3000, False, csc=True)
    assert gnnmp.lib().gnn_spmm_workspace_size(g2.h, 0, 64) > 0
    _agg_check(g2, og2, 64, 2)
    _agg_check(g2, og2, 64, 3, transpose=True, weights="mean")


def test_noalloc_refuses_partials_beyond_its_scratch():
    # 160 hubs of 60,000 in-edges: 18,880 chunks of 512 edges x 1024
    # features x 4 bytes (77 MB) do not fit the 64 MiB scratch
    n, hubs, deg = 70000, 160, 60000
    r = np.random.default_rng(53)
    src = np.concatenate([r.choice(np.arange(hubs, n), deg, replace=False) for _ in range(hubs)]).astype(np.int32)
    dst = np.repeat(np.arange(hubs, dtype=np.int32), deg)
    g = gnnmp.gnn_graph_create(n, src, dst)
    d = 1024
    assert gnnmp.lib().gnn_spmm_workspace_size(g.h, 0, d) > gnnmp.lib().gnn_spmm_noalloc_max_scratch()
    X = torch.zeros((n, d), device="cuda")
    Y = torch.full((n, d), 7.0, device="cuda")
    with pytest.raises(gnnmp.GnnError, match="scratch"):
        gnnmp.gnn_spmm_noalloc(g, X, Y)
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0))
