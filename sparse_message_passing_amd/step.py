"""Whole steps of the hot path over the C ABI, with every buffer allocated
once up front (torch supplies device memory; all arithmetic runs in
libgnnmp's kernels):

* ``GcnStack``  -- an L-layer GCN (ReLU on hidden layers, none on the
  logits), mean softmax cross-entropy, and the backward pass down to the
  first layer's weight gradient.
* ``GatLayer``  -- one GAT layer forward and backward for a given upstream
  gradient.
* ``QuantExchange`` -- one partition's quantised exchange: the marginal rows
  are quantised (one call per bit-width group) and dequantised into the
  aggregation input, then aggregated with the GCN operator.
"""
from __future__ import annotations

import numpy as np
import torch

from . import gnnmp


def _dt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def _padded(n, d, dtype, dev):
    """[n, d] view of a buffer with padded rows, so a gathered row touches as
    few cache lines as its size allows: f32 rows a multiple of 64 bytes (the
    41-wide aggregation: 0.535 ms in 176-byte rows, 0.513 ms in 192-byte
    rows), bf16 rows whole 128-byte lines (100 wide on the 2.45M-node graph:
    5.69 ms in 208-byte rows, 5.08 ms in 256-byte rows)."""
    q = 64 if dtype == torch.bfloat16 else 16
    ld = (d + q - 1) // q * q
    return torch.empty((n, ld), dtype=dtype, device=dev)[:, :d]


class GcnStack:
    def __init__(self, g: gnnmp.Graph, X, Ws, labels, dtype="f32"):
        self.g = g
        dev = X.device
        self.dt = _dt(dtype)
        self.X = X.to(self.dt).contiguous()
        self.Ws = [w.contiguous() for w in Ws]
        self.labels = labels
        n = g.n
        L = len(Ws)
        self.widths = [Ws[0].shape[0]] + [w.shape[1] for w in Ws]
        # activations: hidden layers in the storage type, logits in binary32
        self.H = [self.X] + [_padded(n, self.widths[i + 1], self.dt if i < L - 1 else torch.float32, dev)
                             for i in range(L)]
        self.saved = [_padded(n, self.widths[i], self.dt, dev) if self.widths[i + 1] > self.widths[i] else None
                      for i in range(L)]
        if self.saved[0] is not None and self.X.stride(0) != self.saved[0].stride(0):
            self.X = torch.nn.functional.pad(self.X, (0, self.saved[0].stride(0) - self.widths[0]))[:, :self.widths[0]]
            self.H[0] = self.X
        self.dW = [torch.empty_like(w) for w in self.Ws]
        self.dH = [None] + [_padded(n, self.widths[i], self.dt, dev) for i in range(1, L)]
        self.dlogits = _padded(n, self.widths[-1], torch.float32, dev)
        self.loss = torch.empty(1, dtype=torch.float32, device=dev)
        ws = max(gnnmp.gnn_gcn_workspace_size(g, self.widths[i], self.widths[i + 1]) for i in range(L))
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.xent_ws = torch.empty(max(gnnmp.lib().gnn_softmax_xent_workspace_size(n), 1), dtype=torch.uint8,
                                   device=dev)

    def forward(self):
        L = len(self.Ws)
        for i in range(L):
            gnnmp.gnn_gcn_layer_fwd(self.g, self.H[i], self.Ws[i], self.H[i + 1], relu=i < L - 1,
                                    saved=self.saved[i], ws=self.ws)
        gnnmp.gnn_softmax_xent(self.H[-1], self.labels, self.loss, self.dlogits, ws=self.xent_ws)
        return self.loss

    def backward(self):
        """Layer i's backward returns its input gradient already multiplied by
        the ReLU derivative of layer i-1 (relu_in), so no layer re-masks."""
        L = len(self.Ws)
        dY = self.dlogits
        for i in reversed(range(L)):
            gnnmp.gnn_gcn_layer_bwd(self.g, self.H[i], self.Ws[i], None, dY, relu=False, dW=self.dW[i],
                                    dX=self.dH[i] if i > 0 else None, saved=self.saved[i], ws=self.ws,
                                    relu_in=i > 0)
            dY = self.dH[i]
        return self.dW

    def step(self):
        self.forward()
        return self.backward()

    def spmm_edge_feats(self):
        """Edge x feature products one step aggregates (forward + backward)."""
        L = len(self.Ws)
        tot = 0
        for i in range(L):
            din, dout = self.widths[i], self.widths[i + 1]
            agg = min(din, dout) if dout <= din else din
            tot += agg                       # forward aggregation
            if dout <= din:
                tot += dout                  # backward: A_hat G
            elif i > 0:
                tot += din                   # backward: A_hat (G W^T), not formed for layer 0
        return tot * self.g.nnz


class GatLayer:
    def __init__(self, g: gnnmp.Graph, X, W, a_src, a_dst, heads, d_head, slope, dY):
        self.g, self.X, self.W = g, X.contiguous(), W.contiguous()
        self.a_src, self.a_dst = a_src.contiguous(), a_dst.contiguous()
        self.heads, self.d_head, self.slope = heads, d_head, slope
        self.dY = dY.contiguous()
        dev = X.device
        n, hd = g.n, heads * d_head
        self.Y = torch.empty((n, hd), device=dev)
        self.saved = torch.empty(gnnmp.gnn_gat_saved_size(g, heads, d_head), dtype=torch.uint8, device=dev)
        self.ws = torch.empty(max(gnnmp.gnn_gat_workspace_size(g, X.shape[1], heads, d_head), 1), dtype=torch.uint8,
                              device=dev)
        self.dX = torch.empty_like(self.X)
        self.dW = torch.empty_like(self.W)
        self.da_src = torch.empty_like(self.a_src)
        self.da_dst = torch.empty_like(self.a_dst)

    def forward(self):
        return gnnmp.gnn_gat_layer_fwd(self.g, self.X, self.W, self.a_src, self.a_dst, self.heads, self.d_head,
                                       self.slope, self.Y, self.saved, ws=self.ws)

    def backward(self, need_dX=True):
        return gnnmp.gnn_gat_layer_bwd(self.g, self.X, self.W, self.a_src, self.a_dst, self.heads, self.d_head,
                                       self.slope, self.Y, self.dY, self.saved, self.dW, self.da_src, self.da_dst,
                                       dX=self.dX if need_dX else None, ws=self.ws)

    def step(self):
        self.forward()
        return self.backward()


class QuantExchange:
    """One partition's quantised message exchange (AdaQP Sec. 3): the marginal
    rows are quantised per row (one group per bit-width), "sent", and the
    receiver aggregates them with the central rows.  The plain path
    dequantises into a binary32 copy of the matrix and aggregates it; the
    fused path aggregates straight from the codes (gnn_spmm_dequant), with
    bitwise the same result.  backward() exchanges the embedding gradients of
    the same rows the same way (Philox stream stream_id + 1) and aggregates
    them over the transposed graph (A_hat is symmetric)."""

    def __init__(self, g: gnnmp.Graph, H, rows, bits, seed, stream_id=0, fused=False):
        """bits: 2, 4, 8, or an int array giving each row's width."""
        self.g, self.H = g, H.contiguous()
        dev = H.device
        d = H.shape[1]
        rows = np.asarray(rows, np.int32)
        b = np.full(rows.size, bits, np.int32) if np.isscalar(bits) else np.asarray(bits, np.int32)
        self.groups = []
        for bb in (2, 4, 8):
            sel = rows[b == bb]
            if sel.size == 0:
                continue
            self.groups.append((bb, torch.from_numpy(sel).to(dev),
                                torch.empty((sel.size, d * bb // 8), dtype=torch.uint8, device=dev),
                                torch.empty(sel.size, device=dev), torch.empty(sel.size, device=dev)))
        self.seed, self.stream_id, self.fused = seed, stream_id, fused
        self.Hmix = None if fused else self.H.clone()
        self.Y = torch.empty_like(self.H)
        self.dH = torch.empty_like(self.H)
        self.qslot = torch.empty(g.n, dtype=torch.int32, device=dev)
        gnnmp.gnn_quant_slots(g.n, [gr[1] for gr in self.groups], self.qslot)
        self.qgroups = [(pk, sc, zr, bb) for bb, _, pk, sc, zr in self.groups]
        self.ws = torch.empty(max(gnnmp.lib().gnn_spmm_dequant_workspace_size(g.h, d), 1), dtype=torch.uint8,
                              device=dev)

    def quantize(self, M=None, stream_id=None):
        M = self.H if M is None else M
        sid = self.stream_id if stream_id is None else stream_id
        for bb, rows, pk, sc, zr in self.groups:
            gnnmp.gnn_quantize(M, rows, bb, self.seed, pk, sc, zr, stream_id=sid)

    def dequantize(self, out):
        for bb, rows, pk, sc, zr in self.groups:
            gnnmp.gnn_dequantize(pk, sc, zr, rows, bb, out)

    def step(self):
        self.quantize()
        if self.fused:
            return gnnmp.gnn_spmm_dequant(self.g, self.H, self.qslot, self.qgroups, self.Y, ws=self.ws)
        self.dequantize(self.Hmix)
        return gnnmp.gnn_spmm(self.g, self.Hmix, self.Y, ws=self.ws)

    def backward(self, dY):
        """dH = A_hat^T dY~, the marginal rows of dY exchanged quantised."""
        self.quantize(dY, self.stream_id + 1)
        return gnnmp.gnn_spmm_dequant(self.g, dY, self.qslot, self.qgroups, self.dH, ws=self.ws)


class OverlapExchange:
    """The exchange split as AdaQP does (Eqn. 7; Sec. 3, computation-
    communication parallelisation and its three isolated stages, Fig. 7) on
    one GPU: the aggregation over in-edges from central sources runs on the
    binary32 rows at once, while the marginal rows are quantised, "sent" (a
    device-to-device copy stands in for the transfer) and aggregated from
    their codes over the in-edges from marginal sources, added to the central
    part.  Three schedules of the same kernels, with bitwise the same result:

    * sequential: everything on the caller's stream;
    * free: central aggregation on one stream, quantise + transfer on
      another, the marginal aggregation after both;
    * staged (AdaQP Fig. 7): quantise alone, then the central aggregation
      alongside the transfer, then the marginal aggregation.
    """

    def __init__(self, g: gnnmp.Graph, H, rows, bits, seed, stream_id=0):
        self.g, self.H = g, H.contiguous()
        dev = H.device
        n, d = g.n, H.shape[1]
        rows = np.asarray(rows, np.int32)
        b = np.full(rows.size, bits, np.int32) if np.isscalar(bits) else np.asarray(bits, np.int32)
        marginal = np.zeros(n, dtype=bool)
        marginal[rows] = True
        self.g_local, self.g_remote = gnnmp.gnn_graph_split(g, marginal)
        self.send, self.recv = [], []
        for bb in (2, 4, 8):
            sel = rows[b == bb]
            if sel.size == 0:
                continue
            mk = lambda: (torch.empty((sel.size, d * bb // 8), dtype=torch.uint8, device=dev),
                          torch.empty(sel.size, device=dev), torch.empty(sel.size, device=dev))
            self.send.append((bb, torch.from_numpy(sel).to(dev), *mk()))
            self.recv.append((bb, *mk()))
        self.seed, self.stream_id = seed, stream_id
        self.qslot = torch.empty(n, dtype=torch.int32, device=dev)
        gnnmp.gnn_quant_slots(n, [s[1] for s in self.send], self.qslot)
        self.recv_groups = [(pk, sc, zr, bb) for bb, pk, sc, zr in self.recv]
        self.Y = torch.empty_like(self.H)
        self.ws_l = torch.empty(max(gnnmp.lib().gnn_spmm_workspace_size(self.g_local.h, 0, d), 1),
                                dtype=torch.uint8, device=dev)
        self.ws_r = torch.empty(max(gnnmp.lib().gnn_spmm_dequant_workspace_size(self.g_remote.h, d), 1),
                                dtype=torch.uint8, device=dev)
        self.s_central = torch.cuda.Stream(device=dev)
        self.s_marginal = torch.cuda.Stream(device=dev)
        self.marks = {}

    # -- the four pieces ---------------------------------------------------
    def quantize(self):
        for bb, r, pk, sc, zr in self.send:
            gnnmp.gnn_quantize(self.H, r, bb, self.seed, pk, sc, zr, stream_id=self.stream_id)

    def transfer(self):
        for (_, _, pk, sc, zr), (_, rpk, rsc, rzr) in zip(self.send, self.recv):
            rpk.copy_(pk)
            rsc.copy_(sc)
            rzr.copy_(zr)

    def central(self):
        return gnnmp.gnn_spmm(self.g_local, self.H, self.Y, ws=self.ws_l)

    def marginal(self):
        return gnnmp.gnn_spmm_dequant(self.g_remote, self.H, self.qslot, self.recv_groups, self.Y, ws=self.ws_r,
                                      Z=self.Y)

    # -- schedules -----------------------------------------------------------
    def _mark(self, name, stream):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        self.marks[name] = ev

    def step_sequential(self):
        cur = torch.cuda.current_stream()
        self._mark("start", cur)
        self.quantize()
        self._mark("quantized", cur)
        self.transfer()
        self._mark("transferred", cur)
        self.central()
        self._mark("central", cur)
        self.marginal()
        self._mark("end", cur)
        return self.Y

    def step_free(self):
        cur = torch.cuda.current_stream()
        self._mark("start", cur)
        self.s_central.wait_event(self.marks["start"])
        self.s_marginal.wait_event(self.marks["start"])
        with torch.cuda.stream(self.s_central):
            self.central()
            self._mark("central", self.s_central)
        with torch.cuda.stream(self.s_marginal):
            self.quantize()
            self._mark("quantized", self.s_marginal)
            self.transfer()
            self._mark("transferred", self.s_marginal)
            self.s_marginal.wait_event(self.marks["central"])
            self.marginal()
            self._mark("end", self.s_marginal)
        cur.wait_event(self.marks["end"])
        return self.Y

    def step_staged(self):
        cur = torch.cuda.current_stream()
        self._mark("start", cur)
        self.s_marginal.wait_event(self.marks["start"])
        with torch.cuda.stream(self.s_marginal):          # stage 1: quantise alone
            self.quantize()
            self._mark("quantized", self.s_marginal)
        self.s_central.wait_event(self.marks["quantized"])
        with torch.cuda.stream(self.s_central):           # stage 2: central aggregation ...
            self.central()
            self._mark("central", self.s_central)
        with torch.cuda.stream(self.s_marginal):          # ... alongside the transfer
            self.transfer()
            self._mark("transferred", self.s_marginal)
            self.s_marginal.wait_event(self.marks["central"])
            self.marginal()                               # stage 3: marginal aggregation
            self._mark("end", self.s_marginal)
        cur.wait_event(self.marks["end"])
        return self.Y

    def timeline(self):
        """ms from the start mark to each recorded mark of the last step
        (call after synchronising)."""
        t0 = self.marks["start"]
        return {k: round(t0.elapsed_time(ev), 4) for k, ev in self.marks.items() if k != "start"}


def adaptive_bits(g: gnnmp.Graph, H, rows, avg_bits, edge_w=None):
    """AdaQP's adaptive bit-width assignment with the greedy stand-in for its
    solver: per-row statistics on the GPU (gnn_quant_stats), then the
    assignment on the host (gnn_assign_bits).  Returns (bits, beta) as numpy."""
    rows_d = torch.from_numpy(np.asarray(rows, np.int32)).to(H.device)
    beta = torch.empty(rows_d.numel(), device=H.device)
    rng = torch.empty_like(beta)
    gnnmp.gnn_quant_stats(g, H, rows_d, beta, rng, edge_w=edge_w)
    b = beta.cpu().numpy()
    return gnnmp.gnn_assign_bits(b, H.shape[1], avg_bits), b
