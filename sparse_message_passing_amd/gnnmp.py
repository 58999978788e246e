"""Thin Python binding of libgnnmp.so (ctypes).

Each function carries the name of the C entry point it calls and only
marshals arguments: torch tensors give device pointers, the current torch
stream gives the HIP stream, and workspaces are torch allocations.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgnnmp.so")

GNN_F32, GNN_BF16 = 0, 1
GNN_W_GCN, GNN_W_ONES, GNN_W_EDGE, GNN_W_MEAN = 0, 1, 2, 3
GNN_GRAPH_SYMMETRIZE, GNN_GRAPH_CSC = 0x1, 0x2

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "out of memory", 4: "HIP error",
          5: "graph lacks the required view", 6: "workspace too small"}

# exported symbols and their argument types (P = pointer, I = int64, i = int32, U = uint32, Q = uint64, F = float,
# D = double, S = size_t)
_SIGS = {
    "gnn_status_string": ("i", "P"),
    "gnn_last_error": ("", "P"),
    "gnn_graph_create": ("IIPPUP", "i"),
    "gnn_graph_destroy": ("P", "i"),
    "gnn_graph_split": ("PPPP", "i"),
    "gnn_graph_info": ("PP", "i"),
    "gnn_graph_export": ("PPPPPPPPPPPP", "i"),
    "gnn_spmm_workspace_size": ("PiI", "S"),
    "gnn_spmm": ("PiiPiPiIPiIIiPSP", "i"),
    "gnn_spmm_noalloc_max_scratch": ("", "S"),
    "gnn_spmm_noalloc": ("PiiPiPiIPiIIiP", "i"),
    "gnn_edge_reduce": ("PiPiPP", "i"),
    "gnn_sddmm": ("PiPIPIiiIFPPP", "i"),
    "gnn_edge_softmax": ("PPPiP", "i"),
    "gnn_edge_softmax_bwd": ("PPPPFPiP", "i"),
    "gnn_gemm_workspace_size": ("iiIII", "S"),
    "gnn_gemm": ("iiIIIPiIPiIPiIPSP", "i"),
    "gnn_gemm_q8_workspace_size": ("III", "S"),
    "gnn_gemm_q8": ("IIIPIPIPIQUPSP", "i"),
    "gnn_sddmm_q8_workspace_size": ("PI", "S"),
    "gnn_sddmm_q8": ("PPIPIiIQUPPSP", "i"),
    "gnn_softmax_xent_workspace_size": ("I", "S"),
    "gnn_softmax_xent": ("PIIIPPPIPSP", "i"),
    "gnn_quantize": ("PIIPIiQUPPPP", "i"),
    "gnn_dequantize": ("PPPIIiPPIP", "i"),
    "gnn_quant_slots": ("IiPPPP", "i"),
    "gnn_quant_stats": ("PPPIIPIPPP", "i"),
    "gnn_assign_bits": ("IPIDP", "i"),
    "gnn_spmm_dequant_workspace_size": ("PI", "S"),
    "gnn_spmm_dequant": ("PPIPPiPIPIIiPSP", "i"),
    "gnn_gcn_workspace_size": ("PII", "S"),
    "gnn_gcn_layer_fwd": ("PPiIIPIiPiIPPSP", "i"),
    "gnn_gcn_layer_bwd": ("PPiIIPIiiPPiIPPPPSP", "i"),
    "gnn_sage_workspace_size": ("PII", "S"),
    "gnn_sage_layer_fwd": ("PPiIIPIiPiIPPSP", "i"),
    "gnn_sage_layer_bwd": ("PPiIIPIiiPPiIPPPPSP", "i"),
    "gnn_gat_saved_size": ("PiI", "S"),
    "gnn_gat_workspace_size": ("PIiI", "S"),
    "gnn_gat_layer_fwd": ("PPIPPPiIFPPPSP", "i"),
    "gnn_gat_layer_bwd": ("PPIPPPiIFPPPPPPPPSP", "i"),
    "gnn_timer_start": ("PI", "i"),
    "gnn_timer_stop": ("", "i"),
    "gnn_timer_result": ("PPP", "i"),
    "gnn_timer_keys": ("PS", "i"),
    "gnn_timer_release": ("", "i"),
}
_CT = {"P": C.c_void_p, "I": C.c_int64, "i": C.c_int, "U": C.c_uint32, "Q": C.c_uint64, "F": C.c_float,
       "D": C.c_double, "S": C.c_size_t}

EXPORTED = tuple(_SIGS)


class GnnError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class _Info(C.Structure):
    _fields_ = [("n", C.c_int64), ("nnz", C.c_int64), ("max_in_degree", C.c_int64), ("max_out_degree", C.c_int64),
                ("has_csc", C.c_int), ("row_ptr", C.c_void_p), ("col", C.c_void_p), ("dinv", C.c_void_p),
                ("perm", C.c_void_p), ("col_ptr", C.c_void_p), ("csc_row", C.c_void_p), ("csc_eid", C.c_void_p),
                ("perm_t", C.c_void_p), ("symmetric", C.c_int), ("bucket_threshold", C.c_int64 * 2),
                ("bucket_off", C.c_int64 * 4), ("bucket_off_t", C.c_int64 * 4),
                ("bucket_threshold_t", C.c_int64 * 2)]


_lib = None


def lib():
    """The loaded library; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_message_passing_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = [_CT[a] for a in args]
            fn.restype = C.c_char_p if name in ("gnn_status_string", "gnn_last_error") else _CT[res]
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise GnnError(status, lib().gnn_last_error().decode())


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    return t.data_ptr()


def _dt(t):
    if t.dtype == torch.float32:
        return GNN_F32
    if t.dtype == torch.bfloat16:
        return GNN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _f32(*ts):
    """Entry points whose C signature takes float*: refuse other dtypes before
    any pointer reaches the library (a bf16 buffer read as float would run
    past its end)."""
    for t in ts:
        if t is not None and not isinstance(t, int) and t.dtype != torch.float32:
            raise TypeError(f"expected a float32 tensor, got {t.dtype}")


def _i32(*ts):
    for t in ts:
        if t is not None and t.dtype != torch.int32:
            raise TypeError(f"expected an int32 tensor, got {t.dtype}")


def _shape_at_least(t, rows, cols, what):
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{what}: expected at least [{rows}, {cols}], got {list(t.shape)}")


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _ld(t):
    return t.stride(0) if t.dim() == 2 else t.shape[-1]


# ---------------------------------------------------------------------------
# graph
# ---------------------------------------------------------------------------
class Graph:
    """Owns a library graph handle (CSR by destination, optional CSC view)."""

    def __init__(self, handle, device):
        self.h = handle
        self.device = device
        info = _Info()
        _check(lib().gnn_graph_info(self.h, C.byref(info)))
        self.n, self.nnz = info.n, info.nnz
        self.max_in_degree, self.max_out_degree = info.max_in_degree, info.max_out_degree
        self.has_csc = bool(info.has_csc)
        self.symmetric = bool(info.symmetric)
        self.bucket_threshold = list(info.bucket_threshold)
        self.bucket_off = list(info.bucket_off)
        self.bucket_off_t = list(info.bucket_off_t)
        self.bucket_threshold_t = list(info.bucket_threshold_t)

    def __del__(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.gnn_graph_destroy(self.h)
            self.h = None


def gnn_graph_create(n, src, dst, symmetrize=False, csc=False, device=None):
    """Build on `device` (default: the current device); the handle's arrays live there."""
    src = np.ascontiguousarray(src, dtype=np.int32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    if src.shape != dst.shape:
        raise ValueError("src and dst differ in length")
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    torch.cuda.set_device(dev)
    h = C.c_void_p()
    flags = (GNN_GRAPH_SYMMETRIZE if symmetrize else 0) | (GNN_GRAPH_CSC if csc else 0)
    _check(lib().gnn_graph_create(int(n), src.size, src.ctypes.data_as(C.c_void_p), dst.ctypes.data_as(C.c_void_p),
                                  flags, C.byref(h)))
    return Graph(h, dev)


def gnn_graph_split(g: Graph, marginal):
    """(local, remote): the in-edges from non-marginal / marginal sources
    (marginal: bool or uint8 array over the n nodes), weights kept from g."""
    m = np.ascontiguousarray(np.asarray(marginal) != 0, dtype=np.uint8)
    if m.size != g.n:
        raise ValueError("marginal must have one entry per node")
    torch.cuda.set_device(g.device)
    lo, hi = C.c_void_p(), C.c_void_p()
    _check(lib().gnn_graph_split(g.h, m.ctypes.data_as(C.c_void_p), C.byref(lo), C.byref(hi)))
    return Graph(lo, g.device), Graph(hi, g.device)


def gnn_graph_export(g: Graph):
    n, e = g.n, g.nnz
    out = dict(row_ptr=np.empty(n + 1, np.int64), col=np.empty(e, np.int32), dinv=np.empty(n, np.float32),
               w=np.empty(e, np.float32), perm=np.empty(n, np.int32), bucket_off=np.empty(4, np.int64))
    if g.has_csc:
        out.update(col_ptr=np.empty(n + 1, np.int64), csc_row=np.empty(e, np.int32), csc_eid=np.empty(e, np.int32),
                   perm_t=np.empty(n, np.int32), bucket_off_t=np.empty(4, np.int64))
    P = lambda k: out[k].ctypes.data_as(C.c_void_p) if k in out else None
    _check(lib().gnn_graph_export(g.h, P("row_ptr"), P("col"), P("dinv"), P("w"), P("perm"), P("bucket_off"),
                                  P("col_ptr"), P("csc_row"), P("csc_eid"), P("perm_t"), P("bucket_off_t")))
    return out


# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------
def gnn_spmm(g: Graph, X, Y, weights="gcn", heads=1, transpose=False, relu=False, d=None, ws=None):
    """Y = (G . w) X (transpose: over the reversed graph), optional ReLU.
    weights: "gcn", "ones", "mean" or an f32 tensor [nnz, heads]."""
    d = X.shape[1] if d is None else d
    if isinstance(weights, str):
        wmode, ew = {"gcn": GNN_W_GCN, "ones": GNN_W_ONES, "mean": GNN_W_MEAN}[weights], None
    else:
        wmode, ew = GNN_W_EDGE, weights
        _f32(ew)
    need = lib().gnn_spmm_workspace_size(g.h, int(transpose), d)
    if ws is None:
        ws = _ws(need, X.device)
    _check(lib().gnn_spmm(g.h, int(transpose), wmode, _p(ew), heads, _p(X), _dt(X), _ld(X), _p(Y), _dt(Y), _ld(Y), d,
                          int(relu), _p(ws), ws.numel(), _stream()))
    return Y


def gnn_spmm_noalloc(g: Graph, X, Y, weights="gcn", heads=1, transpose=False, relu=False, d=None):
    """gnn_spmm with the hub-row partials in the library's fixed device scratch
    (no workspace): for callers that cannot allocate."""
    d = X.shape[1] if d is None else d
    if isinstance(weights, str):
        wmode, ew = {"gcn": GNN_W_GCN, "ones": GNN_W_ONES, "mean": GNN_W_MEAN}[weights], None
    else:
        wmode, ew = GNN_W_EDGE, weights
        _f32(ew)
    _check(lib().gnn_spmm_noalloc(g.h, int(transpose), wmode, _p(ew), heads, _p(X), _dt(X), _ld(X), _p(Y), _dt(Y),
                                  _ld(Y), d, int(relu), _stream()))
    return Y


def gnn_edge_reduce(g: Graph, vals, out, by_src=False):
    _f32(vals, out)
    _check(lib().gnn_edge_reduce(g.h, int(by_src), _p(vals), vals.shape[1], _p(out), _stream()))
    return out


def gnn_sddmm(g: Graph, op, src_feat, dst_feat, heads, d_head, out, slope=float("nan"), out_pre=None):
    """op "add": out = LReLU(src[u,k] + dst[v,k]); op "dot": out = <src[u, head k], dst[v, head k]>."""
    opc = {"add": 0, "dot": 1}[op]
    _f32(out, out_pre)
    if op == "add":
        _f32(src_feat, dst_feat)
    _check(lib().gnn_sddmm(g.h, opc, _p(src_feat), _ld(src_feat), _p(dst_feat), _ld(dst_feat), _dt(src_feat), heads,
                           d_head, float(slope), _p(out), _p(out_pre), _stream()))
    return out


def gnn_edge_softmax(g: Graph, E, alpha):
    _f32(E, alpha)
    _check(lib().gnn_edge_softmax(g.h, _p(E), _p(alpha), E.shape[1], _stream()))
    return alpha


def gnn_edge_softmax_bwd(g: Graph, alpha, dalpha, dE, lrelu_pre=None, slope=0.0):
    _f32(alpha, dalpha, dE, lrelu_pre)
    _check(lib().gnn_edge_softmax_bwd(g.h, _p(alpha), _p(dalpha), _p(lrelu_pre), float(slope), _p(dE),
                                      alpha.shape[1], _stream()))
    return dE


def gnn_gemm(A, B, C_, transA=False, transB=False, ws=None):
    """C = op(A) op(B)."""
    M = A.shape[1] if transA else A.shape[0]
    K = A.shape[0] if transA else A.shape[1]
    N = B.shape[0] if transB else B.shape[1]
    if (B.shape[1] if transB else B.shape[0]) != K or tuple(C_.shape) != (M, N):
        raise ValueError("gnn_gemm: shape mismatch")
    need = lib().gnn_gemm_workspace_size(int(transA), int(transB), M, N, K)
    if ws is None:
        ws = _ws(need, A.device)
    _check(lib().gnn_gemm(int(transA), int(transB), M, N, K, _p(A), _dt(A), _ld(A), _p(B), _dt(B), _ld(B), _p(C_),
                          _dt(C_), _ld(C_), _p(ws), ws.numel(), _stream()))
    return C_


def gnn_softmax_xent(logits, labels, loss, dlogits=None, ws=None):
    n, c = logits.shape
    _f32(logits, loss, dlogits)
    _i32(labels)
    if ws is None:
        ws = _ws(lib().gnn_softmax_xent_workspace_size(n), logits.device)
    _check(lib().gnn_softmax_xent(_p(logits), n, c, _ld(logits), _p(labels), _p(loss), _p(dlogits),
                                  _ld(dlogits) if dlogits is not None else c, _p(ws), ws.numel(), _stream()))
    return loss


def gnn_quantize(H, rows, bits, seed, packed, scale, zero, stream_id=0, d=None):
    _f32(H, scale, zero)
    _i32(rows)
    d = H.shape[1] if d is None else d
    _check(lib().gnn_quantize(_p(H), _ld(H), d, _p(rows), rows.numel(), bits, int(seed), int(stream_id), _p(packed),
                              _p(scale), _p(zero), _stream()))
    return packed, scale, zero


def gnn_dequantize(packed, scale, zero, rows, bits, H, d=None):
    _f32(H, scale, zero)
    _i32(rows)
    d = H.shape[1] if d is None else d
    _check(lib().gnn_dequantize(_p(packed), _p(scale), _p(zero), rows.numel(), d, bits, _p(rows), _p(H), _ld(H),
                                _stream()))
    return H


def gnn_gemm_q8(A, B, C, seed, stream_id=0, ws=None):
    """C = dequant(q8(A) q8(B)): Tango's quantisation-aware GEMM (f32 in and out)."""
    _f32(A, B, C)
    M, K = A.shape
    N = B.shape[1]
    if B.shape[0] != K or tuple(C.shape) != (M, N):
        raise ValueError("gnn_gemm_q8: shape mismatch")
    if ws is None:
        ws = _ws(lib().gnn_gemm_q8_workspace_size(M, N, K), A.device)
    _check(lib().gnn_gemm_q8(M, N, K, _p(A), _ld(A), _p(B), _ld(B), _p(C), _ld(C), int(seed), int(stream_id), _p(ws),
                             ws.numel(), _stream()))
    return C


def gnn_sddmm_q8(g: Graph, src_feat, dst_feat, heads, d_head, out, seed, stream_id=0, ws=None):
    """out[e, k] = dequant(q8(src_feat)[u, head k] . q8(dst_feat)[v, head k]):
    Tango's SDDMM dot on 8-bit codes (f32 in and out)."""
    _f32(src_feat, dst_feat, out)
    _shape_at_least(src_feat, g.n, heads * d_head, "gnn_sddmm_q8 src_feat")
    _shape_at_least(dst_feat, g.n, heads * d_head, "gnn_sddmm_q8 dst_feat")
    _shape_at_least(out, g.nnz, heads, "gnn_sddmm_q8 out")
    if ws is None:
        ws = _ws(lib().gnn_sddmm_q8_workspace_size(g.h, heads * d_head), src_feat.device)
    _check(lib().gnn_sddmm_q8(g.h, _p(src_feat), _ld(src_feat), _p(dst_feat), _ld(dst_feat), heads, d_head,
                              int(seed), int(stream_id), _p(out), _p(ws), ws.numel(), _stream()))
    return out


def gnn_quant_stats(g: Graph, H, rows, beta, rng, edge_w=None, d=None):
    """beta[r], range[r] of the listed rows (AdaQP's bit-width statistics)."""
    _f32(H, beta, rng, edge_w)
    _i32(rows)
    d = H.shape[1] if d is None else d
    _check(lib().gnn_quant_stats(g.h, _p(edge_w), _p(H), _ld(H), d, _p(rows), rows.numel(), _p(beta), _p(rng),
                                 _stream()))
    return beta, rng


def gnn_assign_bits(beta, d, avg_bits):
    """Greedy {2, 4, 8} assignment under an average-bits budget (host arrays)."""
    b = np.ascontiguousarray(np.asarray(beta, dtype=np.float32))
    out = np.empty(b.size, dtype=np.int32)
    _check(lib().gnn_assign_bits(b.size, b.ctypes.data_as(C.c_void_p), int(d), float(avg_bits),
                                 out.ctypes.data_as(C.c_void_p)))
    return out


class QGroup(C.Structure):
    """One bit-width buffer of quantised rows (gnn_qgroup_t)."""
    _fields_ = [("packed", C.c_void_p), ("scale", C.c_void_p), ("zero", C.c_void_p), ("n_rows", C.c_int64),
                ("bits", C.c_int)]


def gnn_quant_slots(n, rows_list, qslot):
    """qslot[v] = -1, then (g << 27) | r at rows_list[g][r]."""
    k = len(rows_list)
    rows = (C.c_void_p * max(k, 1))(*[_p(r) for r in rows_list])
    counts = (C.c_int64 * max(k, 1))(*[r.numel() for r in rows_list])
    _check(lib().gnn_quant_slots(n, k, rows, counts, _p(qslot), _stream()))
    return qslot


def gnn_spmm_dequant(g: Graph, X, qslot, groups, Y, relu=False, d=None, ws=None, Z=None):
    """Y = A_hat X~ (+ Z), X~ = X with the slotted rows dequantised in the gather.
    groups: list of (packed, scale, zero, bits)."""
    _f32(X, Y, Z, *[sc for _, sc, _, _ in groups], *[zr for _, _, zr, _ in groups])
    _i32(qslot)
    d = X.shape[1] if d is None else d
    arr = (QGroup * max(len(groups), 1))(*[QGroup(_p(pk), _p(sc), _p(zr), sc.numel(), b)
                                           for pk, sc, zr, b in groups])
    if ws is None:
        ws = _ws(lib().gnn_spmm_dequant_workspace_size(g.h, d), X.device)
    _check(lib().gnn_spmm_dequant(g.h, _p(X), _ld(X), _p(qslot), arr, len(groups), _p(Z),
                                  _ld(Z) if Z is not None else 0, _p(Y), _ld(Y), d, int(relu), _p(ws), ws.numel(),
                                  _stream()))
    return Y


# ---------------------------------------------------------------------------
# layers
# ---------------------------------------------------------------------------
def gnn_gcn_workspace_size(g: Graph, d_in, d_out):
    return lib().gnn_gcn_workspace_size(g.h, d_in, d_out)


def gnn_gcn_layer_fwd(g: Graph, X, W, Y, relu, saved=None, ws=None, _fn="gnn_gcn_layer_fwd"):
    """Y = sigma(A_hat X W); X, Y may be row-strided views (leading dims from their strides)."""
    d_in, d_out = W.shape
    _f32(W)
    if ws is None:
        ws = _ws(gnn_gcn_workspace_size(g, d_in, d_out), X.device)
    if saved is not None and _ld(saved) != _ld(X):
        raise ValueError("saved must have X's row stride")
    _check(getattr(lib(), _fn)(g.h, _p(X), _dt(X), _ld(X), d_in, _p(W), d_out, int(relu), _p(Y), _dt(Y), _ld(Y),
                                   _p(saved), _p(ws), ws.numel(), _stream()))
    return Y


def gnn_gcn_layer_bwd(g: Graph, X, W, Y, dY, relu, dW, dX=None, saved=None, ws=None, relu_in=False,
                      _fn="gnn_gcn_layer_bwd"):
    d_in, d_out = W.shape
    _f32(W, dW)
    if ws is None:
        ws = _ws(gnn_gcn_workspace_size(g, d_in, d_out), dY.device)
    ref = X if X is not None else saved
    for t in (dX, saved):
        if t is not None and _ld(t) != _ld(ref):
            raise ValueError("dX / saved must have X's row stride")
    if Y is not None and _ld(Y) != _ld(dY):
        raise ValueError("Y and dY must share a row stride")
    _check(getattr(lib(), _fn)(g.h, _p(X), _dt(ref), _ld(ref), d_in, _p(W), d_out, int(relu), int(relu_in),
                                   _p(Y), _p(dY), _dt(dY), _ld(dY), _p(saved), _p(dX), _p(dW), _p(ws), ws.numel(),
                                   _stream()))
    return dX, dW


def gnn_sage_layer_fwd(g: Graph, X, W, Y, relu, saved=None, ws=None):
    """Y = sigma(M X W), M the mean aggregation (GraphSAGE)."""
    return gnn_gcn_layer_fwd(g, X, W, Y, relu, saved=saved, ws=ws, _fn="gnn_sage_layer_fwd")


def gnn_sage_layer_bwd(g: Graph, X, W, Y, dY, relu, dW, dX=None, saved=None, ws=None, relu_in=False):
    return gnn_gcn_layer_bwd(g, X, W, Y, dY, relu, dW, dX=dX, saved=saved, ws=ws, relu_in=relu_in,
                             _fn="gnn_sage_layer_bwd")


def gnn_gat_saved_size(g: Graph, heads, d_head):
    return lib().gnn_gat_saved_size(g.h, heads, d_head)


def gnn_gat_workspace_size(g: Graph, d_in, heads, d_head):
    return lib().gnn_gat_workspace_size(g.h, d_in, heads, d_head)


def _gat_check(g, X, W, a_src, a_dst, heads, d_head, saved, Y, dY=None, dX=None):
    """The GAT entry points take contiguous f32 node matrices with n rows."""
    _f32(X, W, a_src, a_dst, Y, dY, dX)
    hd = heads * d_head
    d_in = X.shape[1]
    for t, cols, what in ((X, d_in, "X"), (Y, hd, "Y"), (dY, hd, "dY"), (dX, d_in, "dX")):
        if t is not None and (t.dim() != 2 or tuple(t.shape) != (g.n, cols) or not t.is_contiguous()):
            raise ValueError(f"GAT {what}: expected a contiguous [{g.n}, {cols}] tensor, got {list(t.shape)}")
    for t, shape, what in ((W, (d_in, hd), "W"), (a_src, (heads, d_head), "a_src"), (a_dst, (heads, d_head), "a_dst")):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"GAT {what}: expected a contiguous {list(shape)} tensor, got {list(t.shape)}")
    if saved.numel() * saved.element_size() < gnn_gat_saved_size(g, heads, d_head):
        raise ValueError("GAT: saved is smaller than gnn_gat_saved_size()")
    return d_in


def gnn_gat_layer_fwd(g: Graph, X, W, a_src, a_dst, heads, d_head, slope, Y, saved, ws=None):
    d_in = _gat_check(g, X, W, a_src, a_dst, heads, d_head, saved, Y)
    if ws is None:
        ws = _ws(gnn_gat_workspace_size(g, d_in, heads, d_head), X.device)
    _check(lib().gnn_gat_layer_fwd(g.h, _p(X), d_in, _p(W), _p(a_src), _p(a_dst), heads, d_head, float(slope), _p(Y),
                                   _p(saved), _p(ws), ws.numel(), _stream()))
    return Y


def gnn_gat_layer_bwd(g: Graph, X, W, a_src, a_dst, heads, d_head, slope, Y, dY, saved, dW, da_src, da_dst,
                      dX=None, ws=None):
    d_in = _gat_check(g, X, W, a_src, a_dst, heads, d_head, saved, Y, dY, dX)
    _f32(dW, da_src, da_dst)
    if tuple(dW.shape) != tuple(W.shape) or tuple(da_src.shape) != (heads, d_head) or \
            tuple(da_dst.shape) != (heads, d_head):
        raise ValueError("GAT: dW, da_src, da_dst must have the shapes of W, a_src, a_dst")
    if ws is None:
        ws = _ws(gnn_gat_workspace_size(g, d_in, heads, d_head), X.device)
    _check(lib().gnn_gat_layer_bwd(g.h, _p(X), d_in, _p(W), _p(a_src), _p(a_dst), heads, d_head, float(slope), _p(Y),
                                   _p(dY), _p(saved), _p(dX), _p(dW), _p(da_src), _p(da_dst), _p(ws), ws.numel(),
                                   _stream()))
    return dX, dW, da_src, da_dst


def gat_saved_views(g: Graph, saved, heads, d_head):
    """Views (H', S, D, M, Z) into a GAT forward's saved buffer (the same
    256-byte aligned slices the library carves): M and Z are each
    destination's softmax maximum and 1 / sum of exponentials per head, so
    alpha[e, k] = exp(LReLU(S[src, k] + D[dst, k]) - M[dst, k]) * Z[dst, k]."""
    f = saved.view(torch.float32) if saved.dtype == torch.uint8 else saved
    al = lambda b: (b + 255) // 256 * 256
    n, hd = g.n, heads * d_head
    off = 0
    out = []
    for count, shape in ((n * hd, (n, hd)), (n * heads, (n, heads)), (n * heads, (n, heads)),
                         (n * heads, (n, heads)), (n * heads, (n, heads))):
        out.append(f[off // 4: off // 4 + count].view(*shape))
        off += al(count * 4)
    return tuple(out)


# ---------------------------------------------------------------------------
# kernel timers (measurement)
# ---------------------------------------------------------------------------
def gnn_timer_start(key=None, capacity=4096):
    """Time the launches whose key equals `key` (all instrumented launches
    when None) with HIP events on their streams, until gnn_timer_stop()."""
    _check(lib().gnn_timer_start(None if key is None else key.encode(), int(capacity)))


def gnn_timer_stop():
    _check(lib().gnn_timer_stop())


def gnn_timer_result(key):
    """(launches, total_ms) of the timed launches of `key`."""
    n, ms = C.c_int64(), C.c_double()
    _check(lib().gnn_timer_result(key.encode(), C.byref(n), C.byref(ms)))
    return n.value, ms.value


def gnn_timer_keys():
    buf = C.create_string_buffer(1 << 16)
    _check(lib().gnn_timer_keys(buf, len(buf)))
    return [k for k in buf.value.decode().split("\n") if k]


def gnn_timer_release():
    _check(lib().gnn_timer_release())
