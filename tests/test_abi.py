"""The C-ABI library loads and exports every entry point its header declares
(no compute calls: this runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gnnmp.h")
LIB = os.path.join(ROOT, "sparse_message_passing_amd", "libgnnmp.so")


def declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gnn_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = declared()
    for must in ("gnn_graph_create", "gnn_spmm", "gnn_sddmm", "gnn_edge_softmax", "gnn_edge_softmax_bwd",
                 "gnn_edge_reduce", "gnn_gemm", "gnn_quantize", "gnn_dequantize", "gnn_softmax_xent",
                 "gnn_gcn_layer_fwd", "gnn_gcn_layer_bwd", "gnn_gat_layer_fwd", "gnn_gat_layer_bwd",
                 "gnn_quant_slots", "gnn_spmm_dequant"):
        assert must in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgnnmp.so not built")
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(L, n)]
    assert not missing, missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgnnmp.so not built")
def test_binding_covers_every_declared_symbol():
    from sparse_message_passing_amd import gnnmp
    assert set(declared()) <= set(gnnmp.EXPORTED)


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgnnmp.so not built")
def test_status_strings_and_host_side_validation():
    # argument checks run before any HIP call, so they work without a GPU
    from sparse_message_passing_amd import gnnmp
    L = gnnmp.lib()
    assert L.gnn_status_string(0) == b"ok"
    assert L.gnn_status_string(6) == b"workspace too small"
    # bits not in {2, 4, 8}
    st = L.gnn_quantize(None, 4, 4, None, 1, 3, 0, 0, None, None, None, None)
    assert st == 1 and b"bits" in L.gnn_last_error()
    # ldh < d
    st = L.gnn_dequantize(None, None, None, 1, 8, 4, None, None, 4, None)
    assert st == 1 and b"ldh" in L.gnn_last_error()
    # d*bits not a multiple of 8
    st = L.gnn_quantize(None, 3, 3, None, 1, 2, 0, 0, None, None, None, None)
    assert st == 1
    # NULL graph handle
    st = L.gnn_spmm(None, 0, 0, None, 1, None, 0, 4, None, 0, 4, 4, 0, None, 0, None)
    assert st == 1 and b"NULL" in L.gnn_last_error()
    # gemm: negative size / lda too small / unknown dtype
    assert L.gnn_gemm(0, 0, -1, 1, 1, None, 0, 1, None, 0, 1, None, 0, 1, None, 0, None) == 1
    assert L.gnn_gemm(0, 0, 4, 4, 8, None, 0, 4, None, 0, 4, None, 0, 4, None, 0, None) == 1
    assert L.gnn_gemm(0, 0, 4, 4, 4, None, 7, 4, None, 0, 4, None, 0, 4, None, 0, None) == 1
    # softmax-xent workspace too small
    st = L.gnn_softmax_xent(1, 10, 3, 3, 1, 1, None, 3, 1, 0, None)
    assert st == 6
    # graph creation: out NULL, negative n, unknown flags, id out of range (host-side build)
    assert L.gnn_graph_create(4, 0, None, None, 0, None) == 1
    h = ctypes.c_void_p()
    assert L.gnn_graph_create(-1, 0, None, None, 0, ctypes.byref(h)) == 1
    assert L.gnn_graph_create(4, 0, None, None, 0x10, ctypes.byref(h)) == 1
    import numpy as np
    s = np.array([0, 9], np.int32)
    t = np.array([1, 1], np.int32)
    st = L.gnn_graph_create(4, 2, s.ctypes.data, t.ctypes.data, 0, ctypes.byref(h))
    assert st == 1 and b"out of range" in L.gnn_last_error()
    # slot map: more than 8 groups; negative n
    assert L.gnn_quant_slots(4, 9, None, None, None, None) == 1
    assert L.gnn_quant_slots(-1, 0, None, None, None, None) == 1
    # dequantising aggregation: NULL graph; then d not a multiple of 4 is checked after the graph
    st = L.gnn_spmm_dequant(None, None, 4, None, None, 0, None, 0, None, 4, 4, 0, None, 0, None)
    assert st == 1 and b"NULL" in L.gnn_last_error()


def test_binding_refuses_wrong_dtypes_before_the_library():
    # float* entry points must never receive a bf16 (or integer) buffer: the
    # kernels would read and write past its end.  The binding checks first,
    # so this runs without a GPU (the tensors never reach the library).
    import torch
    from sparse_message_passing_amd import gnnmp
    bf = torch.zeros((4, 16), dtype=torch.bfloat16)
    f = torch.zeros((4, 16))
    rows = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(TypeError):
        gnnmp.gnn_gemm_q8(bf, f.T, f[:, :4], seed=0)
    with pytest.raises(TypeError):
        gnnmp.gnn_gemm_q8(f, f.T, bf[:, :4], seed=0)
    with pytest.raises(TypeError):
        gnnmp.gnn_sddmm_q8(None, bf, f, 1, 16, f, seed=0)
    with pytest.raises(TypeError):
        gnnmp.gnn_quantize(bf, rows, 8, 0, None, f, f)
    with pytest.raises(TypeError):
        gnnmp.gnn_quantize(f, rows.long(), 8, 0, None, f, f)
    with pytest.raises(TypeError):
        gnnmp.gnn_edge_softmax(None, bf, f)
    with pytest.raises(TypeError):
        gnnmp.gnn_gcn_layer_fwd(None, f, bf, f, True)
