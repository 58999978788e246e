"""Host C++ of the graph build under AddressSanitizer + UndefinedBehaviorSanitizer.

The graph build (CSR by destination with one self-loop per node, Sancus Sec. 2;
reverse edges for symmetrised inputs, Tango's dataset preparation; the CSC
view and the degree order) is plain host C++.  This test compiles it with g++
and both sanitizers next to a small driver that checks random edge lists
(loops, repeats, a hub node, up to 150K nodes so the threaded path runs)
against adjacency sets, and that out-of-range ids are refused.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "sparse_message_passing_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_graph_build_under_sanitizers(tmp_path):
    exe = str(tmp_path / "graph_build_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", CSRC,
           os.path.join(HERE, "host", "graph_build_check.cpp"), os.path.join(CSRC, "graph_build.cpp"),
           "-o", exe, "-lpthread"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and "asan" in (b.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + b.stderr[-300:])
    assert b.returncode == 0, b.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "bad=0" in r.stdout, (r.stdout[-1000:], r.stderr[-3000:])
