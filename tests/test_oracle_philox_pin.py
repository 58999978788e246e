"""Pin of the oracle's Philox4x32-10 against an independent implementation.

The stochastic rounding of AdaQP's per-row quantiser (Eqn. 4, round_st)
needs one uniform per element; the build draws it from Philox4x32-10
(Salmon et al., SC'11) at key (seed low, seed high), counter
(node, feature / 4, stream, 0), output word feature mod 4, scaled as
(word >> 8) * 2^-24.  The oracle implements the round function from the
published definition; here it is compared word for word with rocRAND's
engine, a separate implementation that ships as C++ source with ROCm,
compiled on the host and driven only through its seed / subsequence /
skip-ahead interface (tests/host/philox_rocrand.cpp).  A wrong multiplier
word, a swapped product half, a misplaced key bump or a wrong round count
in the oracle fails here.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    if not os.path.exists(HEADER) or shutil.which("g++") is None:
        pytest.skip("rocRAND's source header or g++ is not installed")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_rocrand")
    subprocess.run(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HERE, "host", "philox_rocrand.cpp"), "-o", exe], check=True)

    def run(seed, stream, node, block):
        lines = "".join(f"{int(s)} {int(t)} {int(n)} {int(b)}\n" for s, t, n, b in zip(seed, stream, node, block))
        out = subprocess.run([exe], input=lines, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w) for w in l.split()] for l in out.splitlines()], dtype=np.uint64).astype(np.uint32)

    return run


def _cases(n, seed):
    g = np.random.default_rng(seed)
    seeds = g.integers(0, 2**64, n, dtype=np.uint64)
    seeds[:8] = [0, 1, 2**32 - 1, 2**32, 2**32 + 1, 2**63, 2**64 - 1, 0x123456789ABCDEF0]
    streams = g.integers(0, 2**32, n, dtype=np.uint64)
    streams[8:16] = [0, 1, 2, 2**31, 2**32 - 1, 0, 1, 7]
    streams[16:200] = g.integers(0, 4, 184)
    nodes = g.integers(0, 2**31, n, dtype=np.uint64)
    nodes[:16] = [0, 1, 2**31 - 1, 2**31 - 2, 2**30, 12345, 2**31 - 1, 0, 1, 2, 3, 2**20, 2**21 - 1, 2450000 - 1,
                  2**31 - 3, 314572]
    blocks = g.integers(0, 2**32, n, dtype=np.uint64)
    blocks[:300] = g.integers(0, 64, 300)          # features 0 .. 255 at 4 per counter
    return seeds, streams, nodes, blocks


def test_philox_words_match_rocrand(rocrand_philox):
    seeds, streams, nodes, blocks = _cases(2000, 20231)
    ref = rocrand_philox(seeds, streams, nodes, blocks)
    got = np.empty_like(ref)
    for i in range(seeds.size):
        s = int(seeds[i])
        got[i] = oracle.philox4x32_10([int(nodes[i]), int(blocks[i]), int(streams[i]), 0],
                                      [s & 0xFFFFFFFF, s >> 32])
    bad = np.nonzero(np.any(got != ref, axis=1))[0]
    assert bad.size == 0, f"{bad.size} of {seeds.size} counters differ, first at case {bad[:5]}"


@pytest.mark.parametrize("seed,stream", [(6006, 0), (6006, 1), (2**40 + 77, 5), (2**64 - 1, 2**32 - 1)])
def test_quantiser_uniforms_match_rocrand(rocrand_philox, seed, stream):
    """The uniforms the quantiser draws: counter (node, f/4, stream, 0),
    word f mod 4, u = (word >> 8) 2^-24, for every feature of a 256-wide row."""
    d = 256
    nodes = np.array([0, 1, 1000, 314572, 2**21 - 1, 2**31 - 1], dtype=np.int32)
    u = oracle.philox_uniforms(seed, stream, nodes, d)
    nn = np.repeat(nodes.astype(np.uint64), d // 4)
    bb = np.tile(np.arange(d // 4, dtype=np.uint64), nodes.size)
    words = rocrand_philox(np.full(nn.size, seed, np.uint64), np.full(nn.size, stream, np.uint64), nn, bb)
    words = words.reshape(nodes.size, d // 4, 4).reshape(nodes.size, d)
    ref = (words >> 8).astype(np.float64) * 2.0**-24
    assert np.array_equal(u.astype(np.float64), ref)
