"""Pins of the oracle's quantiser (AdaQP, stochastic integer quantisation,
Eqn. 4-6) and of its counter-based generator (Philox4x32-10)."""
import numpy as np
import pytest

import oracle
from oracle.graph import build_graph


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_range_min_and_error_bound(bits):
    r = np.random.default_rng(bits)
    H = r.standard_normal((64, 32)).astype(np.float32)
    rows = np.arange(0, 64, 3, dtype=np.int32)
    pk, sc, zr = oracle.quantize(H, rows, bits, seed=123)
    q = oracle.unpack_codes(pk, 32, bits)
    assert q.min() >= 0 and q.max() <= 2 ** bits - 1
    for i, v in enumerate(rows):
        assert zr[i] == H[v].min()
        assert q[i, np.argmin(H[v])] == 0
        assert np.isclose(sc[i], (H[v].max() - H[v].min()) / (2 ** bits - 1), rtol=1e-6)
    out = H.copy()
    oracle.dequantize(pk, sc, zr, rows, 32, bits, out)
    err = np.abs(out[rows].astype(np.float64) - H[rows])
    assert np.all(err <= sc[:, None] * (1 + 1e-5) + 1e-6)
    others = np.setdiff1d(np.arange(64), rows)
    assert np.array_equal(out[others], H[others])


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_lossless_grid_rows(bits):
    # rows Z + k*S with S a power of two and both end levels present round-trip exactly
    top = 2 ** bits - 1
    d = 40
    k = np.arange(d) % (top + 1)
    k[0], k[1] = 0, top
    H = np.stack([np.float32(-3.0) + k * np.float32(0.25), np.float32(1.5) + k * np.float32(2.0 ** -6)]).astype(np.float32)
    rows = np.array([0, 1], np.int32)
    pk, sc, zr = oracle.quantize(H, rows, bits, seed=7)
    assert np.array_equal(oracle.unpack_codes(pk, d, bits)[0], k)
    out = np.zeros_like(H)
    oracle.dequantize(pk, sc, zr, rows, d, bits, out)
    assert np.array_equal(out, H)


def test_packing_layout_by_hand():
    # 2-bit codes 0,1,2,3 -> one byte 0b11_10_01_00; 4-bit codes 0..15 pairwise
    H = np.array([[0.0, 1.0, 2.0, 3.0, 3.0, 2.0, 1.0, 0.0]], np.float32)
    pk, _, _ = oracle.quantize(H, np.array([0], np.int32), 2, seed=1)
    assert pk.tolist() == [[0xE4, 0x1B]]
    H4 = np.arange(16, dtype=np.float32)[None]
    pk4, _, _ = oracle.quantize(H4, np.array([0], np.int32), 4, seed=1)
    assert pk4.tolist() == [[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]]


def test_constant_row():
    H = np.full((3, 16), 2.75, np.float32)
    pk, sc, zr = oracle.quantize(H, np.array([1], np.int32), 4, seed=5)
    assert sc[0] == 0.0 and zr[0] == 2.75 and not pk.any()
    out = np.zeros_like(H)
    oracle.dequantize(pk, sc, zr, np.array([1], np.int32), 16, 4, out)
    assert np.all(out[1] == 2.75)


@pytest.mark.parametrize("bits", [2, 8])
def test_unbiased_and_variance(bits):
    # K copies of one row under different node ids draw independent uniforms
    K, d = 4096, 48
    r = np.random.default_rng(100 + bits)
    row = r.standard_normal(d).astype(np.float32)
    H = np.tile(row, (K, 1))
    rows = np.arange(K, dtype=np.int32)
    pk, sc, zr = oracle.quantize(H, rows, bits, seed=99)
    out = np.zeros_like(H)
    oracle.dequantize(pk, sc, zr, rows, d, bits, out)
    S = float(sc[0])
    x = (row.astype(np.float64) - row.min()) / S
    f = x - np.floor(x)
    err = out.astype(np.float64) - row
    var = S * S * f * (1 - f)
    mean = err.mean(0)
    assert np.all(np.abs(mean) <= 4.5 * np.sqrt(var / K) + 1e-6 * S)
    emp = (err ** 2).mean(0)
    assert np.all(np.abs(emp - var) <= 6 * S * S * np.sqrt(1.0 / K) + 1e-6 * S * S)
    assert np.all(var <= S * S / 4 + 1e-12)


def test_row_variance_sixth():
    # with fractional parts spread uniformly the row variance is about D*S^2/6
    K, d = 256, 1024
    r = np.random.default_rng(5)
    H = r.uniform(-1, 1, (K, d)).astype(np.float32)
    rows = np.arange(K, dtype=np.int32)
    pk, sc, zr = oracle.quantize(H, rows, 2, seed=3)
    out = np.zeros_like(H)
    oracle.dequantize(pk, sc, zr, rows, d, 2, out)
    tot = ((out.astype(np.float64) - H) ** 2).sum(1) / (d * sc.astype(np.float64) ** 2)
    assert abs(tot.mean() - 1 / 6) < 0.01


def test_philox_uniformity_and_independence():
    nodes = np.arange(4096, dtype=np.int32)
    u = oracle.philox_uniforms(2024, 0, nodes, 256).ravel()
    assert u.min() >= 0 and u.max() < 1
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))
    counts = np.bincount((u * 256).astype(int), minlength=256)
    exp = u.size / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 255 + 5 * np.sqrt(2 * 255)
    x = u - 0.5
    corr = np.dot(x[:-1], x[1:]) / np.dot(x, x)
    assert abs(corr) < 4 / np.sqrt(u.size)
    # another seed and another stream give other streams
    assert not np.array_equal(u[:256], oracle.philox_uniforms(2025, 0, nodes[:1], 256).ravel())
    assert not np.array_equal(u[:256], oracle.philox_uniforms(2024, 1, nodes[:1], 256).ravel())


def test_philox_avalanche():
    r = np.random.default_rng(17)
    flips = []
    for _ in range(400):
        c = r.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
        k = r.integers(0, 2 ** 32, 2, dtype=np.uint64).astype(np.uint32)
        b = int(r.integers(0, 128))
        c2 = c.copy()
        c2[b // 32] ^= np.uint32(1 << (b % 32))
        o1 = oracle.philox4x32_10(c, k)
        o2 = oracle.philox4x32_10(c2, k)
        flips.append(sum(bin(int(a ^ bb)).count("1") for a, bb in zip(o1, o2)) / 128)
    assert abs(np.mean(flips) - 0.5) < 0.02


def test_signed_zero_extremes():
    # of two equal zeros the minimum is -0 and the maximum +0, whatever the order
    H = np.array([[0.0, -0.0, 0.0, 0.0], [-0.0, 0.0, -0.0, -0.0]], np.float32)
    H[:, 0] = np.array([0.0, -0.0], np.float32)
    pk, sc, zr = oracle.quantize(np.vstack([H, [[1.0, -0.0, 0.0, 2.0]]]).astype(np.float32),
                                 np.array([0, 1, 2], np.int32), 8, seed=1)
    assert np.signbit(zr[0]) and np.signbit(zr[1]) and sc[0] == 0 and sc[1] == 0
    assert zr[2] == 0.0 and np.signbit(zr[2])


# ---------------------------------------------------------------------------
# bit-width statistics and the greedy assignment (AdaQP Sec. 3.2, Problem 11)
# ---------------------------------------------------------------------------
def test_quant_stats_closed_form_on_a_star():
    # star: hub 0 joined to 1..4, symmetrised with self-loops; the hub's row
    # degree is 5, a leaf's 2.  The hub's out-edges carry 1/sqrt(5*2) to each
    # leaf and 1/5 to itself: S2 = 4/10 + 1/25.  A leaf's carry 1/sqrt(10) to
    # the hub and 1/2 to itself: S2 = 1/10 + 1/4.
    from oracle.graph import build_graph
    g = build_graph(np.zeros(4, np.int64), np.arange(1, 5), 5, True)
    H = np.array([[0, 1, 3, -1], [2, 2, 2, 2], [0, 0, 0, 4], [1, 2, 3, 4], [5, -5, 0, 0]], np.float32)
    beta, rng = oracle.quant_stats(g, H, np.array([0, 1, 2]))
    assert np.array_equal(rng, np.array([4, 0, 4], np.float32))
    assert np.allclose(beta, [(0.4 + 0.04) * 4 * 16 / 6, 0.0, (0.1 + 0.25) * 4 * 16 / 6], rtol=1e-6)


def test_quant_variance_matches_measured_error():
    # beta / (2^b - 1)^2 with unit weights (S2 = 1) is D R^2 / (6 (2^b-1)^2),
    # the squared error stochastic rounding leaves in a row whose values are
    # spread evenly: compare with the oracle quantiser's measured error
    K, d = 200, 512
    r = np.random.default_rng(8)
    H = (r.uniform(-1, 1, (K, d)) * r.uniform(0.1, 3, (K, 1))).astype(np.float32)
    rows = np.arange(K, dtype=np.int32)
    rng = (H.max(1) - H.min(1)).astype(np.float64)
    beta = d * rng ** 2 / 6
    for b in (2, 4, 8):
        pk, sc, zr = oracle.quantize(H, rows, b, seed=9)
        out = np.zeros_like(H)
        oracle.dequantize(pk, sc, zr, rows, d, b, out)
        err = float(((out.astype(np.float64) - H) ** 2).sum())
        assert abs(err / oracle.quant_variance(beta, np.full(K, b)) - 1.0) < 0.03, b


def test_greedy_worked_example():
    # d = 4, budget avg 4 bits over 3 rows = 3 units of d/4 bytes:
    # upgrades by variance removed per unit: row 0 2->4 (9*0.1067), row 1
    # 2->4 (0.1067), row 0 4->8 (0.0199, needs 2 units: no longer fits), row 2
    # 2->4 (0, fits)
    assert list(oracle.assign_bits_greedy([9.0, 1.0, 0.0], 4, 4.0)) == [4, 4, 4]
    assert list(oracle.assign_bits_greedy([9.0, 1.0, 0.0], 4, 2.0)) == [2, 2, 2]
    assert list(oracle.assign_bits_greedy([9.0, 1.0, 0.0], 4, 8.0)) == [8, 8, 8]
    # 3 units over two rows: row 1's 2->4 (0.107 per unit) beats row 0's 4->8
    # (0.020 per unit), which then no longer fits; with beta 1000 it is the
    # other way round (2.21 per unit)
    assert list(oracle.assign_bits_greedy([9.0, 1.0], 4, 5.0)) == [4, 4]
    assert list(oracle.assign_bits_greedy([1000.0, 1.0], 4, 5.0)) == [8, 2]


def test_greedy_against_brute_force():
    # on tiny instances: within budget, monotone in the budget, and never worse
    # than the best assignment that leaves out one 4->8 upgrade's worth
    import itertools
    r = np.random.default_rng(5)
    cost = {2: 0, 4: 1, 8: 3}
    for _ in range(300):
        m = int(r.integers(1, 6))
        d = 8
        beta = r.exponential(1.0, m) * (r.random(m) < 0.9)
        avg = 2 + 6 * r.random()
        units = int(np.floor((avg - 2) * m / 2 + 1e-9))
        b = oracle.assign_bits_greedy(beta, d, avg)
        assert sum(cost[int(x)] for x in b) <= units
        more = oracle.assign_bits_greedy(beta, d, min(8.0, avg + 2.0 / m))
        assert oracle.quant_variance(beta, more) <= oracle.quant_variance(beta, b) + 1e-15
        best = min(oracle.quant_variance(beta, c) for c in itertools.product((2, 4, 8), repeat=m)
                   if sum(cost[x] for x in c) <= max(units - 2, 0))
        assert oracle.quant_variance(beta, b) <= best * (1 + 1e-12) + 1e-15


# ---------------------------------------------------------------------------
# Tango's symmetric tensor-level 8-bit quantisation and quantisation-aware GEMM
# ---------------------------------------------------------------------------
def test_sym8_integer_grid_is_exact():
    # max |X| = 127 makes the scale 1 (127/127) and every integer in range its
    # own code: no randomness left, and the GEMM is the exact integer product
    r = np.random.default_rng(50)
    A = r.integers(-127, 128, (33, 70)).astype(np.float32)
    A[0, 0] = 127
    B = r.integers(-127, 128, (70, 19)).astype(np.float32)
    B[3, 2] = -127
    C, qa, qb, sa, sb = oracle.gemm_q8(A, B, seed=1)
    assert sa == 1.0 and sb == 1.0
    assert np.array_equal(qa, A.astype(np.int8)) and np.array_equal(qb, B.astype(np.int8))
    assert np.array_equal(C, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float32))


def test_sym8_zero_tensor():
    C, qa, qb, sa, sb = oracle.gemm_q8(np.zeros((5, 8), np.float32), np.ones((8, 3), np.float32), seed=2)
    assert sa == 0.0 and not qa.any() and not C.any()


def test_sym8_unbiased_and_within_one_step():
    # stochastic rounding: every dequantised value within one step of the
    # input, and the mean over independent draws converges to it
    r = np.random.default_rng(51)
    X = r.standard_normal((16, 64)).astype(np.float32)
    acc = np.zeros(X.shape)
    K = 400
    for seed in range(K):
        q, s = oracle.quantize_sym8(X, seed)
        deq = q.astype(np.float64) * s
        assert np.all(np.abs(deq - X) <= s * (1 + 1e-6))
        acc += deq
    s = np.abs(X).max() / 127
    assert np.all(np.abs(acc / K - X) <= 5 * s * 0.5 / np.sqrt(K))
    assert q.min() >= -127 and q.max() <= 127


def test_q8_gemm_error_bound():
    # |C - A B| <= sum_k (|a| s_B + |b| s_A + s_A s_B) plus the final rounding
    r = np.random.default_rng(52)
    A = r.standard_normal((40, 128)).astype(np.float32)
    B = r.standard_normal((128, 30)).astype(np.float32)
    C, qa, qb, sa, sb = oracle.gemm_q8(A, B, seed=3)
    bound = (np.abs(A) @ np.ones_like(B)) * sb + (np.ones_like(A) @ np.abs(B)) * sa + A.shape[1] * sa * sb
    ref = A.astype(np.float64) @ B
    assert np.all(np.abs(C - ref) <= bound + 1e-6 * np.abs(ref))


# ---------------------------------------------------------------------------
# Tango's SDDMM dot on quantised inputs
# ---------------------------------------------------------------------------
def _small_graph(seed, n=40, m=300):
    r = np.random.default_rng(seed)
    return build_graph(r.integers(0, n, m).astype(np.int32), r.integers(0, n, m).astype(np.int32), n, False)


def test_sddmm_q8_integer_grid_is_exact_dot():
    # integer features with max |x| = 127: scale 1, codes = values, and the
    # quantised SDDMM is the exact SDDMM dot, per head, on every edge
    g = _small_graph(60)
    r = np.random.default_rng(61)
    heads, dh = 3, 16
    S = r.integers(-127, 128, (g.n, heads * dh)).astype(np.float32)
    D = r.integers(-127, 128, (g.n, heads * dh)).astype(np.float32)
    S[1, 2], D[4, 5] = 127, -127
    out, qs, qd, ss, sd = oracle.sddmm_q8(g, S, D, heads, seed=7)
    assert ss == 1.0 and sd == 1.0
    ref = oracle.sddmm_dot(g, D, S, heads)  # out[e] = <S[src], D[dst]>
    assert np.array_equal(out, ref.astype(np.float32))
    # brute force over the edge list
    for e in range(0, g.nnz, 37):
        u, v = g.col[e], g.dst[e]
        for k in range(heads):
            sl = slice(k * dh, (k + 1) * dh)
            assert out[e, k] == float(np.dot(S[u, sl].astype(np.int64), D[v, sl].astype(np.int64)))


def test_sddmm_q8_streams_and_error_bound():
    g = _small_graph(62)
    r = np.random.default_rng(63)
    heads, dh = 2, 32
    S = r.standard_normal((g.n, heads * dh)).astype(np.float32)
    D = r.standard_normal((g.n, heads * dh)).astype(np.float32)
    out, qs, qd, ss, sd = oracle.sddmm_q8(g, S, D, heads, seed=9, stream=4)
    # the operands' codes are quantize_sym8 on streams s and s + 1
    q1, s1 = oracle.quantize_sym8(S, 9, 4)
    q2, s2 = oracle.quantize_sym8(D, 9, 5)
    assert np.array_equal(qs, q1) and np.array_equal(qd, q2) and ss == s1 and sd == s2
    # |out - exact| <= sum_j (|a| s_D + |b| s_S + s_S s_D) per head, plus the final rounding
    ref = oracle.sddmm_dot(g, D, S, heads)
    aS = np.abs(S).reshape(g.n, heads, dh).sum(-1)
    aD = np.abs(D).reshape(g.n, heads, dh).sum(-1)
    bound = aS[g.col] * sd + aD[g.dst] * ss + dh * ss * sd
    assert np.all(np.abs(out - ref) <= bound + 1e-6 * np.abs(ref))


def test_sddmm_q8_zero_operand():
    g = _small_graph(64)
    out, qs, qd, ss, sd = oracle.sddmm_q8(g, np.zeros((g.n, 16), np.float32), np.ones((g.n, 16), np.float32), 1, 3)
    assert ss == 0.0 and not out.any()
