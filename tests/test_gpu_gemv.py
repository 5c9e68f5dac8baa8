"""Parity of the HIP matrix-vector kernels (Q4_0, Q8_0, Q4_K, Q6_K, gated pair)
with the float64 oracle, element by element, through the C ABI.

Bar: |y - y_ref| <= 1e-5 * sum_i |w_i x_i| + 1e-6 for every output; the
gated pair uses the first-order propagation of that bound (oracle.geglu_tol).
"""
import numpy as np
import pytest

import oracle
from quantized_dequant_matrix_amd import synth
from gpu_util import assert_within, dev, empty, host, say

pytestmark = pytest.mark.gpu

FMTS = ["q4_0", "q8_0", "q4_k", "q6_k"]


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


def run_gemv(fmt, W, x, N, K, M=1):
    qmv = _qmv()
    y = empty((M, N))
    getattr(qmv, "qmv_" + fmt)(dev(W), dev(x), y, N, K, M)
    return host(y)


# (N, K): tails in N, K on and off the 256-weight units, the unit-kernel
# limit K = 16128 and just past it, and the workload shapes.
SHAPES = [(1, 256), (5, 512), (64, 256), (65, 256), (3, 768), (100, 1024), (33, 4096), (129, 5376),
          (17, 16128), (9, 16384), (8, 16640), (7, 32), (11, 96), (13, 5408), (257, 2048)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_shapes(fmt, N, K):
    if fmt in ("q4_k", "q6_k") and K % 256:
        pytest.skip("Q4_K and Q6_K need K % 256 == 0")
    seed = 7 * N + K
    say(f"qmv_{fmt} N={N} K={K} seed={seed}")
    W, x = synth.problem(fmt, N, K, 1, seed)
    y = run_gemv(fmt, W, x, N, K)
    yr, S = oracle.qmv(fmt, W, N, K, x)
    assert_within(y, yr, oracle.float_tol(S), f"qmv_{fmt} {N}x{K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_batched_rows(fmt):
    N, K, M = 77, 1280, 3
    say(f"qmv_{fmt} M={M}")
    W, x = synth.problem(fmt, N, K, M, 99)
    y = run_gemv(fmt, W, x, N, K, M)
    yr, S = oracle.qmv(fmt, W, N, K, x, M=M)
    assert_within(y, yr, oracle.float_tol(S), f"qmv_{fmt} M={M}")


@pytest.mark.parametrize("name,fmt", [("c1", "q4_0"), ("c2", "q4_0"), ("c5", "q4_k"), ("q6k_gate", "q6_k")])
def test_workloads_full(name, fmt):
    c = synth.CONFIGS[name]
    say(f"qmv_{fmt} workload {name} N={c['N']} K={c['K']}")
    W, x = synth.config_problem(name)
    y = run_gemv(fmt, W, x, c["N"], c["K"])
    yr, S = oracle.qmv(fmt, W, c["N"], c["K"], x)
    w = assert_within(y, yr, oracle.float_tol(S), name)
    say(f"{name}: worst err/tol {w:.3g}")


def test_logit_workload_rows_sampled():
    # the 262,144 x 5376 Q8_0 GEMV itself (the top-k test checks all rows)
    c = synth.CONFIGS["c3"]
    say("qmv_q8_0 logit workload, 4096 sampled rows")
    W, x = synth.config_problem("c3")
    y = run_gemv("q8_0", W, x, c["N"], c["K"])
    rows = np.random.default_rng(0).choice(c["N"], 4096, replace=False)
    yr, S = oracle.qmv("q8_0", W, c["N"], c["K"], x, rows=rows)
    assert_within(y[:, rows], yr, oracle.float_tol(S), "c3 rows")


@pytest.mark.parametrize("fmt,K", [("q4_0", 512), ("q8_0", 512), ("q4_k", 512), ("q6_k", 512), ("q6_k", 768),
                                   ("q4_0", 96), ("q8_0", 160)])
def test_unit_vectors_give_columns(fmt, K):
    N = 70
    say(f"qmv_{fmt} unit vectors K={K}")
    W, _ = synth.problem(fmt, N, K, 1, 5)
    rb = oracle.row_bytes(fmt, K)
    cols = [c for c in (0, 1, 15, 16, 17, 31, 32, 255) if c < K] + [K - 1]
    E = np.zeros((len(cols), K), dtype=np.float32)
    for j, i in enumerate(cols):
        E[j, i] = 1.0
    y = run_gemv(fmt, W, E, N, K, len(cols))
    dq = np.stack([oracle.dequant_row(fmt, W[n * rb:(n + 1) * rb], K) for n in range(N)])
    ref = dq[:, cols].T
    if fmt in ("q4_k", "q6_k"):
        # d*scale*q - dmin*min, and d*scale*(q - 32) (up to 25 significant
        # bits), are exact in float64 and rounded once to float32
        ref = ref.astype(np.float32)
    assert np.array_equal(y, ref)


# Rows longer than 63 units take the split kernel (K sliced across the
# waves of a workgroup): 64 and 65 units, the FFN down shape's 84 (with row
# tails around its 12 rows per pass), the largest K whose activations fit in
# LDS (157 units) and one past it (generic kernel).
LONG = [(37, 16384), (41, 16640), (1, 21504), (12, 21504), (13, 21504), (29, 21504), (13, 40192), (11, 40448)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", LONG)
def test_long_rows(fmt, N, K):
    seed = 3 * N + K
    say(f"qmv_{fmt} long rows N={N} K={K} seed={seed}")
    W, x = synth.problem(fmt, N, K, 1, seed)
    y = run_gemv(fmt, W, x, N, K)
    yr, S = oracle.qmv(fmt, W, N, K, x)
    assert_within(y, yr, oracle.float_tol(S), f"qmv_{fmt} {N}x{K}")


# More row groups per workgroup than its LDS holds slice sums for: at
# K = 40192 the activations fill 163 KB of LDS, room is left for 14 groups of
# 2 rows, and 9001 rows give each of the 256 workgroups 17 or 18 groups, so
# the split kernel takes its range in two chunks (the second partial) and the
# last group has one row.
@pytest.mark.parametrize("fmt", FMTS)
def test_long_rows_chunked(fmt):
    N, K = 9001, 40192
    say(f"qmv_{fmt} split kernel in chunks N={N} K={K}")
    W, x = synth.problem(fmt, N, K, 1, 4242)
    y = run_gemv(fmt, W, x, N, K)
    yr, S = oracle.qmv(fmt, W, N, K, x)
    assert_within(y, yr, oracle.float_tol(S), f"qmv_{fmt} {N}x{K}")


@pytest.mark.parametrize("name,fmt", [("c4", "q4_0"), ("q4k_down", "q4_k"), ("q6k_down", "q6_k")])
def test_down_shape_full(name, fmt):
    c = synth.CONFIGS[name]
    say(f"qmv_{fmt} down shape {c['N']}x{c['K']}")
    W, x = synth.config_problem(name, M=1)
    y = run_gemv(fmt, W, x, c["N"], c["K"])
    yr, S = oracle.qmv(fmt, W, c["N"], c["K"], x)
    w = assert_within(y, yr, oracle.float_tol(S), name)
    say(f"{name}: worst err/tol {w:.3g}")


def test_long_rows_deterministic_and_batched():
    N, K, M = 300, 21504, 2
    say("qmv_q6_k split kernel: M=2, 5 repeats bit-identical")
    qmv = _qmv()
    W, x = synth.problem("q6_k", N, K, M, 5)
    Wd, xd = dev(W), dev(x)
    outs = []
    for _ in range(5):
        y = empty((M, N))
        qmv.qmv_q6_k(Wd, xd, y, N, K, M)
        outs.append(host(y))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    yr, S = oracle.qmv("q6_k", W, N, K, x, M=M)
    assert_within(outs[0], yr, oracle.float_tol(S), "split M=2")


def test_q6_k_extreme_codes_and_scales():
    # q in {0, 63} and scales in {-128, 127}: the largest products the
    # signed-byte decode forms; rows alternate the super-block alignment
    N, K = 37, 2304
    say("qmv_q6_k extreme codes and scales")
    rng = np.random.default_rng(21)
    nb = N * K // 256
    q = rng.choice(np.array([0, 63, 32, 31, 33], np.uint8), size=(nb, 256))
    sc = rng.choice(np.array([-128, 127, -1, 0], np.int8), size=(nb, 16))
    d = (np.abs(rng.standard_normal(nb)) * 1e-4).astype(np.float16)
    W = synth.pack_q6_k(d, sc, q)
    x = rng.standard_normal((1, K)).astype(np.float32)
    y = run_gemv("q6_k", W, x, N, K)
    yr, S = oracle.qmv("q6_k", W, N, K, x)
    assert_within(y, yr, oracle.float_tol(S), "q6_k extremes")


def test_zero_weights_exactly_zero():
    N, K = 50, 5376
    say("qmv_q4_0 all-zero weights")
    blk = np.frombuffer(np.array([3.0], np.float16).tobytes() + bytes([0x88] * 16), np.uint8)
    W = np.tile(blk, N * K // 32)
    x = np.random.default_rng(1).standard_normal((1, K)).astype(np.float32) * 1e3
    y = run_gemv("q4_0", W, x, N, K)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [768, 21504])  # unit kernel; split kernel (slice sums met in LDS)
def test_non_finite_activations(fmt, K):
    """IEEE semantics as in the float64 oracle: an infinite activation gives
    +-inf in the rows whose weight there is nonzero and NaN (inf * 0) where it
    is zero; a NaN activation makes every row NaN.  The finite entries keep
    the usual bound."""
    N = 96
    say(f"qmv_{fmt} non-finite activations")
    W, x = synth.problem(fmt, N, K, 1, 31)
    for pos, val in ((5, np.inf), (300, -np.inf), (17, np.nan)):
        xs = x.copy()
        xs[0, pos] = val
        y = run_gemv(fmt, W, xs, N, K)[0]
        with np.errstate(invalid="ignore", over="ignore"):
            yr, S = oracle.qmv(fmt, W, N, K, xs)
        yr = yr[0]
        assert np.array_equal(np.isnan(y), np.isnan(yr)), (fmt, pos)
        assert np.array_equal(np.isposinf(y), np.isposinf(yr)), (fmt, pos)
        assert np.array_equal(np.isneginf(y), np.isneginf(yr)), (fmt, pos)
        fin = np.isfinite(yr)
        if fin.any():
            assert_within(y[None, fin], yr[None, fin], oracle.float_tol(S[0][fin])[None, :], f"{fmt} finite rows")


def test_wide_dynamic_range():
    N, K = 40, 4096
    say("qmv wide dynamic range activations")
    for fmt in FMTS:
        W, x = synth.problem(fmt, N, K, 1, 3)
        x = (x * (10.0 ** np.random.default_rng(2).uniform(-15, 15, x.shape))).astype(np.float32)
        y = run_gemv(fmt, W, x, N, K)
        yr, S = oracle.qmv(fmt, W, N, K, x)
        assert_within(y, yr, oracle.float_tol(S), f"{fmt} dynamic range")


def test_deterministic_repeats():
    c = synth.CONFIGS["c2"]
    say("qmv_q4_0 20 repeats, bit identity")
    qmv = _qmv()
    W, x = synth.config_problem("c2")
    Wd, xd = dev(W), dev(x)
    outs = []
    for _ in range(20):
        y = empty((1, c["N"]))
        qmv.qmv_q4_0(Wd, xd, y, c["N"], c["K"], 1)
        outs.append(host(y))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# ------------------------------------------------------------ gated pair
def run_geglu(Wg, Wu, x, N, K, M=1):
    qmv = _qmv()
    h = empty((M, N))
    qmv.qmv_q4_0_geglu(dev(Wg), dev(Wu), dev(x), h, N, K, M)
    return host(h)


def geglu_ref(Wg, Wu, x, N, K, M=1):
    g, Sg = oracle.qmv("q4_0", Wg, N, K, x, M=M)
    u, Su = oracle.qmv("q4_0", Wu, N, K, x, M=M)
    h = oracle.geglu(g, u).reshape(g.shape)
    return h, oracle.geglu_tol(g, u, Sg, Su, h)


@pytest.mark.parametrize("N,K", [(1, 256), (65, 5376), (7, 96), (31, 16640), (300, 4096)])
def test_geglu_shapes(N, K):
    say(f"qmv_q4_0_geglu N={N} K={K}")
    Wg, x = synth.problem("q4_0", N, K, 1, N + K)
    Wu = synth.q4_0_weights(N, K, N + K + 1)
    h = run_geglu(Wg, Wu, x, N, K)
    hr, tol = geglu_ref(Wg, Wu, x, N, K)
    assert_within(h, hr, tol, f"geglu {N}x{K}")


def test_geglu_batched_and_large_gate():
    N, K, M = 50, 1024, 2
    say("qmv_q4_0_geglu M=2, large gate values")
    Wg, x = synth.problem("q4_0", N, K, M, 11)
    Wu = synth.q4_0_weights(N, K, 12)
    x[1] *= 1e4          # pushes g far into both saturated ends of gelu
    h = run_geglu(Wg, Wu, x, N, K, M)
    hr, tol = geglu_ref(Wg, Wu, x, N, K, M)
    assert np.all(np.isfinite(h))
    assert_within(h, hr, tol, "geglu batched")


def test_geglu_non_finite():
    # gelu(+inf) = +inf and gelu(-inf) = -inf * 0 = NaN in the float64 tanh
    # form; with u = +-inf or NaN the product classes follow.  Same on the GPU.
    N, K = 64, 5376
    say("qmv_q4_0_geglu non-finite activations")
    Wg, x = synth.problem("q4_0", N, K, 1, 71)
    Wu = synth.q4_0_weights(N, K, 72)
    for pos, val in ((11, np.inf), (2000, -np.inf), (37, np.nan)):
        xs = x.copy()
        xs[0, pos] = val
        h = run_geglu(Wg, Wu, xs, N, K)[0]
        with np.errstate(invalid="ignore", over="ignore"):
            hr, _ = geglu_ref(Wg, Wu, xs, N, K)
        hr = hr.reshape(-1)
        assert np.array_equal(np.isnan(h), np.isnan(hr)), pos
        assert np.array_equal(np.isposinf(h), np.isposinf(hr)), pos
        assert np.array_equal(np.isneginf(h), np.isneginf(hr)), pos


def test_geglu_workload_full():
    c = synth.CONFIGS["c2"]
    say("qmv_q4_0_geglu workload pair 21504x5376")
    Wg, Wu, x = synth.gate_up_problem()
    h = run_geglu(Wg, Wu, x, c["N"], c["K"])
    hr, tol = geglu_ref(Wg, Wu, x, c["N"], c["K"])
    w = assert_within(h, hr, tol, "c2 pair")
    say(f"c2 pair: worst err/tol {w:.3g}")
