"""Seeded sweep of random small shapes through every matrix-vector entry
point (all formats, the gated pair, the gated down projection, the QKV
launch), each compared with the float64 oracle element by element.  Shapes
are drawn so that N, K and M land on and off every tile and unit boundary
the kernels use (units of 256, rows per pass, long rows past 63 units)."""
import numpy as np
import pytest

import oracle
from quantized_dequant_matrix_amd import synth
from gpu_util import assert_within, dev, empty, host, say

pytestmark = pytest.mark.gpu


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


def draw(rng, fmt):
    unit = 256 if fmt in ("q4_k", "q6_k") else 32
    kind = rng.integers(0, 3)
    if kind == 0:
        K = unit * int(rng.integers(1, 24))            # short rows
    elif kind == 1:
        K = 256 * int(rng.integers(1, 64))             # unit kernel
    else:
        K = 256 * int(rng.integers(64, 100))           # split kernel
    if unit == 32 and rng.integers(0, 2):
        K += 32 * int(rng.integers(1, 8))              # K % 256 != 0
    N = int(rng.integers(1, 400))
    M = int(rng.integers(1, 4))
    return N, K, M


CASES = [(fmt, seed) for fmt in ("q4_0", "q8_0", "q4_k", "q6_k", "mxfp4") for seed in range(6)]


@pytest.mark.parametrize("fmt,seed", CASES)
def test_gemv_random(fmt, seed):
    rng = np.random.default_rng(1000 + seed)
    N, K, M = draw(rng, fmt)
    say(f"random qmv_{fmt} N={N} K={K} M={M} seed={seed}")
    qmv = _qmv()
    y = empty((M, N))
    if fmt == "mxfp4":
        codes, scales, x = synth.mxfp4_problem(N, K, M, 7 + seed)
        qmv.qmv_mxfp4(dev(codes), dev(scales), dev(x), y, N, K, M)
        yr, S = oracle.qmv_mxfp4(codes, scales, N, K, x, M=M)
    else:
        W, x = synth.problem(fmt, N, K, M, 7 + seed)
        getattr(qmv, "qmv_" + fmt)(dev(W), dev(x), y, N, K, M)
        yr, S = oracle.qmv(fmt, W, N, K, x, M=M)
    assert_within(host(y), yr, oracle.float_tol(S), f"{fmt} {N}x{K} M={M}")


@pytest.mark.parametrize("fmt,seed", [(f, s) for f in ("q4_0", "q4_k", "q6_k") for s in range(4)])
def test_geglu_down_random(fmt, seed):
    rng = np.random.default_rng(2000 + seed)
    N, K, M = draw(rng, fmt)
    say(f"random qmv_{fmt}_geglu_down N={N} K={K} M={M} seed={seed}")
    W, g = synth.problem(fmt, N, K, M, 70 + seed)
    u = synth.activations(M, K, 80 + seed)
    y = empty((M, N))
    getattr(_qmv(), f"qmv_{fmt}_geglu_down")(dev(W), dev(g), dev(u), y, N, K, M)
    yr, S, E = oracle.qmv_geglu_down(fmt, W, N, K, g, u, M=M)
    assert_within(host(y), yr, oracle.geglu_down_tol(S, E), f"{fmt} down {N}x{K} M={M}")


@pytest.mark.parametrize("seed", range(4))
def test_pair_and_qkv_random(seed):
    rng = np.random.default_rng(3000 + seed)
    N, K, M = draw(rng, "q4_0")
    say(f"random qmv_q4_0_geglu N={N} K={K} M={M} seed={seed}")
    qmv = _qmv()
    Wg, x = synth.problem("q4_0", N, K, M, 90 + seed)
    Wu = synth.q4_0_weights(N, K, 95 + seed)
    h = empty((M, N))
    qmv.qmv_q4_0_geglu(dev(Wg), dev(Wu), dev(x), h, N, K, M)
    g, Sg = oracle.qmv("q4_0", Wg, N, K, x, M=M)
    u, Su = oracle.qmv("q4_0", Wu, N, K, x, M=M)
    hr = oracle.geglu(g, u).reshape(g.shape)
    assert_within(host(h), hr, oracle.geglu_tol(g, u, Sg, Su, hr), "pair")

    K2 = 256 * int(rng.integers(1, 90))
    Nq, Nk, Nv = (int(v) for v in rng.integers(1, 300, size=3))
    say(f"random qmv_q4_k_q6_k_qkv Nq={Nq} Nk={Nk} Nv={Nv} K={K2} M={M}")
    Wq, xq = synth.problem("q4_k", Nq, K2, M, 100 + seed)
    Wk = synth.q4_k_weights(Nk, K2, 110 + seed)
    Wv = synth.q6_k_weights(Nv, K2, 120 + seed)
    q, k, v = empty((M, Nq)), empty((M, Nk)), empty((M, Nv))
    qmv.qmv_q4_k_q6_k_qkv(dev(Wq), dev(Wk), dev(Wv), dev(xq), q, k, v, Nq, Nk, Nv, K2, M)
    for name, fmt, W, Nn, out in (("q", "q4_k", Wq, Nq, q), ("k", "q4_k", Wk, Nk, k), ("v", "q6_k", Wv, Nv, v)):
        yr, S = oracle.qmv(fmt, W, Nn, K2, xq, M=M)
        assert_within(host(out), yr, oracle.float_tol(S), f"qkv {name}")
