"""Parity of the MXFP4 matrix-vector product (codes and E8M0 scales in two
planes, gfx950's packed FP4 conversion) with the float64 oracle, element by
element, through the C ABI (qmv_mxfp4).  Bar: |y - y_ref| <= 1e-5 * sum|w x|
+ 1e-6; unit vectors give the dequantized column bit for bit (every weight
is exact in float32)."""
import numpy as np
import pytest

import oracle
from quantized_dequant_matrix_amd import synth
from gpu_util import assert_within, dev, empty, host, say

pytestmark = pytest.mark.gpu


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


def run(codes, scales, x, N, K, M=1):
    y = empty((M, N))
    _qmv().qmv_mxfp4(dev(codes), dev(scales), dev(x), y, N, K, M)
    return host(y)


# unit kernel (K % 256 == 0, K <= 16128), split kernel (longer K), generic
# kernel (K % 256 != 0, and K > 40192)
SHAPES = [(1, 32), (5, 64), (7, 96), (64, 256), (65, 256), (3, 768), (33, 4096), (129, 5376), (17, 16128),
          (9, 16384), (8, 16640), (13, 5408), (29, 21504), (12, 21504), (5, 40960), (9001, 40192)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_shapes(N, K):
    seed = 5 * N + K
    say(f"qmv_mxfp4 N={N} K={K} seed={seed}")
    codes, scales, x = synth.mxfp4_problem(N, K, 1, seed)
    y = run(codes, scales, x, N, K)
    yr, S = oracle.qmv_mxfp4(codes, scales, N, K, x)
    assert_within(y, yr, oracle.float_tol(S), f"mxfp4 {N}x{K}")


@pytest.mark.parametrize("name", ["mxfp4_gate", "mxfp4_down"])
def test_workloads_full(name):
    c = synth.CONFIGS[name]
    N, K = c["N"], c["K"]
    say(f"qmv_mxfp4 workload {N}x{K}")
    codes, scales, x = synth.mxfp4_problem(N, K, 1, synth.SEEDS[name])
    y = run(codes, scales, x, N, K)
    yr, S = oracle.qmv_mxfp4(codes, scales, N, K, x)
    w = assert_within(y, yr, oracle.float_tol(S), name)
    say(f"{name}: worst err/tol {w:.3g}")


@pytest.mark.parametrize("K", [512, 96, 21504])
def test_unit_vectors_give_columns(K):
    N = 40
    say(f"qmv_mxfp4 unit vectors K={K}")
    codes, scales, _ = synth.mxfp4_problem(N, K, 1, 6)
    cols = [0, 1, 2, 15, 16, 31, 32, 33, K - 2, K - 1]
    E = np.zeros((len(cols), K), np.float32)
    for j, i in enumerate(cols):
        E[j, i] = 1.0
    y = run(codes, scales, E, N, K, len(cols))
    cb, sb = codes.reshape(N, -1), scales.reshape(N, -1)
    dq = np.stack([oracle.dequant_mxfp4_row(cb[n], sb[n], K) for n in range(N)])
    assert np.array_equal(y, dq[:, cols].T)


@pytest.mark.parametrize("e", [0, 1, 60, 127, 200, 240])
def test_scale_exponent_range(e):
    # every block at exponent e, x scaled by 2^(120 - e) so that the products
    # stay normal float32 numbers of order one
    N, K = 24, 2304
    say(f"qmv_mxfp4 all scales e={e}")
    codes, _, x = synth.mxfp4_problem(N, K, 1, 100 + e)
    scales = np.full(N * K // 32, e, np.uint8)
    x = (x.astype(np.float64) * 2.0 ** (120 - e)).astype(np.float32)
    y = run(codes, scales, x, N, K)
    yr, S = oracle.qmv_mxfp4(codes, scales, N, K, x)
    assert np.all(np.isfinite(y))
    assert_within(y, yr, oracle.float_tol(S), f"e={e}")


def test_nan_scale_makes_its_row_nan():
    N, K = 10, 4096
    say("qmv_mxfp4 E8M0 NaN scale")
    codes, scales, x = synth.mxfp4_problem(N, K, 1, 8)
    scales = scales.copy().reshape(N, -1)
    scales[3, 17] = 255
    scales[7, 0] = 255
    y = run(codes, scales.reshape(-1), x, N, K)
    yr, S = oracle.qmv_mxfp4(codes, scales.reshape(-1), N, K, x)
    nan = np.isnan(yr)
    assert nan[0].tolist() == [n in (3, 7) for n in range(N)]
    assert np.array_equal(np.isnan(y), nan)
    assert_within(y[~nan], yr[~nan], oracle.float_tol(S)[~nan], "finite rows")


def test_batched_rows():
    N, K, M = 70, 5376, 3
    say("qmv_mxfp4 M=3")
    codes, scales, x = synth.mxfp4_problem(N, K, M, 9)
    y = run(codes, scales, x, N, K, M)
    yr, S = oracle.qmv_mxfp4(codes, scales, N, K, x, M=M)
    assert_within(y, yr, oracle.float_tol(S), "M=3")


@pytest.mark.parametrize("K", [768, 21504])
def test_non_finite_activations(K):
    # as the float64 oracle: inf gives +-inf, or NaN where the weight is 0
    # (or the block scale is NaN); a NaN activation makes every row NaN
    N = 64
    say(f"qmv_mxfp4 non-finite activations K={K}")
    codes, scales, x = synth.mxfp4_problem(N, K, 1, 57)
    for pos, val in ((9, np.inf), (400, -np.inf), (33, np.nan)):
        xs = x.copy()
        xs[0, pos] = val
        y = run(codes, scales, xs, N, K)[0]
        with np.errstate(invalid="ignore", over="ignore"):
            yr, S = oracle.qmv_mxfp4(codes, scales, N, K, xs)
        yr = yr[0]
        assert np.array_equal(np.isnan(y), np.isnan(yr)), pos
        assert np.array_equal(np.isposinf(y), np.isposinf(yr)), pos
        assert np.array_equal(np.isneginf(y), np.isneginf(yr)), pos
