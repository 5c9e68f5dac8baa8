"""Pins of the oracle's down projection with the GELU gate on its input:
gates of +-64 make gelu exactly 64 or -0 in float64, which turns the product
into 64 W u (exact power-of-two scaling of the plain product) or zero,
independently of the GELU formula; u = 0 gives zero."""
import numpy as np
import pytest

import oracle
from quantized_dequant_matrix_amd import synth


@pytest.mark.parametrize("fmt,K", [("q4_0", 96), ("q8_0", 64), ("q4_k", 512), ("q6_k", 512)])
def test_saturated_gates(fmt, K):
    N, M = 6, 2
    W, u = synth.problem(fmt, N, K, M, seed=31)
    rng = np.random.default_rng(31)
    sign = rng.integers(0, 2, size=(M, K)) * 2 - 1
    g = (64.0 * sign).astype(np.float32)
    assert oracle.gelu_tanh(64.0) == 64.0 and oracle.gelu_tanh(-64.0) == 0.0
    y, S, E = oracle.qmv_geglu_down(fmt, W, N, K, g, u, M=M)
    um = np.where(sign > 0, u, np.float32(0)).astype(np.float32)
    yp, Sp = oracle.qmv(fmt, W, N, K, um, M=M)
    assert np.array_equal(y, 64.0 * yp)
    assert np.array_equal(S, 64.0 * Sp)
    # E = sum |w| |u| (64 + gelu): 128 |w u| where the gate is +64, 64 |w u| where it is -64
    rb = oracle.row_bytes(fmt, K)
    wabs = np.stack([np.abs(oracle.dequant_row(fmt, W[n * rb:(n + 1) * rb], K)) for n in range(N)])
    Eref = (np.abs(u).astype(np.float64) * np.where(sign > 0, 128.0, 64.0)) @ wabs.T
    assert np.allclose(E, Eref, rtol=1e-12, atol=0)


def test_zero_up_or_zero_gate_gives_zero():
    N, K = 4, 256
    W, g = synth.problem("q6_k", N, K, 1, seed=8)
    y, S, E = oracle.qmv_geglu_down("q6_k", W, N, K, g, np.zeros_like(g))
    assert np.all(y == 0) and np.all(S == 0) and np.all(E == 0)
    y, S, E = oracle.qmv_geglu_down("q6_k", W, N, K, np.zeros_like(g), g)
    assert np.all(y == 0) and np.all(S == 0)


def test_rows_subset_and_rejects_bad_shapes():
    N, K, M = 5, 64, 2
    W, g = synth.problem("q8_0", N, K, M, seed=4)
    u = np.flip(g, axis=1).copy()
    y, S, E = oracle.qmv_geglu_down("q8_0", W, N, K, g, u, M=M)
    ys, Ss, Es = oracle.qmv_geglu_down("q8_0", W, N, K, g, u, M=M, rows=[4, 0])
    assert np.array_equal(ys, y[:, [4, 0]]) and np.array_equal(Es, E[:, [4, 0]])
    with pytest.raises(ValueError):
        oracle.qmv_geglu_down("q8_0", W, N, K, g[:, :32], u, M=M)
