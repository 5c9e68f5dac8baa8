"""Parity of the Q4_0 x Q8-activation path: the quantized activations and the
integer block sums bit for bit, the float outputs within the tolerance."""
import numpy as np
import pytest
import torch

import oracle
from quantized_dequant_matrix_amd import synth
from gpu_util import assert_within, dev, empty, host, say

pytestmark = pytest.mark.gpu

C4 = synth.CONFIGS["c4"]


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


def gpu_quantize(x, M, K):
    qmv = _qmv()
    q = empty((M, K), dtype=torch.int8)
    d = empty((M, K // 32))
    qmv.qmvdbg_quantize_q8(dev(x), q, d, K, M)
    return host(q), host(d)


def gpu_blocksums(W, qx, N, K, M):
    qmv = _qmv()
    isum = empty((M, N, K // 32), dtype=torch.int32)
    qmv.qmvdbg_q4_0_q8_blocksums(dev(W), dev(qx), isum, N, K, M)
    return host(isum)


def gpu_qmm(W, x, N, K, M):
    qmv = _qmv()
    wsb = qmv.qmm_q4_0_q8act_ws_bytes(N, K, M)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    y = empty((M, N))
    qmv.qmm_q4_0_q8act(dev(W), dev(x), y, N, K, M, ws, wsb)
    return host(y)


@pytest.mark.parametrize("M", [1, 16, 512])
def test_quantizer_bit_exact(M):
    K = C4["K"]
    say(f"qmvdbg_quantize_q8 M={M} K={K}")
    x = synth.activations(M, K, synth.SEEDS["c4"])
    q, d = gpu_quantize(x, M, K)
    qr, dr = oracle.quantize_q8(x, M, K)
    assert np.array_equal(d.view(np.uint32), dr.view(np.uint32))
    assert np.array_equal(q, qr)


def test_quantizer_ties_and_zero_blocks():
    say("qmvdbg_quantize_q8 ties / zero blocks / wide range")
    K = 256
    x = np.zeros((3, K), np.float32)
    x[0, :32] = 127.0
    x[0, 1:9] = [2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5, -126.5]
    x[1] = np.random.default_rng(0).standard_normal(K) * 10.0 ** np.random.default_rng(1).uniform(-30, 30, K)
    x[2, 40] = -1e-38
    q, d = gpu_quantize(x, 3, K)
    qr, dr = oracle.quantize_q8(x, 3, K)
    assert np.array_equal(d.view(np.uint32), dr.view(np.uint32))
    assert np.array_equal(q, qr)


@pytest.mark.parametrize("M", [1, 16, 512])
def test_blocksums_bit_exact(M):
    K = C4["K"]
    n0, n = 1000, 96 if M < 512 else 24
    say(f"qmvdbg_q4_0_q8_blocksums M={M} rows {n0}..{n0 + n}")
    W, x = synth.config_problem("c4", M=M)
    rb = oracle.row_bytes("q4_0", K)
    Wsub = W[n0 * rb:(n0 + n) * rb]
    qx, _ = oracle.quantize_q8(x, M, K)
    got = gpu_blocksums(Wsub, qx, n, K, M)
    ref = oracle.q4_0_q8_blocksums(Wsub, n, K, qx, M)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("N,K,M", [(5, 64, 1), (70, 256, 3), (33, 5408, 2), (129, 4096, 16), (64, 2048, 40)])
def test_blocksums_shapes(N, K, M):
    say(f"qmvdbg_q4_0_q8_blocksums N={N} K={K} M={M}")
    W, x = synth.problem("q4_0", N, K, M, N * M + K)
    qx, _ = oracle.quantize_q8(x, M, K)
    assert np.array_equal(gpu_blocksums(W, qx, N, K, M), oracle.q4_0_q8_blocksums(W, N, K, qx, M))


def _qmm_ref(W, x, N, K, M, rows=None):
    qx, dx = oracle.quantize_q8(x, M, K)
    return oracle.qmm_q4_0_q8(W, N, K, qx, dx, M, rows=rows)


@pytest.mark.parametrize("M", [1, 16])
def test_qmm_workload_full(M):
    N, K = C4["N"], C4["K"]
    say(f"qmm_q4_0_q8act workload M={M}")
    W, x = synth.config_problem("c4", M=M)
    y = gpu_qmm(W, x, N, K, M)
    yr, S = _qmm_ref(W, x, N, K, M)
    w = assert_within(y, yr, oracle.float_tol(S), f"c4 M={M}")
    say(f"c4 M={M}: worst err/tol {w:.3g}")


def test_qmm_workload_m512_sampled():
    N, K, M = C4["N"], C4["K"], 512
    say("qmm_q4_0_q8act workload M=512, 48 sampled rows")
    W, x = synth.config_problem("c4", M=M)
    y = gpu_qmm(W, x, N, K, M)
    rows = np.sort(np.random.default_rng(4).choice(N, 48, replace=False))
    yr, S = _qmm_ref(W, x, N, K, M, rows=rows)
    w = assert_within(y[:, rows], yr, oracle.float_tol(S), "c4 M=512")
    assert np.all(np.isfinite(y))
    say(f"c4 M=512: worst err/tol {w:.3g}")


def test_qmm_wide_ragged_sampled():
    """The wide tiling with N and M off the 64-row tiles and a half-full last
    weight chunk (K / 32 = 24 blocks: one chunk of 16, one of 8)."""
    N, K, M = 8200, 768, 520
    say(f"qmm_q4_0_q8act wide tiling N={N} K={K} M={M}, sampled rows")
    W, x = synth.problem("q4_0", N, K, M, 77)
    y = gpu_qmm(W, x, N, K, M)
    rows = np.unique(np.concatenate([[0, 63, 64, 8191, 8192, N - 1],
                                     np.random.default_rng(5).choice(N, 40, replace=False)]))
    yr, S = _qmm_ref(W, x, N, K, M, rows=rows)
    assert_within(y[:, rows], yr, oracle.float_tol(S), "wide ragged")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("N,K,M", [(1, 32, 1), (9, 96, 2), (65, 256, 5), (200, 5376, 17), (31, 16640, 3)])
def test_qmm_shapes(N, K, M):
    say(f"qmm_q4_0_q8act N={N} K={K} M={M}")
    W, x = synth.problem("q4_0", N, K, M, 3 * N + K + M)
    y = gpu_qmm(W, x, N, K, M)
    yr, S = _qmm_ref(W, x, N, K, M)
    assert_within(y, yr, oracle.float_tol(S), "qmm")


def test_qmm_integer_valued_is_exact():
    say("qmm_q4_0_q8act integer-valued case")
    rng = np.random.default_rng(8)
    N, K, M = 300, 21504, 16
    q = rng.integers(0, 16, size=(N * K // 32, 32), dtype=np.uint8)
    W = synth.pack_q4_0(np.ones(N * K // 32, np.float16), q)
    x = rng.integers(-64, 65, size=(M, K)).astype(np.float32)
    x.reshape(M, K // 32, 32)[:, :, 5] = 127.0
    y = gpu_qmm(W, x, N, K, M)
    yr, _ = _qmm_ref(W, x, N, K, M)
    assert np.array_equal(y, yr)
