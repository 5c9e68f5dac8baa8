"""Parity of the three-matrix attention projection (Q and K rows in Q4_K, V
rows in Q6_K, one launch) with the float64 oracle, element by element,
through the C ABI (qmv_q4_k_q6_k_qkv).  Bar: the float bound of every
output, |y - y_ref| <= 1e-5 * sum|w x| + 1e-6; and each output equals the
single-matrix entry point's bit for bit (the same per-row arithmetic)."""
import numpy as np
import pytest

import oracle
from quantized_dequant_matrix_amd import synth
from gpu_util import assert_within, dev, empty, host, say

pytestmark = pytest.mark.gpu


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


def problem(Nq, Nk, Nv, K, M, seed):
    Wq, x = synth.problem("q4_k", Nq, K, M, seed)
    Wk = synth.q4_k_weights(Nk, K, seed + 1)
    Wv = synth.q6_k_weights(Nv, K, seed + 2)
    return Wq, Wk, Wv, x


def run(Wq, Wk, Wv, x, Nq, Nk, Nv, K, M):
    q, k, v = empty((M, Nq)), empty((M, Nk)), empty((M, Nv))
    _qmv().qmv_q4_k_q6_k_qkv(dev(Wq), dev(Wk), dev(Wv), dev(x), q, k, v, Nq, Nk, Nv, K, M)
    return host(q), host(k), host(v)


SHAPES = [(1, 1, 1, 256), (7, 3, 5, 512), (64, 65, 66, 768), (300, 100, 200, 5376), (130, 2, 70, 16128),
          (9, 5, 11, 21504)]


@pytest.mark.parametrize("Nq,Nk,Nv,K", SHAPES)
def test_shapes(Nq, Nk, Nv, K):
    say(f"qmv_q4_k_q6_k_qkv Nq={Nq} Nk={Nk} Nv={Nv} K={K}")
    Wq, Wk, Wv, x = problem(Nq, Nk, Nv, K, 1, Nq + Nk + Nv + K)
    q, k, v = run(Wq, Wk, Wv, x, Nq, Nk, Nv, K, 1)
    for name, fmt, W, N, y in (("q", "q4_k", Wq, Nq, q), ("k", "q4_k", Wk, Nk, k), ("v", "q6_k", Wv, Nv, v)):
        yr, S = oracle.qmv(fmt, W, N, K, x)
        assert_within(y, yr, oracle.float_tol(S), f"qkv {name} {N}x{K}")


def test_workload_shape_and_single_matrix_identity():
    c = synth.CONFIGS["qkv"]
    Nq, Nk, Nv, K = c["Nq"], c["Nk"], c["Nv"], c["K"]
    say(f"qmv_q4_k_q6_k_qkv workload {Nq}+{Nk}+{Nv} x {K}")
    Wq, Wk, Wv, x = synth.qkv_problem()
    q, k, v = run(Wq, Wk, Wv, x, Nq, Nk, Nv, K, 1)
    qmv = _qmv()
    for name, fmt, W, N, y in (("q", "q4_k", Wq, Nq, q), ("k", "q4_k", Wk, Nk, k), ("v", "q6_k", Wv, Nv, v)):
        yr, S = oracle.qmv(fmt, W, N, K, x)
        assert_within(y, yr, oracle.float_tol(S), f"qkv workload {name}")
        ys = empty((1, N))
        getattr(qmv, "qmv_" + fmt)(dev(W), dev(x), ys, N, K, 1)
        assert np.array_equal(y, host(ys)), f"{name}: fused launch differs from qmv_{fmt}"


def test_batched_rows():
    Nq, Nk, Nv, K, M = 50, 20, 30, 1024, 3
    say("qmv_q4_k_q6_k_qkv M=3")
    Wq, Wk, Wv, x = problem(Nq, Nk, Nv, K, M, 4)
    q, k, v = run(Wq, Wk, Wv, x, Nq, Nk, Nv, K, M)
    for name, fmt, W, N, y in (("q", "q4_k", Wq, Nq, q), ("k", "q4_k", Wk, Nk, k), ("v", "q6_k", Wv, Nv, v)):
        yr, S = oracle.qmv(fmt, W, N, K, x, M=M)
        assert_within(y, yr, oracle.float_tol(S), f"qkv M=3 {name}")
