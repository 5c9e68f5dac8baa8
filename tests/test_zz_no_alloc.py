"""logits_topk_noalloc: the top-k logit path with its workspace in the
library's fixed device array, against logits_topk with a caller's workspace
(same kernels: identical indices and values) and the oracle, on two calls in
a row, the second smaller than the first."""
import numpy as np
import pytest
import torch

import oracle
from quantized_dequant_matrix_amd import synth
from gpu_util import dev, empty, host, say

pytestmark = pytest.mark.gpu

STATIC_BYTES = 8 << 20


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


def _with_workspace(W, x, N, K, M, k, cap):
    qmv = _qmv()
    wsb = qmv.logits_topk_ws_bytes(N, M, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    v, i = empty((M, k)), empty((M, k), dtype=torch.int32)
    qmv.logits_topk(W, x, v, i, N, K, M, k, cap, ws, wsb)
    return host(v), host(i)


def _noalloc(W, x, N, K, M, k, cap):
    qmv = _qmv()
    v, i = empty((M, k)), empty((M, k), dtype=torch.int32)
    qmv.logits_topk_noalloc(W, x, v, i, N, K, M, k, cap)
    return host(v), host(i)


def _check_against_oracle(Wh, xh, N, K, M, k, cap, v, i):
    y, S = oracle.qmv("q8_0", Wh, N, K, xh, M=M)
    T = oracle.float_tol(S)
    for m in range(M):
        ref = oracle.topk(y[m], k + 1)
        band = 2 * T[m].max()
        kth, nxt = y[m][ref[k - 1]], y[m][ref[k]]
        if kth - nxt >= band:  # one correct index set
            assert sorted(i[m].tolist()) == sorted(ref[:k].tolist())
        else:  # several: every chosen logit within the band of the k-th
            assert np.all(y[m][i[m]] >= kth - band)
        zr = oracle.softcap(y[m][i[m]], cap)
        assert np.all(np.abs(v[m].astype(np.float64) - zr) <= T[m][i[m]] + 1e-5)


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_matches_workspace_path(order):
    qmv = _qmv()
    cases = [(262144, 256, 2, 10, 30.0, 301), (50000, 512, 3, 40, 20.0, 302)]
    if order == "small_then_large":
        cases = cases[::-1]
    for N, K, M, k, cap, seed in cases:
        assert qmv.logits_topk_ws_bytes(N, M, k) <= STATIC_BYTES
        say(f"logits_topk_noalloc N={N} K={K} M={M} k={k}")
        Wh, xh = synth.problem("q8_0", N, K, M, seed)
        W, x = dev(Wh), dev(xh)
        v0, i0 = _with_workspace(W, x, N, K, M, k, cap)
        v1, i1 = _noalloc(W, x, N, K, M, k, cap)
        assert np.array_equal(i0, i1)
        assert np.array_equal(v0.view(np.uint32), v1.view(np.uint32))
        _check_against_oracle(Wh, xh, N, K, M, k, cap, v1, i1)


def test_noalloc_rejects_requests_beyond_the_static_workspace():
    qmv = _qmv()
    N, K, M, k = 262144, 64, 8, 10
    assert qmv.logits_topk_ws_bytes(N, M, k) > STATIC_BYTES
    say("logits_topk_noalloc beyond the static workspace")
    W = empty((N * 2 * 34,), dtype=torch.uint8)
    x = empty((M, K))
    v, i = empty((M, k)), empty((M, k), dtype=torch.int32)
    with pytest.raises(qmv.QmvError) as e:
        qmv.logits_topk_noalloc(W, x, v, i, N, K, M, k, 30.0)
    assert e.value.status == qmv.QMV_ERR_WORKSPACE
