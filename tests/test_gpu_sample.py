"""Parity of the token selection after the logit projection (top-k, then a
top-p draw at temperature T from the caller's uniform numbers).

The draw is a decision taken in float32 on both sides of a threshold, so it
is compared where the decision is unique: when the oracle's float64 prefix
sums lie more than 1e-5 of the total away from both thresholds (top_p times
the total, and u times the nucleus sum), the token and the nucleus size must
be identical; otherwise the GPU's choice must be one of the two the float32
rounding can reach."""
import numpy as np
import pytest
import torch

import oracle
from quantized_dequant_matrix_amd import synth
from gpu_util import dev, empty, host, say
from test_gpu_topk import check_selection

pytestmark = pytest.mark.gpu

MARGIN = 1e-5


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


def margins(cum, n, T_p, u):
    total = cum[-1]
    if total <= 0:
        return np.inf
    # the last prefix sum is the total itself, which reaches top_p * total on
    # both sides for every top_p <= 1: only the earlier sums can flip n
    a = np.min(np.abs(cum[:-1] - T_p * total)) / total if cum.size > 1 else np.inf
    b = np.min(np.abs(cum[:n] - u * cum[n - 1])) / total
    return min(a, b)


def check_draw(vals, idx, u, tok, nuc, T, p, what):
    decided = 0
    for m in range(vals.shape[0]):
        rt, rn, cum = oracle.sample_topp(vals[m].astype(np.float64), idx[m], T, p, float(u[m]))
        if margins(cum, rn, p, float(u[m])) > MARGIN:
            assert (int(tok[m]), int(nuc[m])) == (rt, rn), f"{what} row {m}"
            decided += 1
        else:
            assert abs(int(nuc[m]) - rn) <= 1, f"{what} row {m}: nucleus {nuc[m]} vs {rn}"
            pos = list(idx[m]).index(int(tok[m]))
            assert pos < max(int(nuc[m]), rn), f"{what} row {m}: token outside the nucleus"
    return decided


@pytest.mark.parametrize("k", [1, 7, 40, 64])
@pytest.mark.parametrize("T,p", [(1.0, 1.0), (0.7, 0.9), (1.5, 0.5), (1.0, 0.05)])
def test_sampler_on_given_pairs(k, T, p):
    qmv = _qmv()
    M = 256
    rng = np.random.default_rng(k * 100 + int(T * 10) + int(p * 1000))
    vals = -np.sort(-rng.normal(0.0, 2.0, size=(M, k)), axis=1).astype(np.float32)
    vals[:3] = vals[:3, :1]                      # equal values: flat weights
    idx = rng.permutation(262144)[: M * k].reshape(M, k).astype(np.int32)
    u = rng.random(M).astype(np.float32)
    say(f"qmvdbg_sample_f32 k={k} T={T} top_p={p}")
    tok = empty((M,), dtype=torch.int32)
    nuc = empty((M,), dtype=torch.int32)
    qmv.qmvdbg_sample_f32(dev(vals), dev(idx), dev(u), tok, nuc, M, k, T, p)
    decided = check_draw(vals, idx, u, host(tok), host(nuc), T, p, f"k={k} T={T} p={p}")
    assert decided >= M // 2  # the rest sit within float32 rounding of a threshold


def test_sampler_nan_rows():
    qmv = _qmv()
    M, k = 4, 5
    vals = np.array([[3.0, 2.0, np.nan, np.nan, np.nan], [np.nan] * 5, [1.0, 1.0, 1.0, 1.0, 1.0],
                     [5.0, -20.0, -40.0, -60.0, -80.0]], dtype=np.float32)
    idx = np.arange(M * k, dtype=np.int32).reshape(M, k)
    u = np.array([0.99, 0.5, 0.61, 0.999], dtype=np.float32)
    tok = empty((M,), dtype=torch.int32)
    nuc = empty((M,), dtype=torch.int32)
    say("qmvdbg_sample_f32 NaN rows")
    qmv.qmvdbg_sample_f32(dev(vals), dev(idx), dev(u), tok, nuc, M, k, 1.0, 1.0)
    check_draw(vals, idx, u, host(tok), host(nuc), 1.0, 1.0, "nan rows")
    assert host(tok)[1] == 5 and host(nuc)[1] == 1


@pytest.mark.parametrize("K", [1024, 5376])
def test_logits_sample(K):
    """The tied-output shapes: the 1024-wide drafter projection and the
    5376-wide target projection, over the 262,144-entry vocabulary."""
    qmv = _qmv()
    N, M, k, cap, T, p = 262144, 2, 40, 30.0, 1.0, 0.95
    W = synth.q8_0_weights(N, K, 300 + K)
    x = synth.activations(M, K, 301 + K)
    u = np.array([0.3, 0.77], dtype=np.float32)
    say(f"logits_sample N={N} K={K} M={M} k={k}")
    wsb = qmv.logits_topk_ws_bytes(N, M, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    vals, idx = empty((M, k)), empty((M, k), dtype=torch.int32)
    tok, nuc = empty((M,), dtype=torch.int32), empty((M,), dtype=torch.int32)
    qmv.logits_sample(dev(W), dev(x), dev(u), tok, nuc, vals, idx, N, K, M, k, cap, T, p, ws, wsb)
    y = host(ws[: M * N * 4].view(torch.float32).reshape(M, N))
    vals, idx = host(vals), host(idx)
    yr, S = oracle.qmv("q8_0", W, N, K, x, M=M)
    for m in range(M):
        check_selection(idx[m], vals[m], y[m], yr[m], S[m], k, cap, f"K={K} row {m}")
    check_draw(vals, idx, u, host(tok), host(nuc), T, p, f"logits_sample K={K}")


@pytest.mark.parametrize("N,K,k", [(262144, 64, 1), (262144, 64, 10), (262144, 64, 16), (262144, 64, 17),
                                   (262144, 64, 64), (100003, 96, 40), (4 * 1024 * 1024 + 1, 32, 10)])
def test_logits_sample_paths(N, K, k):
    """Every selection path of logits_sample: the rounds and tournament
    (k <= 16) and the sorted threshold selection (k > 16) make the draw in the
    selection kernel itself; past 4M logits the scan merge is followed by the
    separate draw kernel.  The draw must equal, bit for bit, what the draw
    export makes from the selected pairs, and pass the oracle's check."""
    qmv = _qmv()
    M, cap, T, p = 3, 30.0, 0.8, 0.9
    W = synth.q8_0_weights(N, K, 500 + k)
    x = synth.activations(M, K, 501 + k)
    u = np.array([0.05, 0.5, 0.95], dtype=np.float32)
    say(f"logits_sample paths N={N} K={K} M={M} k={k}")
    wsb = qmv.logits_topk_ws_bytes(N, M, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    vals, idx = empty((M, k)), empty((M, k), dtype=torch.int32)
    tok, nuc = empty((M,), dtype=torch.int32), empty((M,), dtype=torch.int32)
    ud = dev(u)
    qmv.logits_sample(dev(W), dev(x), ud, tok, nuc, vals, idx, N, K, M, k, cap, T, p, ws, wsb)
    tok2, nuc2 = empty((M,), dtype=torch.int32), empty((M,), dtype=torch.int32)
    qmv.qmvdbg_sample_f32(vals, idx, ud, tok2, nuc2, M, k, T, p)
    assert np.array_equal(host(tok), host(tok2)) and np.array_equal(host(nuc), host(nuc2))
    y = host(ws[: M * N * 4].view(torch.float32).reshape(M, N))
    vals, idx = host(vals), host(idx)
    yr, S = oracle.qmv("q8_0", W, N, K, x, M=M)
    for m in range(M):
        check_selection(idx[m], vals[m], y[m], yr[m], S[m], k, cap, f"N={N} k={k} row {m}")
    check_draw(vals, idx, u, host(tok), host(nuc), T, p, f"logits_sample N={N} k={k}")
