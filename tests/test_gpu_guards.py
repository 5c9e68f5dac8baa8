"""Every entry point writes only its outputs (and, where it takes one, its
workspace up to the size it asked for), and leaves its inputs untouched:
outputs and workspaces get a sentinel tail that must survive the call, and
the weights and activations must be bit-identical afterwards.  Shapes are
ragged so that the last row, tile and pass of every kernel are partial."""
import numpy as np
import pytest
import torch

from quantized_dequant_matrix_amd import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

GUARD = 4096
SENT = 0x7FBADBAD  # a NaN pattern no kernel produces


def _qmv():
    from quantized_dequant_matrix_amd import qmv
    return qmv


def guarded(n, dtype=torch.float32):
    """(full buffer, view of the first n elements) with a sentinel tail."""
    full = torch.empty(n + GUARD, dtype=torch.int32, device="cuda:0")
    full.fill_(SENT)
    return full, full[:n].view(dtype)


def tail_ok(full, n):
    t = full[n:].cpu().numpy()
    return bool(np.all(t == SENT))


def same(before, t):
    return torch.equal(before, t)


@pytest.mark.parametrize("fmt,N,K", [("q4_0", 77, 5376), ("q8_0", 65, 2080), ("q4_k", 131, 21504),
                                     ("q6_k", 29, 5376), ("q6_k", 13, 21504), ("q4_0", 9, 96)])
def test_gemv_writes_only_y(fmt, N, K):
    M = 2
    say(f"guards qmv_{fmt} N={N} K={K}")
    W, x = synth.problem(fmt, N, K, M, 5)
    Wd, xd = dev(W), dev(x)
    W0, x0 = Wd.clone(), xd.clone()
    full, y = guarded(M * N)
    getattr(_qmv(), "qmv_" + fmt)(Wd, xd, y, N, K, M)
    torch.cuda.synchronize()
    assert tail_ok(full, M * N)
    assert same(W0, Wd) and same(x0, xd)
    assert not torch.isnan(y).any()


@pytest.mark.parametrize("N,K", [(41, 5376), (11, 21504), (7, 96)])
def test_mxfp4_and_gated_paths_write_only_outputs(N, K):
    qmv = _qmv()
    say(f"guards mxfp4 / geglu / down N={N} K={K}")
    codes, scales, x = synth.mxfp4_problem(N, K, 1, 3)
    cd, sd, xd = dev(codes), dev(scales), dev(x)
    c0, s0, x0 = cd.clone(), sd.clone(), xd.clone()
    full, y = guarded(N)
    qmv.qmv_mxfp4(cd, sd, xd, y, N, K, 1)
    torch.cuda.synchronize()
    assert tail_ok(full, N) and same(c0, cd) and same(s0, sd) and same(x0, xd)

    Wg, _ = synth.problem("q4_0", N, K, 1, 4)
    Wu = synth.q4_0_weights(N, K, 6)
    gd, ud = dev(Wg), dev(Wu)
    full, h = guarded(N)
    qmv.qmv_q4_0_geglu(gd, ud, xd, h, N, K, 1)
    torch.cuda.synchronize()
    assert tail_ok(full, N)

    u = dev(synth.activations(1, K, 8))
    u0 = u.clone()
    full, y = guarded(N)
    qmv.qmv_q4_0_geglu_down(gd, xd, u, y, N, K, 1)
    torch.cuda.synchronize()
    assert tail_ok(full, N) and same(u0, u) and same(x0, xd)


def test_qkv_writes_only_its_three_outputs():
    qmv = _qmv()
    Nq, Nk, Nv, K = 70, 13, 31, 5376
    say("guards qmv_q4_k_q6_k_qkv")
    Wq, x = synth.problem("q4_k", Nq, K, 1, 9)
    Wk = synth.q4_k_weights(Nk, K, 10)
    Wv = synth.q6_k_weights(Nv, K, 11)
    fq, q = guarded(Nq)
    fk, k = guarded(Nk)
    fv, v = guarded(Nv)
    qmv.qmv_q4_k_q6_k_qkv(dev(Wq), dev(Wk), dev(Wv), dev(x), q, k, v, Nq, Nk, Nv, K, 1)
    torch.cuda.synchronize()
    assert tail_ok(fq, Nq) and tail_ok(fk, Nk) and tail_ok(fv, Nv)


@pytest.mark.parametrize("M", [1, 16, 70])
def test_qmm_writes_only_y_and_its_workspace(M):
    qmv = _qmv()
    N, K = 197, 4096
    say(f"guards qmm_q4_0_q8act / f32act M={M}")
    W, x = synth.problem("q4_0", N, K, M, 12)
    Wd, xd = dev(W), dev(x)
    W0, x0 = Wd.clone(), xd.clone()
    for name in ("qmm_q4_0_q8act", "qmm_q4_0_f32act"):
        wsb = getattr(qmv, name + "_ws_bytes")(N, K, M)
        fws = torch.empty((wsb + 4 * GUARD + 3) // 4, dtype=torch.int32, device="cuda:0")
        fws.fill_(SENT)
        ws = fws.view(torch.uint8)[:wsb]
        full, y = guarded(M * N)
        getattr(qmv, name)(Wd, xd, y, N, K, M, ws, wsb)
        torch.cuda.synchronize()
        assert tail_ok(full, M * N), name
        tail = fws.view(torch.uint8)[wsb:wsb + 4 * GUARD].cpu().numpy()
        assert np.all(tail == np.frombuffer(np.array([SENT] * GUARD, np.int32).tobytes(), np.uint8)), name
        assert same(W0, Wd) and same(x0, xd)


@pytest.mark.parametrize("k", [10, 40])
def test_logits_paths_write_only_outputs_and_workspace(k):
    qmv = _qmv()
    N, K, M = 30001, 1024, 2
    say(f"guards logits_topk / logits_sample k={k}")
    W, x = synth.problem("q8_0", N, K, M, 13)
    Wd, xd = dev(W), dev(x)
    wsb = qmv.logits_topk_ws_bytes(N, M, k)
    fws = torch.empty((wsb + 4 * GUARD + 3) // 4, dtype=torch.int32, device="cuda:0")
    fws.fill_(SENT)
    ws = fws.view(torch.uint8)[:wsb]
    fv, vals = guarded(M * k)
    fi, idx = guarded(M * k, torch.int32)
    qmv.logits_topk(Wd, xd, vals, idx, N, K, M, k, 30.0, ws, wsb)
    torch.cuda.synchronize()
    assert tail_ok(fv, M * k) and tail_ok(fi, M * k)
    tail = fws.view(torch.uint8)[wsb:wsb + 4 * GUARD].cpu().numpy()
    assert np.all(tail == np.frombuffer(np.array([SENT] * GUARD, np.int32).tobytes(), np.uint8))
    u = dev(np.array([0.3, 0.7], np.float32))
    ft, tok = guarded(M, torch.int32)
    fn, nuc = guarded(M, torch.int32)
    qmv.logits_sample(Wd, xd, u, tok, nuc, vals, idx, N, K, M, k, 30.0, 0.8, 0.9, ws, wsb)
    torch.cuda.synchronize()
    assert tail_ok(ft, M) and tail_ok(fn, M) and tail_ok(fv, M * k) and tail_ok(fi, M * k)
