"""The C-ABI library loads, exports every entry point include/qmv.h declares,
and rejects bad arguments on the host before touching the GPU.

No compute call is made here: EVERY call below must fail argument checking
(the fake addresses are never valid device memory), so a new case must be
one that the host-side checks reject."""
import os
import re

import pytest

from quantized_dequant_matrix_amd import qmv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qmv.h")

OK, NUL, SHAPE, ALIGN, WS, LAUNCH, ARG = range(7)
FAKE = 1 << 20          # a non-null, 256-byte aligned address that is never dereferenced here
S = None                # null stream


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert "qmv_q4_0" in names and "logits_topk" in names and len(names) == 24
    for n in names:
        assert hasattr(qmv.lib, n), n
    assert sorted(qmv.EXPORTS) == names


def test_launch_path_allocates_copies_and_waits_for_nothing():
    """The library is launch-only: among the HIP runtime calls it imports there
    is no allocation, no copy or fill, no synchronisation and no graph call, so
    every buffer is the caller's and every call only enqueues work."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm (binutils) is not installed")
    out = subprocess.run([nm, "-D", "--undefined-only", qmv._LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    hip = sorted({ln.split()[-1].split("@")[0] for ln in out.splitlines() if "hip" in ln})
    assert "hipLaunchKernel" in hip
    banned = re.compile(r"^hip(Malloc|Free|HostMalloc|HostRegister|Memcpy|Memset|.*Synchronize|Graph|StreamCreate|EventCreate)")
    assert [h for h in hip if banned.match(h)] == [], hip


def test_status_strings():
    for s in range(7):
        assert qmv.status_str(s)
    assert qmv.status_str(99) == "unknown status"


def call(name, *args):
    return getattr(qmv.lib, name)(*args)


@pytest.mark.parametrize("name", ["qmv_q4_0", "qmv_q8_0", "qmv_q4_k", "qmv_q6_k"])
def test_gemv_validation(name):
    assert call(name, None, FAKE, FAKE, 8, 256, 1, S) == NUL
    assert call(name, FAKE, None, FAKE, 8, 256, 1, S) == NUL
    assert call(name, FAKE, FAKE, None, 8, 256, 1, S) == NUL
    assert call(name, FAKE, FAKE, FAKE, 0, 256, 1, S) == SHAPE
    assert call(name, FAKE, FAKE, FAKE, 8, 256, 0, S) == SHAPE
    assert call(name, FAKE, FAKE, FAKE, 8, 0, 1, S) == SHAPE
    assert call(name, FAKE, FAKE, FAKE, 8, 16, 1, S) == SHAPE
    assert call(name, FAKE, FAKE, FAKE, 8, 33 * 32 + 1, 1, S) == SHAPE
    assert call(name, FAKE, FAKE, FAKE, 1 << 31, 256, 1, S) == SHAPE
    assert call(name, FAKE, FAKE, FAKE, 8, 1 << 21, 1 << 41, S) == SHAPE  # M*K*4 overflows int64
    assert call(name, FAKE, FAKE, FAKE, 1, 256, 65536, S) == SHAPE      # activation rows are bounded
    assert call(name, FAKE + 8, FAKE, FAKE, 8, 256, 1, S) == ALIGN
    assert call(name, FAKE, FAKE + 2, FAKE, 8, 256, 1, S) == ALIGN
    assert call(name, FAKE, FAKE, FAKE + 1, 8, 256, 1, S) == ALIGN


@pytest.mark.parametrize("name", ["qmv_q4_k", "qmv_q6_k"])
def test_k_quants_need_whole_superblocks(name):
    assert call(name, FAKE, FAKE, FAKE, 8, 288, 1, S) == SHAPE
    assert call(name, FAKE, FAKE, FAKE, 8, 256 * 84 + 32, 1, S) == SHAPE


def test_geglu_validation():
    assert call("qmv_q4_0_geglu", FAKE, None, FAKE, FAKE, 8, 256, 1, S) == NUL
    assert call("qmv_q4_0_geglu", None, FAKE, FAKE, FAKE, 8, 256, 1, S) == NUL
    assert call("qmv_q4_0_geglu", FAKE, FAKE + 4, FAKE, FAKE, 8, 256, 1, S) == ALIGN
    assert call("qmv_q4_0_geglu", FAKE, FAKE, FAKE, FAKE, 8, 48, 1, S) == SHAPE


@pytest.mark.parametrize("name", ["qmv_q4_0_geglu_down", "qmv_q4_k_geglu_down", "qmv_q6_k_geglu_down"])
def test_geglu_down_validation(name):
    assert call(name, None, FAKE, FAKE, FAKE, 8, 256, 1, S) == NUL
    assert call(name, FAKE, None, FAKE, FAKE, 8, 256, 1, S) == NUL
    assert call(name, FAKE, FAKE, None, FAKE, 8, 256, 1, S) == NUL
    assert call(name, FAKE, FAKE, FAKE, None, 8, 256, 1, S) == NUL
    assert call(name, FAKE + 8, FAKE, FAKE, FAKE, 8, 256, 1, S) == ALIGN
    assert call(name, FAKE, FAKE, FAKE + 2, FAKE, 8, 256, 1, S) == ALIGN
    assert call(name, FAKE, FAKE, FAKE, FAKE, 0, 256, 1, S) == SHAPE
    assert call(name, FAKE, FAKE, FAKE, FAKE, 8, 48, 1, S) == SHAPE
    if name != "qmv_q4_0_geglu_down":
        assert call(name, FAKE, FAKE, FAKE, FAKE, 8, 288, 1, S) == SHAPE


def test_mxfp4_validation():
    c = lambda *a: call("qmv_mxfp4", *a)
    assert c(None, FAKE, FAKE, FAKE, 8, 256, 1, S) == NUL
    assert c(FAKE, None, FAKE, FAKE, 8, 256, 1, S) == NUL
    assert c(FAKE, FAKE, None, FAKE, 8, 256, 1, S) == NUL
    assert c(FAKE, FAKE, FAKE, None, 8, 256, 1, S) == NUL
    assert c(FAKE + 8, FAKE, FAKE, FAKE, 8, 256, 1, S) == ALIGN
    assert c(FAKE, FAKE + 8, FAKE, FAKE, 8, 256, 1, S) == ALIGN
    assert c(FAKE, FAKE, FAKE + 2, FAKE, 8, 256, 1, S) == ALIGN
    assert c(FAKE, FAKE, FAKE, FAKE, 8, 48, 1, S) == SHAPE
    assert c(FAKE, FAKE, FAKE, FAKE, 0, 64, 1, S) == SHAPE


def test_qkv_validation():
    args = [FAKE] * 7 + [8, 4, 4, 256, 1, S]

    def with_(i, v):
        a = list(args)
        a[i] = v
        return call("qmv_q4_k_q6_k_qkv", *a)

    for i in range(7):
        assert with_(i, None) == NUL
    for i in range(3):
        assert with_(i, FAKE + 8) == ALIGN
    for i in range(3, 7):
        assert with_(i, FAKE + 2) == ALIGN
    assert with_(7, 0) == SHAPE and with_(8, 0) == SHAPE and with_(9, 0) == SHAPE
    assert with_(10, 288) == SHAPE and with_(10, 32) == SHAPE
    assert with_(11, 0) == SHAPE


def test_qmm_validation_and_workspace():
    need = qmv.qmm_q4_0_q8act_ws_bytes(5376, 21504, 512)
    assert need >= 512 * 21504 + 512 * 672 * 4
    # small M splits K across workgroups: partial sums [splits][M][N] join the workspace
    assert qmv.qmm_q4_0_q8act_ws_bytes(5376, 21504, 16) > 16 * 21504 + 16 * 672 * 4 + 5376 * 16 * 4
    assert qmv.qmm_q4_0_q8act_ws_bytes(8, 33, 1) == 0
    assert qmv.qmm_q4_0_q8act_ws_bytes(8, 64, 0) == 0
    assert qmv.qmm_q4_0_q8act_ws_bytes(0, 64, 1) == 0
    assert call("qmm_q4_0_q8act", FAKE, FAKE, FAKE, 8, 64, 1, None, 1 << 20, S) == NUL
    assert call("qmm_q4_0_q8act", FAKE, FAKE, FAKE, 8, 64, 1, FAKE, 16, S) == WS
    assert call("qmm_q4_0_q8act", FAKE, FAKE, FAKE, 8, 64, 1, FAKE + 4, 1 << 20, S) == ALIGN
    assert call("qmm_q4_0_q8act", FAKE, FAKE, FAKE, 8, 40, 1, FAKE, 1 << 20, S) == SHAPE
    assert call("qmm_q4_0_q8act", None, FAKE, FAKE, 8, 64, 1, FAKE, 1 << 20, S) == NUL


def test_qmm_f32act_validation_and_workspace():
    # split activations: two float16 terms per element (4 B) plus a scale per block
    need = qmv.qmm_q4_0_f32act_ws_bytes(21504, 5376, 8)
    assert need >= 16 * 5376 * 4 + 16 * 168 * 4
    assert qmv.qmm_q4_0_f32act_ws_bytes(21504, 5376, 32) >= 32 * 5376 * 4 + 32 * 168 * 4
    # M == 1 and K % 256 != 0 use the matrix-vector kernels: a token workspace
    assert qmv.qmm_q4_0_f32act_ws_bytes(8, 96, 3) == 256
    assert qmv.qmm_q4_0_f32act_ws_bytes(8, 33, 2) == 0
    assert qmv.qmm_q4_0_f32act_ws_bytes(8, 256, 0) == 0
    assert call("qmm_q4_0_f32act", FAKE, FAKE, FAKE, 8, 256, 2, None, 1 << 20, S) == NUL
    assert call("qmm_q4_0_f32act", FAKE, FAKE, FAKE, 8, 256, 2, FAKE, 16, S) == WS
    assert call("qmm_q4_0_f32act", FAKE, FAKE, FAKE, 8, 256, 2, FAKE + 4, 1 << 20, S) == ALIGN
    assert call("qmm_q4_0_f32act", FAKE + 8, FAKE, FAKE, 8, 256, 2, FAKE, 1 << 20, S) == ALIGN
    assert call("qmm_q4_0_f32act", FAKE, FAKE, FAKE, 8, 40, 2, FAKE, 1 << 20, S) == SHAPE
    assert call("qmm_q4_0_f32act", FAKE, FAKE, None, 8, 256, 2, FAKE, 1 << 20, S) == NUL


def test_logits_topk_validation():
    need = qmv.logits_topk_ws_bytes(262144, 1, 10)
    assert need >= 262144 * 4
    args = lambda **kw: dict(dict(W=FAKE, x=FAKE, v=FAKE, i=FAKE, N=1000, K=64, M=1, k=10, cap=30.0,
                                  ws=FAKE, wsb=1 << 30), **kw)

    def run(**kw):
        a = args(**kw)
        return call("logits_topk", a["W"], a["x"], a["v"], a["i"], a["N"], a["K"], a["M"], a["k"],
                    a["cap"], a["ws"], a["wsb"], S)

    assert run(W=None) == NUL
    assert run(ws=None) == NUL
    assert run(i=None) == NUL
    assert run(k=0) == ARG
    assert run(k=65) == ARG
    assert run(N=5, k=6) == ARG
    assert run(cap=0.0) == ARG
    assert run(cap=-1.0) == ARG
    assert run(cap=float("inf")) == ARG
    assert run(cap=float("nan")) == ARG
    assert run(wsb=16) == WS
    assert run(ws=FAKE + 8) == ALIGN
    assert run(i=FAKE + 2) == ALIGN
    assert run(K=48) == SHAPE
    assert run(M=70000) == SHAPE


def test_logits_sample_validation():
    args = lambda **kw: dict(dict(W=FAKE, x=FAKE, u=FAKE, t=FAKE, n=FAKE, v=FAKE, i=FAKE, N=1000, K=64, M=1,
                                  k=40, cap=30.0, T=1.0, p=0.9, ws=FAKE, wsb=1 << 30), **kw)

    def run(**kw):
        a = args(**kw)
        return call("logits_sample", a["W"], a["x"], a["u"], a["t"], a["n"], a["v"], a["i"], a["N"], a["K"],
                    a["M"], a["k"], a["cap"], a["T"], a["p"], a["ws"], a["wsb"], S)

    assert run(u=None) == NUL
    assert run(t=None) == NUL
    assert run(n=None) == NUL
    assert run(W=None) == NUL
    assert run(T=0.0) == ARG
    assert run(T=float("inf")) == ARG
    assert run(T=float("nan")) == ARG
    assert run(p=0.0) == ARG
    assert run(p=1.5) == ARG
    assert run(p=float("nan")) == ARG
    assert run(k=65) == ARG
    assert run(u=FAKE + 2) == ALIGN
    assert run(t=FAKE + 1) == ALIGN
    assert run(wsb=16) == WS
    assert run(K=48) == SHAPE
    assert call("qmvdbg_sample_f32", FAKE, FAKE, FAKE, FAKE, FAKE, 1, 65, 1.0, 0.9, S) == ARG
    assert call("qmvdbg_sample_f32", FAKE, FAKE, FAKE, FAKE, FAKE, 0, 10, 1.0, 0.9, S) == SHAPE
    assert call("qmvdbg_sample_f32", FAKE, None, FAKE, FAKE, FAKE, 1, 10, 1.0, 0.9, S) == NUL
    assert call("qmvdbg_sample_f32", FAKE, FAKE, FAKE, FAKE, FAKE, 1, 10, -1.0, 0.9, S) == ARG
    assert call("qmvdbg_sample_f32", FAKE + 1, FAKE, FAKE, FAKE, FAKE, 1, 10, 1.0, 0.9, S) == ALIGN


def test_debug_entry_validation():
    assert call("qmvdbg_quantize_q8", FAKE, FAKE, FAKE, 40, 1, S) == SHAPE
    assert call("qmvdbg_quantize_q8", None, FAKE, FAKE, 64, 1, S) == NUL
    bs = "qmvdbg_qmm_q4_0_q8act_blocksums"
    assert call(bs, FAKE, FAKE + 2, FAKE, 8, 64, 1, 0, 8, FAKE, 1 << 20, S) == ALIGN
    assert call(bs, FAKE, FAKE, FAKE, 8, 64, 1, 0, 8, FAKE + 8, 1 << 20, S) == ALIGN
    assert call(bs, FAKE, FAKE, FAKE, 8, 64, 1, 4, 4, FAKE, 1 << 20, S) == ARG
    assert call(bs, FAKE, FAKE, FAKE, 8, 64, 1, 0, 9, FAKE, 1 << 20, S) == ARG
    assert call(bs, FAKE, FAKE, FAKE, 8, 64, 1, -1, 2, FAKE, 1 << 20, S) == ARG
    assert call(bs, FAKE, FAKE, None, 8, 64, 1, 0, 8, FAKE, 1 << 20, S) == NUL
    assert call(bs, FAKE, FAKE, FAKE, 8, 64, 1, 0, 8, FAKE, 16, S) == WS
    assert call(bs, FAKE, FAKE, FAKE, 8, 48, 1, 0, 8, FAKE, 1 << 20, S) == SHAPE
    assert call("qmvdbg_topk_f32", FAKE, FAKE, FAKE, 100, 1, 101, 30.0, FAKE, 1 << 20, S) == ARG


def test_noalloc_topk_validation():
    """logits_topk_noalloc rejects, before it asks the runtime for its static
    workspace, every request that logits_topk would reject and every one
    whose workspace exceeds the 8 MiB static array."""
    f = "logits_topk_noalloc"
    assert call(f, None, FAKE, FAKE, FAKE, 1000, 64, 1, 10, 30.0, S) == NUL
    assert call(f, FAKE, FAKE, None, FAKE, 1000, 64, 1, 10, 30.0, S) == NUL
    assert call(f, FAKE, FAKE, FAKE, FAKE, 1000, 48, 1, 10, 30.0, S) == SHAPE
    assert call(f, FAKE, FAKE, FAKE, FAKE, 1000, 64, 1, 65, 30.0, S) == ARG
    assert call(f, FAKE, FAKE, FAKE, FAKE, 1000, 64, 1, 10, 0.0, S) == ARG
    assert call(f, FAKE + 8, FAKE, FAKE, FAKE, 1000, 64, 1, 10, 30.0, S) == ALIGN
    assert call(f, FAKE, FAKE, FAKE + 2, FAKE, 1000, 64, 1, 10, 30.0, S) == ALIGN
    # 262,144 logits: 7 rows fit at k = 10, 8 do not; 5 fit at k = 64, 6 do not
    assert qmv.logits_topk_ws_bytes(262144, 7, 10) <= 8 << 20 < qmv.logits_topk_ws_bytes(262144, 8, 10)
    assert qmv.logits_topk_ws_bytes(262144, 5, 64) <= 8 << 20 < qmv.logits_topk_ws_bytes(262144, 6, 64)
    assert call(f, FAKE, FAKE, FAKE, FAKE, 262144, 64, 8, 10, 30.0, S) == WS
    assert call(f, FAKE, FAKE, FAKE, FAKE, 262144, 64, 6, 64, 30.0, S) == WS


def test_stream_read_validation():
    assert call("qmvdbg_stream_read", None, 4096, FAKE, 8, S) == NUL
    assert call("qmvdbg_stream_read", FAKE, 4096, None, 8, S) == NUL
    assert call("qmvdbg_stream_read", FAKE, 0, FAKE, 8, S) == SHAPE
    assert call("qmvdbg_stream_read", FAKE, 4100, FAKE, 8, S) == SHAPE
    assert call("qmvdbg_stream_read", FAKE, 4096, FAKE, 0, S) == ARG
    assert call("qmvdbg_stream_read", FAKE, 4096, FAKE, 65537, S) == ARG
    assert call("qmvdbg_stream_read", FAKE + 8, 4096, FAKE, 8, S) == ALIGN
    assert call("qmvdbg_stream_read", FAKE, 4096, FAKE + 2, 8, S) == ALIGN
