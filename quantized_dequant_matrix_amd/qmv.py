"""Python binding of libqmv.so (argument marshalling only).

Every function has the name and argument order of the C entry point declared
in include/qmv.h.  Buffer arguments are torch tensors on the GPU (or raw
device addresses as ints); sizes are ints; ``stream`` is a torch stream (None:
torch's current stream).  A non-zero status raises QmvError.  All compute
happens in the HIP kernels of libqmv.so; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so that libqmv.so binds to torch's HIP runtime

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmv.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python -m quantized_dequant_matrix_amd.build`")

lib = ctypes.CDLL(_LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_F = ctypes.c_float

_SIGS = {
    "qmv_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "qmv_q4_0": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q8_0": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q4_k": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q6_k": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_mxfp4": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q4_0_geglu": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q4_0_geglu_down": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q4_k_geglu_down": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q6_k_geglu_down": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q4_k_q6_k_qkv": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmm_q4_0_q8act_ws_bytes": ([_I64, _I64, _I64], _SZ),
    "qmm_q4_0_q8act": ([_P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], ctypes.c_int),
    "qmm_q4_0_f32act_ws_bytes": ([_I64, _I64, _I64], _SZ),
    "qmm_q4_0_f32act": ([_P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], ctypes.c_int),
    "logits_topk_ws_bytes": ([_I64, _I64, _I32], _SZ),
    "logits_topk": ([_P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _P, _SZ, _P], ctypes.c_int),
    "logits_topk_noalloc": ([_P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _P], ctypes.c_int),
    "logits_sample": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _F, _F, _F, _P, _SZ, _P], ctypes.c_int),
    "qmvdbg_quantize_q8": ([_P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "qmvdbg_qmm_q4_0_q8act_blocksums": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _SZ, _P], ctypes.c_int),
    "qmvdbg_topk_f32": ([_P, _P, _P, _I64, _I64, _I32, _F, _P, _SZ, _P], ctypes.c_int),
    "qmvdbg_sample_f32": ([_P, _P, _P, _P, _P, _I64, _I32, _F, _F, _P], ctypes.c_int),
    "qmvdbg_stream_read": ([_P, _I64, _P, _I32, _P], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTS = tuple(_SIGS)

QMV_OK, QMV_ERR_NULL, QMV_ERR_SHAPE, QMV_ERR_ALIGN, QMV_ERR_WORKSPACE, QMV_ERR_LAUNCH, QMV_ERR_ARG = range(7)


class QmvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def status_str(status: int) -> str:
    return lib.qmv_status_str(status).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _call(name: str, *args) -> None:
    rc = getattr(lib, name)(*args)
    if rc != QMV_OK:
        raise QmvError(rc, name)


def qmv_q4_0(W, x, y, N, K, M=1, stream=None):
    _call("qmv_q4_0", _ptr(W), _ptr(x), _ptr(y), N, K, M, _stream(stream))


def qmv_q8_0(W, x, y, N, K, M=1, stream=None):
    _call("qmv_q8_0", _ptr(W), _ptr(x), _ptr(y), N, K, M, _stream(stream))


def qmv_q4_k(W, x, y, N, K, M=1, stream=None):
    _call("qmv_q4_k", _ptr(W), _ptr(x), _ptr(y), N, K, M, _stream(stream))


def qmv_q6_k(W, x, y, N, K, M=1, stream=None):
    _call("qmv_q6_k", _ptr(W), _ptr(x), _ptr(y), N, K, M, _stream(stream))


def qmv_mxfp4(W_codes, W_scales, x, y, N, K, M=1, stream=None):
    _call("qmv_mxfp4", _ptr(W_codes), _ptr(W_scales), _ptr(x), _ptr(y), N, K, M, _stream(stream))


def qmv_q4_0_geglu(W_gate, W_up, x, h, N, K, M=1, stream=None):
    _call("qmv_q4_0_geglu", _ptr(W_gate), _ptr(W_up), _ptr(x), _ptr(h), N, K, M, _stream(stream))


def qmv_q4_0_geglu_down(W_down, g, u, y, N, K, M=1, stream=None):
    _call("qmv_q4_0_geglu_down", _ptr(W_down), _ptr(g), _ptr(u), _ptr(y), N, K, M, _stream(stream))


def qmv_q4_k_geglu_down(W_down, g, u, y, N, K, M=1, stream=None):
    _call("qmv_q4_k_geglu_down", _ptr(W_down), _ptr(g), _ptr(u), _ptr(y), N, K, M, _stream(stream))


def qmv_q6_k_geglu_down(W_down, g, u, y, N, K, M=1, stream=None):
    _call("qmv_q6_k_geglu_down", _ptr(W_down), _ptr(g), _ptr(u), _ptr(y), N, K, M, _stream(stream))


def qmv_q4_k_q6_k_qkv(Wq, Wk, Wv, x, q, k, v, Nq, Nk, Nv, K, M=1, stream=None):
    _call("qmv_q4_k_q6_k_qkv", _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(x), _ptr(q), _ptr(k), _ptr(v), Nq, Nk, Nv, K, M,
          _stream(stream))


def qmm_q4_0_q8act_ws_bytes(N, K, M) -> int:
    return int(lib.qmm_q4_0_q8act_ws_bytes(N, K, M))


def qmm_q4_0_q8act(W, x, y, N, K, M, ws, ws_bytes, stream=None):
    _call("qmm_q4_0_q8act", _ptr(W), _ptr(x), _ptr(y), N, K, M, _ptr(ws), ws_bytes, _stream(stream))


def qmm_q4_0_f32act_ws_bytes(N, K, M) -> int:
    return int(lib.qmm_q4_0_f32act_ws_bytes(N, K, M))


def qmm_q4_0_f32act(W, x, y, N, K, M, ws, ws_bytes, stream=None):
    _call("qmm_q4_0_f32act", _ptr(W), _ptr(x), _ptr(y), N, K, M, _ptr(ws), ws_bytes, _stream(stream))


def logits_topk_ws_bytes(N, M, k) -> int:
    return int(lib.logits_topk_ws_bytes(N, M, k))


def logits_topk(W_q8_0, x, top_val, top_idx, N, K, M, k, softcap, ws, ws_bytes, stream=None):
    _call("logits_topk", _ptr(W_q8_0), _ptr(x), _ptr(top_val), _ptr(top_idx), N, K, M, k, softcap,
          _ptr(ws), ws_bytes, _stream(stream))


def logits_topk_noalloc(W_q8_0, x, top_val, top_idx, N, K, M, k, softcap, stream=None):
    _call("logits_topk_noalloc", _ptr(W_q8_0), _ptr(x), _ptr(top_val), _ptr(top_idx), N, K, M, k, softcap,
          _stream(stream))


def qmvdbg_quantize_q8(x, q, d, K, M, stream=None):
    _call("qmvdbg_quantize_q8", _ptr(x), _ptr(q), _ptr(d), K, M, _stream(stream))


def qmvdbg_qmm_q4_0_q8act_blocksums(W, x, isum, N, K, M, n0, n1, ws, ws_bytes, stream=None):
    _call("qmvdbg_qmm_q4_0_q8act_blocksums", _ptr(W), _ptr(x), _ptr(isum), N, K, M, n0, n1, _ptr(ws), ws_bytes,
          _stream(stream))


def qmvdbg_topk_f32(y, top_val, top_idx, N, M, k, softcap, ws, ws_bytes, stream=None):
    _call("qmvdbg_topk_f32", _ptr(y), _ptr(top_val), _ptr(top_idx), N, M, k, softcap, _ptr(ws), ws_bytes,
          _stream(stream))


def logits_sample(W_q8_0, x, u, token, nucleus, top_val, top_idx, N, K, M, k, softcap, temperature, top_p, ws,
                  ws_bytes, stream=None):
    _call("logits_sample", _ptr(W_q8_0), _ptr(x), _ptr(u), _ptr(token), _ptr(nucleus), _ptr(top_val),
          _ptr(top_idx), N, K, M, k, softcap, temperature, top_p, _ptr(ws), ws_bytes, _stream(stream))


def qmvdbg_sample_f32(top_val, top_idx, u, token, nucleus, M, k, temperature, top_p, stream=None):
    _call("qmvdbg_sample_f32", _ptr(top_val), _ptr(top_idx), _ptr(u), _ptr(token), _ptr(nucleus), M, k,
          temperature, top_p, _stream(stream))


def qmvdbg_stream_read(p, nbytes, out, workgroups, stream=None):
    _call("qmvdbg_stream_read", _ptr(p), nbytes, _ptr(out), workgroups, _stream(stream))
