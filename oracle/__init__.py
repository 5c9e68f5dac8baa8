"""CPU oracle for the fused-dequant quantized GEMV path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.

This module is argument marshalling around ``liboracle.so`` (plain C, float64,
see ``oracle.c`` for the definitions and the passages of the pages each one
follows) plus the tolerance rules the parity tests apply.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q4_0, Q8_0, Q4_K, Q6_K = 0, 1, 2, 3
FORMATS = {"q4_0": Q4_0, "q8_0": Q8_0, "q4_k": Q4_K, "q6_k": Q6_K}

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (no fast-math: IEEE float32 division and
    rounding are part of the quantizer's definition)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-std=gnu11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_fp16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_fp16_to_f64.restype = ctypes.c_double
    lib.oracle_row_bytes.argtypes = [ctypes.c_int, I64]
    lib.oracle_row_bytes.restype = I64
    lib.oracle_dequant_row.argtypes = [ctypes.c_int, P, I64, P]
    lib.oracle_q4_k_scale_min.argtypes = [P, ctypes.c_int, P, P]
    lib.oracle_qmv.argtypes = [ctypes.c_int, P, I64, I64, P, I64, P, I64, P, P]
    lib.oracle_gelu_tanh.argtypes = [ctypes.c_double]
    lib.oracle_gelu_tanh.restype = ctypes.c_double
    lib.oracle_geglu.argtypes = [P, P, I64, P]
    lib.oracle_e2m1_to_f64.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_to_f64.restype = ctypes.c_double
    lib.oracle_e8m0_to_f64.argtypes = [ctypes.c_int]
    lib.oracle_e8m0_to_f64.restype = ctypes.c_double
    lib.oracle_dequant_mxfp4_row.argtypes = [P, P, I64, P]
    lib.oracle_qmv_mxfp4.argtypes = [P, P, I64, I64, P, I64, P, I64, P, P]
    lib.oracle_qmv_geglu_down.argtypes = [ctypes.c_int, P, I64, I64, P, P, I64, P, I64, P, P, P]
    lib.oracle_softcap.argtypes = [P, I64, ctypes.c_double, P]
    lib.oracle_quantize_q8.argtypes = [P, I64, I64, P, P]
    lib.oracle_q4_0_q8_blocksums.argtypes = [P, I64, I64, P, I64, P, I64, P]
    lib.oracle_qmm_q4_0_q8.argtypes = [P, I64, I64, P, P, I64, P, I64, P, P]
    lib.oracle_topk.argtypes = [P, I64, ctypes.c_int32, P]
    lib.oracle_sample_topp.argtypes = [P, P, ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                       P, P, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _rows_arg(rows, N):
    if rows is None:
        return None, N
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, len(r)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops (for timing only)."""
    _load().oracle_set_num_threads(int(n))


def fp16_to_f64(h: int) -> float:
    return float(_load().oracle_fp16_to_f64(int(h) & 0xFFFF))


def row_bytes(fmt: str, K: int) -> int:
    return int(_load().oracle_row_bytes(FORMATS[fmt], K))


def dequant_row(fmt: str, row: np.ndarray, K: int) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    if row.size != row_bytes(fmt, K):
        raise ValueError("row has the wrong number of bytes")
    w = np.empty(K, dtype=np.float64)
    rc = _load().oracle_dequant_row(FORMATS[fmt], _ptr(row), K, _ptr(w))
    if rc:
        raise ValueError(f"oracle_dequant_row failed ({rc})")
    return w


def q4_k_scale_min(packed12: np.ndarray, j: int):
    p = np.ascontiguousarray(packed12, dtype=np.uint8)
    sc = ctypes.c_int()
    mn = ctypes.c_int()
    _load().oracle_q4_k_scale_min(_ptr(p), j, ctypes.byref(sc), ctypes.byref(mn))
    return sc.value, mn.value


def qmv(fmt: str, W: np.ndarray, N: int, K: int, x: np.ndarray, M: int = 1, rows=None):
    """float64 y[M, nrows] and S[M, nrows] = sum |w x| for the selected rows."""
    W = np.ascontiguousarray(W).view(np.uint8).reshape(-1)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    if W.size != N * row_bytes(fmt, K) or x.size != M * K:
        raise ValueError("shape mismatch")
    r, nrows = _rows_arg(rows, N)
    y = np.empty((M, nrows), dtype=np.float64)
    S = np.empty((M, nrows), dtype=np.float64)
    rc = _load().oracle_qmv(FORMATS[fmt], _ptr(W), N, K, _ptr(x), M,
                            None if r is None else _ptr(r), nrows, _ptr(y), _ptr(S))
    if rc:
        raise ValueError(f"oracle_qmv failed ({rc})")
    return y, S


def e2m1(code: int) -> float:
    return float(_load().oracle_e2m1_to_f64(int(code)))


def e8m0(e: int) -> float:
    return float(_load().oracle_e8m0_to_f64(int(e)))


def dequant_mxfp4_row(codes: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    scales = np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1)
    if K % 32 or codes.size != K // 2 or scales.size != K // 32:
        raise ValueError("shape mismatch")
    w = np.empty(K, dtype=np.float64)
    _load().oracle_dequant_mxfp4_row(_ptr(codes), _ptr(scales), K, _ptr(w))
    return w


def qmv_mxfp4(codes: np.ndarray, scales: np.ndarray, N: int, K: int, x: np.ndarray, M: int = 1, rows=None):
    """float64 y[M, nrows] and S = sum |w x| for an MXFP4 matrix (two planes)."""
    codes = np.ascontiguousarray(codes).view(np.uint8).reshape(-1)
    scales = np.ascontiguousarray(scales).view(np.uint8).reshape(-1)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    if K % 32 or codes.size != N * K // 2 or scales.size != N * K // 32 or x.size != M * K:
        raise ValueError("shape mismatch")
    r, nrows = _rows_arg(rows, N)
    y = np.empty((M, nrows), dtype=np.float64)
    S = np.empty((M, nrows), dtype=np.float64)
    rc = _load().oracle_qmv_mxfp4(_ptr(codes), _ptr(scales), N, K, _ptr(x), M,
                                  None if r is None else _ptr(r), nrows, _ptr(y), _ptr(S))
    if rc:
        raise ValueError(f"oracle_qmv_mxfp4 failed ({rc})")
    return y, S


def gelu_tanh(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    lib = _load()
    return np.vectorize(lambda t: lib.oracle_gelu_tanh(float(t)), otypes=[np.float64])(v)


def geglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64).reshape(-1)
    u = np.ascontiguousarray(u, dtype=np.float64).reshape(-1)
    h = np.empty_like(g)
    _load().oracle_geglu(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def qmv_geglu_down(fmt: str, W: np.ndarray, N: int, K: int, g: np.ndarray, u: np.ndarray, M: int = 1, rows=None):
    """float64 y[M, nrows] = W (gelu(g) * u), with S = sum |w h| and
    E = sum |w| |u| (|g| + |gelu(g)|) for the selected rows."""
    W = np.ascontiguousarray(W).view(np.uint8).reshape(-1)
    g = np.ascontiguousarray(g, dtype=np.float32).reshape(-1)
    u = np.ascontiguousarray(u, dtype=np.float32).reshape(-1)
    if W.size != N * row_bytes(fmt, K) or g.size != M * K or u.size != M * K:
        raise ValueError("shape mismatch")
    r, nrows = _rows_arg(rows, N)
    y = np.empty((M, nrows), dtype=np.float64)
    S = np.empty((M, nrows), dtype=np.float64)
    E = np.empty((M, nrows), dtype=np.float64)
    rc = _load().oracle_qmv_geglu_down(FORMATS[fmt], _ptr(W), N, K, _ptr(g), _ptr(u), M,
                                       None if r is None else _ptr(r), nrows, _ptr(y), _ptr(S), _ptr(E))
    if rc:
        raise ValueError(f"oracle_qmv_geglu_down failed ({rc})")
    return y, S, E


def softcap(y: np.ndarray, cap: float) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64).reshape(-1)
    z = np.empty_like(y)
    _load().oracle_softcap(_ptr(y), y.size, float(cap), _ptr(z))
    return z


def quantize_q8(x: np.ndarray, M: int, K: int):
    """int8 codes [M, K] and float32 scales [M, K/32] (float32 arithmetic)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    if x.size != M * K:
        raise ValueError("shape mismatch")
    q = np.empty((M, K), dtype=np.int8)
    d = np.empty((M, K // 32), dtype=np.float32)
    rc = _load().oracle_quantize_q8(_ptr(x), M, K, _ptr(q), _ptr(d))
    if rc:
        raise ValueError(f"oracle_quantize_q8 failed ({rc})")
    return q, d


def q4_0_q8_blocksums(W: np.ndarray, N: int, K: int, qx: np.ndarray, M: int, rows=None):
    """int32 isum[M, nrows, K/32] (exact, overflow-checked)."""
    W = np.ascontiguousarray(W).view(np.uint8).reshape(-1)
    qx = np.ascontiguousarray(qx, dtype=np.int8).reshape(-1)
    r, nrows = _rows_arg(rows, N)
    out = np.empty((M, nrows, K // 32), dtype=np.int32)
    rc = _load().oracle_q4_0_q8_blocksums(_ptr(W), N, K, _ptr(qx), M,
                                          None if r is None else _ptr(r), nrows, _ptr(out))
    if rc:
        raise ValueError(f"oracle_q4_0_q8_blocksums failed ({rc})")
    return out


def qmm_q4_0_q8(W: np.ndarray, N: int, K: int, qx: np.ndarray, dx: np.ndarray, M: int, rows=None):
    W = np.ascontiguousarray(W).view(np.uint8).reshape(-1)
    qx = np.ascontiguousarray(qx, dtype=np.int8).reshape(-1)
    dx = np.ascontiguousarray(dx, dtype=np.float32).reshape(-1)
    r, nrows = _rows_arg(rows, N)
    y = np.empty((M, nrows), dtype=np.float64)
    S = np.empty((M, nrows), dtype=np.float64)
    rc = _load().oracle_qmm_q4_0_q8(_ptr(W), N, K, _ptr(qx), _ptr(dx), M,
                                    None if r is None else _ptr(r), nrows, _ptr(y), _ptr(S))
    if rc:
        raise ValueError(f"oracle_qmm_q4_0_q8 failed ({rc})")
    return y, S


def topk(y: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best values: descending, ties to the lower index,
    NaN after all numbers (full stable sort)."""
    y = np.ascontiguousarray(y, dtype=np.float64).reshape(-1)
    out = np.empty(k, dtype=np.int32)
    rc = _load().oracle_topk(_ptr(y), y.size, k, _ptr(out))
    if rc:
        raise ValueError(f"oracle_topk failed ({rc})")
    return out


def sample_topp(z, idx, T: float, top_p: float, u: float):
    """(token, nucleus size, prefix sums of the weights) for one row of k
    sorted pairs: softmax at temperature T over z, top-p nucleus, inverse-CDF
    draw with the uniform u (oracle_sample_topp)."""
    z = np.ascontiguousarray(z, dtype=np.float64).reshape(-1)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1)
    k = z.size
    cum = np.empty(k, dtype=np.float64)
    tok = np.zeros(1, dtype=np.int32)
    nuc = np.zeros(1, dtype=np.int32)
    rc = _load().oracle_sample_topp(_ptr(z), _ptr(idx), k, float(T), float(top_p), float(u), _ptr(tok), _ptr(nuc),
                                    _ptr(cum))
    if rc:
        raise ValueError(f"oracle_sample_topp failed ({rc})")
    return int(tok[0]), int(nuc[0]), cum


# --------------------------------------------------------------------------
# Tolerances.  The float bound is the one the target states for every float
# output: |y - y_ref| <= 1e-5 * sum_i |w_i x_i| + 1e-6.
# --------------------------------------------------------------------------
REL_TOL = 1e-5
ABS_TOL = 1e-6


def float_tol(S: np.ndarray) -> np.ndarray:
    return REL_TOL * np.asarray(S, dtype=np.float64) + ABS_TOL


# float32 evaluation of h = gelu(g) * u: |dh| <= 2^-20 |u| (|g| + |gelu(g)|).
# The inner polynomial has no cancellation (v and 0.044715 v^3 share a sign),
# so it carries a few float32 roundings.  Evaluated as v/2 (1 + tanhf(z)),
# tanhf adds a couple of ulps and at most 0.45 times the inner's relative
# error, and 1 + t, the products and the halving a few more: about 8 units of
# 2^-24 on |g| |u|.  Evaluated as the same function v / (1 + e^(-2z)), the
# exponential, sum, reciprocal and products add about 6 units on |gelu(g)| |u|,
# and the rounding of the exponent's argument at most 0.37 units on |g| |u|
# (x e^-x <= 1/e).  2^-20 = 16 units leaves a factor-2 margin over either.
H_F32_REL = 2.0**-20


def geglu_down_tol(S, E):
    """|y - y_ref| <= 1e-5 S + 2^-20 E + 1e-6 for y = W (gelu(g) * u): the
    linear bound on the products, plus the propagated float32 error of h."""
    return float_tol(S) + H_F32_REL * np.asarray(E, dtype=np.float64)


def geglu_tol(g_ref, u_ref, Sg, Su, h_ref):
    """First-order propagation of the linear bound through h = gelu(g) * u.
    sup |gelu'| < 1.13, so |dh| <= 1.13 Tg (|u| + Tu) + |gelu(g)| Tu, plus a
    relative 1e-6 for the float32 evaluation of gelu and the product."""
    Tg = float_tol(Sg)
    Tu = float_tol(Su)
    gg = gelu_tanh(g_ref)
    return 1.13 * Tg * (np.abs(u_ref) + Tu) + np.abs(gg) * Tu + 1e-6 * np.abs(h_ref) + 1e-6
