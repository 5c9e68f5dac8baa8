"""Seeded synthetic inputs: packed Q4_0 / Q8_0 / Q4_K / Q6_K weight bytes and
f32 activations.

This module only draws random numbers and lays them out in the block
formats' byte layout; it holds none of the arithmetic of the method (no
dequantization, no dot product).  Both the HIP path and the CPU oracle consume
the very same bytes, so a reader can regenerate any test input from its seed.

Generator: numpy PCG64, one seed per workload.  Draw order inside one call:
block scales first (all blocks, row-major), then the code bytes (all blocks,
row-major), then the extra Q4_K fields (dmin, sub-block scales, sub-block
mins) or Q6_K fields (sub-block scales), and finally the activations.

Value distributions (the synthetic stand-ins for real model weights):
  Q4_0: d = fp16(|N(0,1)| * 0.02), q uniform in 0..15     (w = (q - 8) d)
  Q8_0: d = fp16(|N(0,1)| * 0.01), q uniform in -127..127 (w = q d)
  Q4_K: d, dmin = fp16(|N(0,1)| * 0.01), sub-block scales and mins uniform
        in 0..63, q uniform in 0..15
  Q6_K: d = fp16(|N(0,1)| * 0.0001) (about half of them fp16 subnormals,
        as in real Q6_K tensors), sub-block scales uniform int8 in
        -128..127, 6-bit q uniform in 0..63 (w = d s (q - 32))
  MXFP4 (two planes): E8M0 block exponents uniform in 116..124 (scales
        2^-11 .. 2^-3), E2M1 codes as whole uniform random bytes (every
        4-bit code, -0 included, uniform)
  x:    f32 ~ N(0,1)
N(0,1) is drawn in float32, scaled in float32 and rounded to fp16 by numpy
(round to nearest even, subnormals kept).  4-bit codes are drawn as whole
uniform random bytes, whose two nibbles are independent and uniform in 0..15.
Q8_0 codes are uniform random bytes read as int8; every -128 is drawn again
(in chunks of 2^24 codes, in order) until none is left, so they are uniform
in -127..127.

Byte layouts (GGUF block formats, as loaded by the pages' engines):
  Q4_0 (18 B / 32): fp16 d | 16 bytes, byte j = q[j] | q[j+16] << 4
  Q8_0 (34 B / 32): fp16 d | 32 int8
  Q4_K (144 B / 256): fp16 d | fp16 dmin | 12 bytes of 6-bit scales/mins |
        128 code bytes; byte 32c+l = q[64c+l] | q[64c+32+l] << 4
  Q6_K (210 B / 256): 128 bytes ql | 64 bytes qh | 16 int8 scales | fp16 d;
        element 128h+32g+l: low (g < 2) or high (g >= 2) nibble of
        ql[64h+32(g%2)+l], two high bits at bits 2g, 2g+1 of qh[32h+l]
  MXFP4: codes [N][K/32][16 B], element 2i in the low and 2i+1 in the high
        nibble of byte i; scales [N][K/32], one E8M0 byte per block
"""
from __future__ import annotations

import numpy as np

BLOCK_BYTES = {"q4_0": 18, "q8_0": 34, "q4_k": 144, "q6_k": 210}
BLOCK_ELEMS = {"q4_0": 32, "q8_0": 32, "q4_k": 256, "q6_k": 256}

# Seeds of the five workloads; the up-projection matrix of the gated pair
# uses its own seed.
SEEDS = {"c1": 101, "c2": 102, "c2_up": 1102, "c3": 103, "c4": 104, "c5": 105,
         "q6k_gate": 106, "q6k_down": 107, "qkv": 108, "q4k_down": 109, "mxfp4_gate": 110,
         "mxfp4_down": 111}


def row_bytes(fmt: str, K: int) -> int:
    e = BLOCK_ELEMS[fmt]
    if K % e:
        raise ValueError(f"K={K} is not a multiple of {e} for {fmt}")
    return K // e * BLOCK_BYTES[fmt]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _fp16_scales(rng: np.random.Generator, n: int, mult: float) -> np.ndarray:
    return (np.abs(rng.standard_normal(n, dtype=np.float32)) * np.float32(mult)).astype(np.float16)


def _random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def pack_q4_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """d: float16[nb], q: uint8[nb, 32] in 0..15 -> uint8[nb * 18]."""
    nb = d.size
    out = np.empty((nb, 18), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(nb, 2)
    out[:, 2:] = (q[:, :16] & 15) | ((q[:, 16:] & 15) << 4)
    return out.reshape(-1)


def pack_q8_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """d: float16[nb], q: int8[nb, 32] -> uint8[nb * 34]."""
    nb = d.size
    out = np.empty((nb, 34), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(nb, 2)
    out[:, 2:] = np.ascontiguousarray(q, dtype=np.int8).view(np.uint8)
    return out.reshape(-1)


def pack_q4_k_scales(sc: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """sc, mn: uint8[nb, 8] in 0..63 -> uint8[nb, 12] (6-bit packing)."""
    sc = sc.astype(np.uint8)
    mn = mn.astype(np.uint8)
    P = np.empty((sc.shape[0], 12), dtype=np.uint8)
    for j in range(4):
        P[:, j] = (sc[:, j] & 63) | ((sc[:, j + 4] >> 4) << 6)
        P[:, j + 4] = (mn[:, j] & 63) | ((mn[:, j + 4] >> 4) << 6)
        P[:, j + 8] = (sc[:, j + 4] & 15) | ((mn[:, j + 4] & 15) << 4)
    return P


def pack_q4_k(d, dmin, sc, mn, q) -> np.ndarray:
    """d, dmin: float16[nb]; sc, mn: uint8[nb, 8]; q: uint8[nb, 256] -> uint8[nb*144]."""
    nb = d.size
    out = np.empty((nb, 144), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = np.ascontiguousarray(dmin, dtype=np.float16).view(np.uint8).reshape(nb, 2)
    out[:, 4:16] = pack_q4_k_scales(sc, mn)
    qq = q.reshape(nb, 4, 64)
    out[:, 16:] = ((qq[:, :, :32] & 15) | ((qq[:, :, 32:] & 15) << 4)).reshape(nb, 128)
    return out.reshape(-1)


def pack_q6_k(d, sc, q) -> np.ndarray:
    """d: float16[nb]; sc: int8[nb, 16]; q: uint8[nb, 256] in 0..63 -> uint8[nb*210]."""
    nb = d.size
    q = np.asarray(q, dtype=np.uint8).reshape(nb, 2, 4, 32)  # [block, h, g, l]
    lo = q & 15
    hi = (q >> 4) & 3
    ql = np.empty((nb, 2, 2, 32), dtype=np.uint8)             # [block, h, g % 2, l]
    ql[:, :, 0] = lo[:, :, 0] | (lo[:, :, 2] << 4)
    ql[:, :, 1] = lo[:, :, 1] | (lo[:, :, 3] << 4)
    qh = hi[:, :, 0] | (hi[:, :, 1] << 2) | (hi[:, :, 2] << 4) | (hi[:, :, 3] << 6)
    out = np.empty((nb, 210), dtype=np.uint8)
    out[:, 0:128] = ql.reshape(nb, 128)
    out[:, 128:192] = qh.reshape(nb, 64)
    out[:, 192:208] = np.ascontiguousarray(sc, dtype=np.int8).view(np.uint8).reshape(nb, 16)
    out[:, 208:210] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(nb, 2)
    return out.reshape(-1)


def _blocks(nb: int, nbytes: int) -> np.ndarray:
    return np.empty((nb, nbytes), dtype=np.uint8)


def q4_0_weights(N: int, K: int, seed: int, rng=None) -> np.ndarray:
    rng = rng or _rng(seed)
    row_bytes("q4_0", K)
    nb = N * (K // 32)
    d = _fp16_scales(rng, nb, 0.02)
    out = _blocks(nb, 18)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:] = _random_bytes(rng, (nb, 16))
    return out.reshape(-1)


def q8_0_weights(N: int, K: int, seed: int, rng=None) -> np.ndarray:
    rng = rng or _rng(seed)
    row_bytes("q8_0", K)
    nb = N * (K // 32)
    d = _fp16_scales(rng, nb, 0.01)
    q = _random_bytes(rng, (nb, 32))
    flat = q.reshape(-1)
    chunk = 1 << 24
    for s in range(0, flat.size, chunk):
        c = flat[s:s + chunk]
        bad = c == 0x80
        n = int(np.count_nonzero(bad))
        while n:
            c[bad] = _random_bytes(rng, n)
            bad = c == 0x80
            n = int(np.count_nonzero(bad))
    out = _blocks(nb, 34)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:] = q
    return out.reshape(-1)


def q4_k_weights(N: int, K: int, seed: int, rng=None) -> np.ndarray:
    rng = rng or _rng(seed)
    row_bytes("q4_k", K)
    nb = N * (K // 256)
    d = _fp16_scales(rng, nb, 0.01)
    codes = _random_bytes(rng, (nb, 128))
    dmin = _fp16_scales(rng, nb, 0.01)
    sc = rng.integers(0, 64, size=(nb, 8), dtype=np.uint8)
    mn = rng.integers(0, 64, size=(nb, 8), dtype=np.uint8)
    out = _blocks(nb, 144)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    out[:, 4:16] = pack_q4_k_scales(sc, mn)
    out[:, 16:] = codes
    return out.reshape(-1)


def q6_k_weights(N: int, K: int, seed: int, rng=None) -> np.ndarray:
    rng = rng or _rng(seed)
    row_bytes("q6_k", K)
    nb = N * (K // 256)
    d = _fp16_scales(rng, nb, 0.0001)
    codes = _random_bytes(rng, (nb, 192))  # ql and qh: every 6-bit code uniform
    sc = _random_bytes(rng, (nb, 16))
    out = _blocks(nb, 210)
    out[:, 0:192] = codes
    out[:, 192:208] = sc
    out[:, 208:210] = d.view(np.uint8).reshape(nb, 2)
    return out.reshape(-1)


def mxfp4_weights(N: int, K: int, seed: int, rng=None):
    """(codes uint8[N * K/2], scales uint8[N * K/32]): block exponents first,
    then the code bytes."""
    rng = rng or _rng(seed)
    if K % 32:
        raise ValueError(f"K={K} is not a multiple of 32 for mxfp4")
    nb = N * (K // 32)
    scales = rng.integers(116, 125, size=nb, dtype=np.uint8)
    codes = _random_bytes(rng, nb * 16)
    return codes, scales


def mxfp4_problem(N: int, K: int, M: int, seed: int):
    rng = _rng(seed)
    codes, scales = mxfp4_weights(N, K, seed, rng=rng)
    x = activations(M, K, seed, rng=rng)
    return codes, scales, x


def activations(M: int, K: int, seed: int, rng=None) -> np.ndarray:
    rng = rng or _rng(seed)
    return rng.standard_normal(M * K, dtype=np.float32).reshape(M, K)


WEIGHTS = {"q4_0": q4_0_weights, "q8_0": q8_0_weights, "q4_k": q4_k_weights, "q6_k": q6_k_weights}


def problem(fmt: str, N: int, K: int, M: int, seed: int):
    """Weights then activations from one generator: (W bytes, x[M, K])."""
    rng = _rng(seed)
    W = WEIGHTS[fmt](N, K, seed, rng=rng)
    x = activations(M, K, seed, rng=rng)
    return W, x


# The five workloads (shapes of a 31B-class dense model: 5376 embedding,
# 21504 FFN, 262144 vocabulary).
CONFIGS = {
    "c1": dict(fmt="q4_0", N=4096, K=4096, M=1),
    "c2": dict(fmt="q4_0", N=21504, K=5376, M=1),
    "c3": dict(fmt="q8_0", N=262144, K=5376, M=1, k=10, softcap=30.0),
    "c4": dict(fmt="q4_0", N=5376, K=21504, Ms=(1, 16, 512)),
    "c5": dict(fmt="q4_k", N=21504, K=5376, M=1),
    # Q6_K at the FFN gate shape (the unit kernel's shape, next to c5) and at
    # the FFN down shape 5376 x 21504, where Q4_K_M files keep Q6_K
    "q6k_gate": dict(fmt="q6_k", N=21504, K=5376, M=1),
    "q6k_down": dict(fmt="q6_k", N=5376, K=21504, M=1),
    "q4k_down": dict(fmt="q4_k", N=5376, K=21504, M=1),
    # attention input projections of a Q4_K_M model at the 5376 embedding:
    # 32 query heads and 16 key/value heads of 128 (Q, K in Q4_K, V in Q6_K)
    "qkv": dict(Nq=4096, Nk=2048, Nv=2048, K=5376, M=1),
    # MXFP4 at the FFN gate and down shapes
    "mxfp4_gate": dict(fmt="mxfp4", N=21504, K=5376, M=1),
    "mxfp4_down": dict(fmt="mxfp4", N=5376, K=21504, M=1),
}


def config_problem(name: str, M: int | None = None):
    c = CONFIGS[name]
    m = M if M is not None else c.get("M", 1)
    return problem(c["fmt"], c["N"], c["K"], m, SEEDS[name])


def qkv_problem():
    """(Wq, Wk, Wv, x) of the attention projection workload: Q4_K Q and K,
    Q6_K V, each matrix from its own seed offset, x from the first."""
    c = CONFIGS["qkv"]
    seed = SEEDS["qkv"]
    Wq, x = problem("q4_k", c["Nq"], c["K"], 1, seed)
    Wk = q4_k_weights(c["Nk"], c["K"], seed + 1000)
    Wv = q6_k_weights(c["Nv"], c["K"], seed + 2000)
    return Wq, Wk, Wv, x


def gate_up_problem():
    """The gated pair at the FFN gate shape: (W_gate, W_up, x)."""
    c = CONFIGS["c2"]
    Wg, x = problem("q4_0", c["N"], c["K"], 1, SEEDS["c2"])
    Wu = q4_0_weights(c["N"], c["K"], SEEDS["c2_up"])
    return Wg, Wu, x
