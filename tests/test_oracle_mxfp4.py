"""Pins of the oracle's MXFP4 decoders and product: E8M0 against torch's
float8_e8m0fnu for every byte; E2M1 against a generic minifloat decoder
written here and checked first on two library formats (numpy float16,
torch float8_e4m3fn); the plane layout and element order on hand-built
blocks; an exact rational brute force; the e_i column identity."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from quantized_dequant_matrix_amd import synth


def minifloat(bits: int, ebits: int, mbits: int, bias: int) -> Fraction:
    """Value of a finite sign/exponent/mantissa code as an exact fraction
    (exponent 0 is subnormal: 2^(1-bias) * m / 2^mbits)."""
    sign = -1 if (bits >> (ebits + mbits)) & 1 else 1
    e = (bits >> mbits) & ((1 << ebits) - 1)
    m = bits & ((1 << mbits) - 1)
    if e == 0:
        mag = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return sign * mag


def test_minifloat_decoder_matches_float16():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in range(0, 65536, 7):
        if (b >> 10) & 31 == 31:
            continue  # inf / NaN
        assert float(minifloat(b, 5, 10, 15)) == ref[b]


def test_minifloat_decoder_matches_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        if b & 0x7F == 0x7F:
            continue  # NaN codes of e4m3fn
        assert float(minifloat(b, 4, 3, 7)) == ref[b]


def test_e2m1_all_codes():
    for c in range(16):
        got = oracle.e2m1(c)
        assert got == float(minifloat(c, 2, 1, 1))
        assert np.signbit(got) == bool(c & 8)
    assert oracle.e2m1(7) == 6.0 and oracle.e2m1(1) == 0.5


def test_e8m0_all_bytes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for e in range(256):
        got = oracle.e8m0(e)
        if np.isnan(ref[e]):
            assert np.isnan(got)
        else:
            assert got == ref[e]
    assert oracle.e8m0(0) == 2.0**-127 and oracle.e8m0(254) == 2.0**127


def test_block_layout_and_element_order():
    codes = np.array([(i & 15) | ((15 - i) << 4) for i in range(16)], np.uint8)
    w = oracle.dequant_mxfp4_row(codes, np.array([126], np.uint8), 32)
    for i in range(16):
        assert w[2 * i] == 0.5 * float(minifloat(i, 2, 1, 1))
        assert w[2 * i + 1] == 0.5 * float(minifloat(15 - i, 2, 1, 1))
    # two blocks: the second block's scale applies to elements 32..63 only
    codes2 = np.concatenate([np.full(16, 0x22, np.uint8), np.full(16, 0x77, np.uint8)])
    w2 = oracle.dequant_mxfp4_row(codes2, np.array([127, 130], np.uint8), 64)
    assert np.all(w2[:32] == 1.0) and np.all(w2[32:] == 6.0 * 8)


def test_nan_scale_and_extreme_scales():
    codes = np.full(16, 0x71, np.uint8)  # 0.5 and 6
    assert np.all(np.isnan(oracle.dequant_mxfp4_row(codes, np.array([255], np.uint8), 32)))
    w = oracle.dequant_mxfp4_row(codes, np.array([0], np.uint8), 32)
    assert w[0] == 2.0**-128 and w[1] == 6 * 2.0**-127


@pytest.mark.parametrize("K", [32, 64, 256])
def test_brute_force_exact(K):
    N = 4
    codes, scales, x = synth.mxfp4_problem(N, K, 1, seed=2000 + K)
    y, S = oracle.qmv_mxfp4(codes, scales, N, K, x)
    cb = codes.reshape(N, K // 32, 16)
    sb = scales.reshape(N, K // 32)
    xf = [Fraction(float(v)) for v in x[0]]
    for n in range(N):
        w = []
        for b in range(K // 32):
            sc = Fraction(2) ** (int(sb[n, b]) - 127)
            for i in range(16):
                w.append(minifloat(int(cb[n, b, i]) & 15, 2, 1, 1) * sc)
                w.append(minifloat(int(cb[n, b, i]) >> 4, 2, 1, 1) * sc)
        exact = sum(a * b for a, b in zip(w, xf))
        sabs = sum(abs(a * b) for a, b in zip(w, xf))
        bound = K * 2.0**-53 * float(sabs)
        assert abs(y[0, n] - float(exact)) <= bound
        assert abs(S[0, n] - float(sabs)) <= bound


def test_unit_vector_gives_column():
    N, K = 6, 96
    codes, scales, _ = synth.mxfp4_problem(N, K, 1, seed=3)
    for i in (0, 1, 2, 31, 32, 33, 95):
        e = np.zeros((1, K), np.float32)
        e[0, i] = 1.0
        y, _ = oracle.qmv_mxfp4(codes, scales, N, K, e)
        col = [oracle.dequant_mxfp4_row(codes[n * K // 2:(n + 1) * K // 2], scales[n * K // 32:(n + 1) * K // 32], K)[i]
               for n in range(N)]
        assert y[0].tolist() == col


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.qmv_mxfp4(np.zeros(16, np.uint8), np.zeros(1, np.uint8), 1, 48, np.zeros((1, 48), np.float32))
