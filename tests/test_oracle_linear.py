"""Pins of the oracle's dense MXFP4 linear layer (y = bf16(sum_k x_k w_nk), fp32 accumulate).

Checked against: one-hot row extraction, exact rational sums (brute force),
numpy fp64 matmul at unit scale, and exact sign / power-of-two invariants.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic

U32 = 2.0 ** -24  # fp32 unit roundoff


def bf16_to_f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f_to_bf16_exact(v: np.ndarray) -> np.ndarray:
    """Bits of fp32 values that are exactly representable in bf16."""
    u = np.asarray(v, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


@pytest.fixture(scope="module")
def mags(golden_dir):
    with open(os.path.join(golden_dir, "mxfp4_format.json")) as f:
        return json.load(f)["magnitudes"]


def decode_py(w, s, mags):
    """Independent numpy decode: nibble 2j low, scale per 32 consecutive K."""
    rows, kb = w.shape
    K = kb * 2
    codes = np.empty((rows, K), np.int64)
    codes[:, 0::2] = w & 15
    codes[:, 1::2] = w >> 4
    table = np.array(mags + [-m for m in mags], np.float64)
    sc = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    return table[codes] * sc


def ulp_bf16(v: float) -> float:
    a = abs(v)
    if a < 2.0 ** -126:
        return 2.0 ** -133
    return 2.0 ** (math.floor(math.log2(a)) - 7)


def test_one_hot_extracts_weight_column(mags):
    rng = np.random.default_rng(1)
    K, N = 96, 8
    w = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.integers(115, 135, size=(N, K // 32), dtype=np.uint8)
    W = decode_py(w, s, mags)
    one = np.uint16(0x3F80)  # bf16 1.0
    for k in range(K):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = one
        y, acc, sd = oracle.mx_linear(x, w, s, 1, K, N)
        assert np.array_equal(acc[0], W[:, k].astype(np.float32) + np.float32(0.0))
        nz = W[:, k] != 0
        assert np.array_equal(y[0, nz], f_to_bf16_exact(W[nz, k].astype(np.float32)))
        assert np.all(y[0, ~nz] == 0)  # +0 + (+-0) = +0


@pytest.mark.parametrize("T,K,N", [(1, 32, 4), (2, 64, 8), (3, 96, 5)])
def test_exact_rational_sums(T, K, N, mags):
    rng = np.random.default_rng(100 + K)
    x = synthetic.bf16_bits_normal((T, K), seed=K)
    w = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.integers(120, 130, size=(N, K // 32), dtype=np.uint8)
    y, acc, sd = oracle.mx_linear(x, w, s, T, K, N)
    xf = bf16_to_f(x).astype(np.float64)
    W = decode_py(w, s, mags)
    for t in range(T):
        for n in range(N):
            exact = sum(Fraction(float(xf[t, k])) * Fraction(float(W[n, k])) for k in range(K))
            absum = sum(abs(Fraction(float(xf[t, k])) * Fraction(float(W[n, k]))) for k in range(K))
            bound = (K - 1) * Fraction(U32) * absum
            assert abs(Fraction(float(acc[t, n])) - exact) <= bound
            assert float(sd[t, n]) == pytest.approx(float(absum), rel=1e-15)
            yv = float(bf16_to_f([y[t, n]])[0])
            assert abs(Fraction(yv) - exact) <= bound + Fraction(ulp_bf16(yv)) / 2


def test_unit_scale_matches_numpy_matmul(mags):
    rng = np.random.default_rng(7)
    T, K, N = 3, 512, 16
    x = synthetic.bf16_bits_normal((T, K), seed=9)
    w = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = np.full((N, K // 32), 127, np.uint8)
    y, acc, sd = oracle.mx_linear(x, w, s, T, K, N)
    xf = bf16_to_f(x).astype(np.float64)
    W = decode_py(w, s, mags)
    ref = xf @ W.T
    absum = np.abs(xf) @ np.abs(W).T
    assert np.all(np.abs(acc - ref) <= (K - 1) * U32 * absum + 1e-30)


def test_sign_flip_negates_exactly():
    cfg = synthetic.LinearConfig("t", T=2, K=256, N=32, e_lo=-4, e_hi=2, seed=3)
    x, w, s = synthetic.linear_inputs(cfg)
    y, acc, _ = oracle.mx_linear(x, w, s, 2, 256, 32)
    y2, acc2, _ = oracle.mx_linear(x, w ^ np.uint8(0x88), s, 2, 256, 32)
    nz = acc != 0
    assert np.array_equal(acc2[nz], -acc[nz])
    assert np.array_equal(y2[nz], y[nz] ^ np.uint16(0x8000))


def test_scale_increment_doubles_column():
    cfg = synthetic.LinearConfig("t", T=2, K=256, N=16, e_lo=-4, e_hi=2, seed=4)
    x, w, s = synthetic.linear_inputs(cfg)
    y, acc, _ = oracle.mx_linear(x, w, s, 2, 256, 16)
    s2 = s.copy()
    s2[5] += 1
    y2, acc2, _ = oracle.mx_linear(x, w, s2, 2, 256, 16)
    assert np.array_equal(acc2[:, 5], acc[:, 5] * 2)
    others = [n for n in range(16) if n != 5]
    assert np.array_equal(acc2[:, others], acc[:, others])
    nz = acc[:, 5] != 0
    assert np.array_equal(y2[nz, 5], y[nz, 5] + np.uint16(0x0080))  # exponent + 1


def test_zero_input_gives_positive_zero():
    cfg = synthetic.LinearConfig("t", T=2, K=128, N=8, e_lo=-4, e_hi=2, seed=5)
    _, w, s = synthetic.linear_inputs(cfg)
    x = np.zeros((2, 128), np.uint16)
    y, acc, sd = oracle.mx_linear(x, w, s, 2, 128, 8)
    assert np.all(y == 0) and np.all(sd == 0)


def test_nan_scale_propagates():
    cfg = synthetic.LinearConfig("t", T=1, K=128, N=4, e_lo=-4, e_hi=2, seed=6)
    x, w, s = synthetic.linear_inputs(cfg)
    s = s.copy()
    s[2, 3] = 255
    y, acc, _ = oracle.mx_linear(x, w, s, 1, 128, 4)
    assert math.isnan(acc[0, 2]) and (y[0, 2] & 0x7FFF) > 0x7F80
    assert not np.isnan(acc[0, [0, 1, 3]]).any()
