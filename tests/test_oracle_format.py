"""Pins of the oracle's MXFP4 decode against the format the pages fix.

The code table, scale bytes, packing and bf16 rounding are each checked against
something other than the oracle: the page's magnitude list (golden fixture),
the E2M1 float definition, math.ldexp, and torch's float32 -> bfloat16 cast.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


@pytest.fixture(scope="module")
def fmt(golden_dir):
    with open(os.path.join(golden_dir, "mxfp4_format.json")) as f:
        return json.load(f)


def test_e2m1_magnitudes_match_page(fmt):
    mags = [oracle.e2m1(c) for c in range(8)]
    assert mags == fmt["magnitudes"]
    for c in range(8):
        neg = oracle.e2m1(c | 8)
        assert neg == -mags[c]
        assert math.copysign(1.0, neg) == -1.0  # code 8 is -0.0


def test_e2m1_is_the_1_2_1_float():
    # E2M1: sign bit, 2 exponent bits with bias 1, 1 mantissa bit, exponent 0 subnormal.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1 + m / 2)
        v = -v if s else v
        assert oracle.e2m1(c) == v and math.copysign(1, oracle.e2m1(c)) == math.copysign(1, v)


def test_e8m0_all_bytes(fmt):
    for s in range(256):
        v = oracle.e8m0(s)
        if s == fmt["e8m0_nan_byte"]:
            assert math.isnan(v)
        else:
            assert v == math.ldexp(1.0, s - fmt["e8m0_bias"])
    assert oracle.e8m0(0) == 2.0 ** -127  # no zero encoding


def test_bits_per_value(fmt):
    block_bytes = fmt["block_size"] * fmt["element_bits"] // 8 + fmt["scale_bits"] // 8
    assert block_bytes * 8 / fmt["block_size"] == fmt["bits_per_value"]
    assert abs(16 / fmt["bits_per_value"] - fmt["bytes_ratio_vs_bf16_approx"]) < 0.05
    assert abs(fmt["bits_per_value"] / 8 - fmt["bytes_ratio_vs_fp8_approx"]) < 0.05


def test_pack_unpack_roundtrip():
    allb = np.arange(256, dtype=np.uint8)
    codes = oracle.unpack_codes(allb)
    assert np.array_equal(codes[0::2], allb & 15) and np.array_equal(codes[1::2], allb >> 4)
    assert np.array_equal(oracle.pack_codes(codes), allb)
    rng = np.random.default_rng(5)
    c = rng.integers(0, 16, size=4096, dtype=np.uint8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(c)), c)
    assert oracle.pack_codes(np.array([1, 2], np.uint8))[0] == 0x21  # element 0 in the low nibble


def test_dequant_indexing(fmt):
    rng = np.random.default_rng(11)
    rows, K = 5, 96
    w = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s = rng.integers(100, 140, size=(rows, K // 32), dtype=np.uint8)
    s[2, 1] = 255
    got = oracle.dequant(w, s, rows, K)
    mags = fmt["magnitudes"]
    for r in range(rows):
        for k in range(K):
            byte = int(w[r, k // 2])
            code = (byte >> 4) if (k % 2) else (byte & 15)
            sc = int(s[r, k // 32])
            if sc == 255:
                assert math.isnan(got[r, k])
                continue
            v = mags[code & 7] * 2.0 ** (sc - 127) * (-1 if code & 8 else 1)
            assert got[r, k] == v


def _torch_bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def test_bf16_rne_matches_torch_cast_on_floats():
    rng = np.random.default_rng(3)
    f = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(1e3),
        (rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895313e38, 3.3961775e38, 1e-40,
                  -1e-42, 9.2e-41], np.float32),
    ])
    f = f[np.isfinite(f)]
    want = _torch_bf16_bits(f)
    got = np.array([oracle.bf16_rne(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rne_on_doubles_is_nearest():
    # Brute force: the result is the nearest of the two bf16 neighbours (ties to even).
    rng = np.random.default_rng(4)
    vals = list(rng.standard_normal(300) * 10.0) + [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40]
    for v in vals:
        b = oracle.bf16_rne(v)
        r = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        e = math.frexp(abs(v))[1]
        q = Fraction(2) ** (e - 8)
        lo = (Fraction(abs(v)) // q) * q
        cands = [lo, lo + q]
        dists = [abs(Fraction(abs(v)) - c) for c in cands]
        if dists[0] != dists[1]:
            best = cands[0] if dists[0] < dists[1] else cands[1]
        else:  # tie: even significand
            best = cands[0] if (lo / q) % 2 == 0 else cands[1]
        assert Fraction(abs(r)) == best and math.copysign(1, r) == math.copysign(1, v)
