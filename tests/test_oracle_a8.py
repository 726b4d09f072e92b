"""Pins of the oracle's MXFP8 activation functions (the AMD megakernel blog, "Bringing
Ultra-Fast, Interactive LLM Inference to AMD Instinct MI355X GPUs", section "3. Low-Precision
Data Types": MXFP4 weights with MXFP8 activations).

E4M3 decode and rounding are checked against torch's float8_e4m3fn (a library
implementation of the same OCP format), the nearest-value rule by enumeration, the scale
rule by closed forms, and the a8 layers by reduction to the pinned bf16 layers and by exact
rational sums on tiny shapes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.test_oracle_moe import bf16_to_f, decode_py, tiny_cfg, ulp_bf16, U32

ALL_CODES = np.arange(256, dtype=np.uint8)


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_cast_e4m3(v):
    """Round float64 values (exact in fp32) to E4M3 codes with torch (nearest, ties to even)."""
    t = torch.from_numpy(np.asarray(v, np.float64).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def f_to_bf16_bits(v):
    return np.array([oracle.bf16_rne(float(a)) for a in np.ravel(v)], np.uint16).reshape(np.shape(v))


def test_e4m3_decode_matches_torch():
    ours = np.array([oracle.e4m3(c) for c in ALL_CODES])
    ref = torch_e4m3(ALL_CODES)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert oracle.e4m3(0x7E) == 448.0 and oracle.e4m3(0x01) == 2.0 ** -9 and oracle.e4m3(0x08) == 2.0 ** -6


def blocks_with_amax(amax_bits, fill_bits):
    """Blocks of 32 whose element 0 is amax_bits and the rest come from fill_bits (|fill| <= amax)."""
    fill = np.asarray(fill_bits, np.uint16)
    n = (fill.size + 30) // 31
    fill = np.concatenate([fill, np.zeros(n * 31 - fill.size, np.uint16)])
    blocks = np.empty((n, 32), np.uint16)
    blocks[:, 0] = amax_bits
    blocks[:, 1:] = fill.reshape(n, 31)
    return blocks


@pytest.mark.parametrize("amax_exp", [-131, -127, -119, -118, -8, 0, 7, 100, 127])
@pytest.mark.parametrize("mant", [1.75, 2 - 2.0 ** -7])
def test_quantize_rounds_like_torch_over_all_bf16(amax_exp, mant):
    """Every finite bf16 value v with |v| <= amax (amax = mant * 2^amax_exp, subnormal when
    amax_exp < -126) is rounded like torch's E4M3 cast of v / scale, and the scale is the
    closed form 2^(floor(log2 amax) - 8), clamped to the E8M0 range.  With mant near 2 the
    largest values divided by the scale pass 448 and saturate."""
    amax = mant * 2.0 ** amax_exp
    ab = int(f_to_bf16_bits(amax))
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = bf16_to_f(allb).astype(np.float64)
    fill = allb[np.isfinite(vals) & (np.abs(vals) <= bf16_to_f([ab])[0])]
    blocks = blocks_with_amax(ab, fill)
    codes, scales = oracle.mxfp8_quantize(blocks, blocks.shape[0], 32)
    amax_v = float(bf16_to_f([ab])[0])
    want = min(max(math.floor(math.log2(amax_v)) - 8 + 127, 0), 254)
    assert np.all(scales == want)
    v = bf16_to_f(blocks).astype(np.float64) / 2.0 ** (want - 127)
    inrange = np.abs(v) < 448
    ref = torch_cast_e4m3(np.where(inrange, v, 0.0))
    assert np.array_equal(codes[inrange], ref[inrange])
    sat = ~inrange
    assert np.array_equal(codes[sat], np.where(np.signbit(v[sat]), 0xFE, 0x7E).astype(np.uint8))


def test_quantize_picks_a_nearest_value_by_enumeration():
    """Each code is a nearest E4M3 magnitude to |x| / scale (ties to the even code),
    found by scanning all 127 magnitudes; values past 448 saturate."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 64)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    x[:, 5] *= 1e-4
    xb = f_to_bf16_bits(x)
    codes, scales = oracle.mxfp8_quantize(xb, 64, 64)
    mags = np.array([oracle.e4m3(c) for c in range(0x7F)])
    xv = bf16_to_f(xb).astype(np.float64)
    for r in range(64):
        for k in range(64):
            a = abs(xv[r, k]) / 2.0 ** (int(scales[r, k // 32]) - 127)
            d = np.abs(mags - min(a, 448.0))
            best = np.flatnonzero(d == d.min())
            c = int(best[0]) if best.size == 1 else int([b for b in best if b % 2 == 0][0])
            assert codes[r, k] & 0x7F == c, (r, k, a)
            assert (codes[r, k] >> 7) == (1 if np.signbit(xv[r, k]) else 0)


def test_quantize_invariants():
    rng = np.random.default_rng(4)
    xb = f_to_bf16_bits(rng.standard_normal((16, 96)))
    c0, s0 = oracle.mxfp8_quantize(xb, 16, 96)
    # negation flips the sign bit only
    c1, s1 = oracle.mxfp8_quantize(xb ^ np.uint16(0x8000), 16, 96)
    assert np.array_equal(c1, c0 ^ np.uint8(0x80)) and np.array_equal(s1, s0)
    # doubling (exact in bf16 here) raises every scale by one and keeps the codes
    x2 = f_to_bf16_bits(bf16_to_f(xb).astype(np.float64) * 2)
    c2, s2 = oracle.mxfp8_quantize(x2, 16, 96)
    assert np.array_equal(c2, c0) and np.array_equal(s2, s0 + 1)
    # a block of one power of two: scale 2^(p - 8), code 0x78 (= 256)
    for p in (-100, -3, 0, 5, 120):
        b = np.zeros((1, 32), np.uint16)
        b[0, 7] = f_to_bf16_bits(2.0 ** p)
        c, s = oracle.mxfp8_quantize(b, 1, 32)
        assert int(s[0, 0]) == p - 8 + 127 and c[0, 7] == 0x78 and np.all(np.delete(c[0], 7) == 0)
    # zero block, non-finite blocks
    z = np.zeros((3, 32), np.uint16)
    z[1, 3] = 0x7FC0  # NaN
    z[2, 9] = 0xFF80  # -Inf
    c, s = oracle.mxfp8_quantize(z, 3, 32)
    assert s[0, 0] == 0 and np.all(c[0] == 0)
    assert np.all(s[1:, 0] == 0xFF) and np.all(c[1:] == 0x7F)


def quantize_torch(xb):
    """Independent MXFP8 quantization of bf16 rows (K % 32 == 0) with the closed-form scale
    and torch's E4M3 cast plus saturation: exact fp64 values of the quantized activations."""
    xv = bf16_to_f(xb).astype(np.float64)
    rows, K = xv.shape
    out = np.empty_like(xv)
    for r in range(rows):
        for b in range(K // 32):
            blk = xv[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            s = 0 if amax == 0 else min(max(math.floor(math.log2(amax)) - 8 + 127, 0), 254)
            v = np.clip(blk / 2.0 ** (s - 127), -448, 448)
            out[r, 32 * b:32 * b + 32] = torch_e4m3(torch_cast_e4m3(v)) * 2.0 ** (s - 127)
    return out


def test_a8_linear_one_hot_extracts_weight_column():
    rng = np.random.default_rng(5)
    N, K = 24, 96
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = rng.integers(110, 135, (N, K // 32), dtype=np.uint8)
    W = oracle.dequant(w, s, N, K)
    for kk in (0, 31, 32, 77, 95):
        x = np.zeros((1, K), np.uint16)
        x[0, kk] = 0x3F80  # 1.0
        y, acc, _ = oracle.mx_linear_a8(x, w, s, 1, K, N)
        assert np.array_equal(acc[0].astype(np.float64), W[:, kk])


def test_a8_linear_equals_bf16_linear_on_mxfp8_exact_activations():
    """Activations that are already MXFP8 values (E4M3 codes times their block's scale,
    with the scale the quantizer would pick) pass through unchanged: the a8 layer equals
    the pinned bf16 layer bit for bit."""
    rng = np.random.default_rng(6)
    T, K, N = 5, 256, 40
    codes = rng.integers(0, 0x7F, (T, K)).astype(np.uint8) | (rng.integers(0, 2, (T, K)) << 7).astype(np.uint8)
    codes[:, ::32] = 0x7E  # each block's largest value is 448 * scale, so the quantizer picks that scale
    sc = rng.integers(100, 130, (T, K // 32))
    xv = torch_e4m3(codes) * np.repeat(2.0 ** (sc - 127), 32, axis=1)
    xb = f_to_bf16_bits(xv)
    assert np.array_equal(bf16_to_f(xb).astype(np.float64), xv)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = rng.integers(115, 130, (N, K // 32), dtype=np.uint8)
    ya, aa, sa = oracle.mx_linear_a8(xb, w, s, T, K, N)
    yb, ab, sb = oracle.mx_linear(xb, w, s, T, K, N)
    assert np.array_equal(ya, yb) and np.array_equal(aa, ab) and np.array_equal(sa, sb)


def test_a8_linear_is_the_bf16_linear_of_the_quantized_activations():
    rng = np.random.default_rng(7)
    T, K, N = 4, 512, 48
    xb = f_to_bf16_bits(rng.standard_normal((T, K)))
    q = quantize_torch(xb)
    qb = f_to_bf16_bits(q)
    assert np.array_equal(bf16_to_f(qb).astype(np.float64), q)  # normal range: exact in bf16
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = rng.integers(115, 130, (N, K // 32), dtype=np.uint8)
    ya, aa, _ = oracle.mx_linear_a8(xb, w, s, T, K, N)
    yb, ab, _ = oracle.mx_linear(qb, w, s, T, K, N)
    assert np.array_equal(ya, yb) and np.array_equal(aa, ab)


@pytest.mark.parametrize("seed", [0, 1])
def test_a8_linear_brute_force_exact_sums(seed, mags):
    rng = np.random.default_rng(10 + seed)
    T, K, N = 3, 96, 8
    xb = f_to_bf16_bits(rng.standard_normal((T, K)) * np.exp2(rng.integers(-3, 4, (T, K))))
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = rng.integers(118, 132, (N, K // 32), dtype=np.uint8)
    y, acc, sd = oracle.mx_linear_a8(xb, w, s, T, K, N)
    q = quantize_torch(xb)
    W = decode_py(w, s, mags)
    for t in range(T):
        for n in range(N):
            exact = sum(Fraction(q[t, k]) * Fraction(W[n, k]) for k in range(K))
            absum = sum(abs(Fraction(q[t, k]) * Fraction(W[n, k])) for k in range(K))
            assert abs(Fraction(float(acc[t, n])) - exact) <= (K - 1) * U32 * absum
            yo = float(bf16_to_f([y[t, n]])[0])
            assert abs(Fraction(yo) - exact) <= (K - 1) * U32 * absum + Fraction(ulp_bf16(yo)) / 2
            assert sd[t, n] == pytest.approx(float(absum), rel=1e-12)


@pytest.fixture(scope="module")
def mags(golden_dir):
    import json
    import os
    with open(os.path.join(golden_dir, "mxfp4_format.json")) as f:
        return json.load(f)["magnitudes"]


def test_a8_moe_single_expert_reduces_to_a8_linear():
    cfg = tiny_cfg(15, T=3, H=128, I=64, E=1, k=1, e_lo=-8, e_hi=-3)
    inp = synthetic.moe_inputs_host(cfg)
    y, sm, h = oracle.moe_tokens(inp["x"], inp["logits"], 1, inp["wgu"], inp["sgu"], inp["wd"], inp["sd"],
                                 3, 128, 64, 1, want_h=True, act8=True)
    _, acc, _ = oracle.mx_linear_a8(inp["x"], inp["wgu"][0], inp["sgu"][0], 3, 128, 128)
    g, u = acc[:, :64].astype(np.float64), acc[:, 64:].astype(np.float64)
    hv = g / (1 + np.exp(-g)) * u
    h_ref = np.array([[oracle.bf16_rne(v) for v in row] for row in hv], np.uint16)
    assert np.array_equal(h, h_ref)
    y_ref, _, sd = oracle.mx_linear_a8(h, inp["wd"][0], inp["sd"][0], 3, 64, 128)
    assert np.array_equal(y, y_ref)  # gate = 1 exactly when k = 1
    assert np.array_equal(sm, sd)


@pytest.mark.parametrize("seed", [0, 1])
def test_a8_moe_brute_force_tiny(seed, mags):
    """Exact sums over the torch-quantized x and the torch-quantized bf16 h the oracle
    returns: h within half a bf16 ulp plus the propagated fp32 error, y within the fp32
    accumulation bound."""
    cfg = tiny_cfg(20 + seed)
    inp = synthetic.moe_inputs_host(cfg)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    y, sm, h = oracle.moe_tokens(inp["x"], inp["logits"], k, inp["wgu"], inp["sgu"], inp["wd"], inp["sd"],
                                 T, H, I, E, want_h=True, act8=True)
    xq = quantize_torch(inp["x"].reshape(T, H))
    hq = quantize_torch(h.reshape(T * k, I))
    for t in range(T):
        lg = [float(v) for v in inp["logits"][t]]
        sel = sorted(range(E), key=lambda e: (-lg[e], e))[:k]
        ex = [math.exp(lg[e] - lg[sel[0]]) for e in sel]
        gates = [v / sum(ex) for v in ex]
        y_ref = [Fraction(0)] * H
        y_abs = [Fraction(0)] * H
        for j, e in enumerate(sel):
            Wg = decode_py(inp["wgu"][e], inp["sgu"][e], mags)
            Wd = decode_py(inp["wd"][e], inp["sd"][e], mags)
            p = t * k + j
            for n in range(I):
                g = sum(Fraction(xq[t, i]) * Fraction(Wg[n, i]) for i in range(H))
                u = sum(Fraction(xq[t, i]) * Fraction(Wg[I + n, i]) for i in range(H))
                ga = sum(abs(Fraction(xq[t, i]) * Fraction(Wg[n, i])) for i in range(H))
                ua = sum(abs(Fraction(xq[t, i]) * Fraction(Wg[I + n, i])) for i in range(H))
                gf, uf = float(g), float(u)
                hv = gf / (1 + math.exp(-gf)) * uf
                dg, du = H * U32 * float(ga), H * U32 * float(ua)
                sil = abs(gf / (1 + math.exp(-gf)))
                bound = 0.5 * ulp_bf16(hv) + 1.1 * dg * (abs(uf) + du) + (sil + 1.1 * dg) * du + 1e-300
                ho = float(bf16_to_f([h[p, n]])[0])
                assert abs(ho - hv) <= bound * (1 + 1e-9), (t, j, n, ho, hv)
            gj = Fraction(float(np.float32(gates[j])))
            for n in range(H):
                y_ref[n] += gj * sum(Fraction(hq[p, i]) * Fraction(Wd[n, i]) for i in range(I))
                y_abs[n] += gj * sum(abs(Fraction(hq[p, i]) * Fraction(Wd[n, i])) for i in range(I))
        for n in range(H):
            yo = float(bf16_to_f([y[t, n]])[0])
            bound = (I + k) * U32 * y_abs[n] + Fraction(ulp_bf16(yo)) / 2
            assert abs(Fraction(yo) - y_ref[n]) <= bound, (t, n, yo, float(y_ref[n]))
            assert sm[t, n] == pytest.approx(float(y_abs[n]), rel=2e-7)
