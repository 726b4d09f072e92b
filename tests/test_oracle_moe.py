"""Pins of the oracle's MoE layer: reduction to the dense layer, identical-expert
invariance, and a separately written fp64 brute force on tiny shapes."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic

U32 = 2.0 ** -24


def bf16_to_f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def ulp_bf16(v: float) -> float:
    a = abs(v)
    if a < 2.0 ** -126:
        return 2.0 ** -133
    return 2.0 ** (math.floor(math.log2(a)) - 7)


@pytest.fixture(scope="module")
def mags(golden_dir):
    with open(os.path.join(golden_dir, "mxfp4_format.json")) as f:
        return json.load(f)["magnitudes"]


def decode_py(w, s, mags):
    rows, kb = w.shape
    K = kb * 2
    codes = np.empty((rows, K), np.int64)
    codes[:, 0::2] = w & 15
    codes[:, 1::2] = w >> 4
    table = np.array(mags + [-m for m in mags], np.float64)
    return table[codes] * np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)


def tiny_cfg(seed, T=3, H=64, I=32, E=4, k=2, e_lo=-6, e_hi=-2, routing="normal"):
    return synthetic.MoEConfig("tiny", T=T, H=H, I=I, E=E, k=k, routing=routing, e_lo=e_lo, e_hi=e_hi, seed=seed)


def run_oracle(inp, cfg, want_h=False):
    return oracle.moe_tokens(inp["x"], inp["logits"], cfg.k, inp["wgu"], inp["sgu"], inp["wd"], inp["sd"],
                             cfg.T, cfg.H, cfg.I, cfg.E, want_h=want_h)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny_moe(seed, mags):
    cfg = tiny_cfg(seed)
    inp = synthetic.moe_inputs_host(cfg)
    y, sm, h = run_oracle(inp, cfg, want_h=True)
    x = bf16_to_f(inp["x"]).astype(np.float64)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    for t in range(T):
        lg = [float(v) for v in inp["logits"][t]]
        sel = sorted(range(E), key=lambda e: (-lg[e], e))[:k]
        ex = [math.exp(lg[e] - lg[sel[0]]) for e in sel]
        gates = [v / sum(ex) for v in ex]
        assert abs(sum(float(np.float32(g)) for g in gates) - 1) < 1e-6
        y_ref = [Fraction(0)] * H   # exact sum_j gate_j * d_j[n], from the oracle's own h
        y_abs = [Fraction(0)] * H   # sum_j gate_j * sum_i |h_i w_ni|
        for j, e in enumerate(sel):
            Wg = decode_py(inp["wgu"][e], inp["sgu"][e], mags)
            Wd = decode_py(inp["wd"][e], inp["sd"][e], mags)
            p = t * k + j
            # gate_up + SwiGLU: within half a bf16 ulp plus the propagated fp32 error of g and u
            for n in range(I):
                g = sum(Fraction(x[t, i]) * Fraction(Wg[n, i]) for i in range(H))
                u = sum(Fraction(x[t, i]) * Fraction(Wg[I + n, i]) for i in range(H))
                ga = sum(abs(Fraction(x[t, i]) * Fraction(Wg[n, i])) for i in range(H))
                ua = sum(abs(Fraction(x[t, i]) * Fraction(Wg[I + n, i])) for i in range(H))
                gf, uf = float(g), float(u)
                hv = gf / (1 + math.exp(-gf)) * uf
                dg, du = H * U32 * float(ga), H * U32 * float(ua)
                sil = abs(gf / (1 + math.exp(-gf)))
                bound = 0.5 * ulp_bf16(hv) + 1.1 * dg * (abs(uf) + du) + (sil + 1.1 * dg) * du + 1e-300
                ho = float(bf16_to_f([h[p, n]])[0])
                assert abs(ho - hv) <= bound * (1 + 1e-9), (t, j, n, ho, hv)
            # down projection, weighted by the fp32 gate
            hv = bf16_to_f(h[p]).astype(np.float64)
            gj = Fraction(float(np.float32(gates[j])))
            for n in range(H):
                y_ref[n] += gj * sum(Fraction(hv[i]) * Fraction(Wd[n, i]) for i in range(I))
                y_abs[n] += gj * sum(abs(Fraction(hv[i]) * Fraction(Wd[n, i])) for i in range(I))
        for n in range(H):
            yo = float(bf16_to_f([y[t, n]])[0])
            bound = (I + k) * U32 * y_abs[n] + Fraction(ulp_bf16(yo)) / 2
            assert abs(Fraction(yo) - y_ref[n]) <= bound, (t, n, yo, float(y_ref[n]))
            assert sm[t, n] == pytest.approx(float(y_abs[n]), rel=2e-7)


def test_single_expert_reduces_to_dense_mlp():
    cfg = tiny_cfg(5, T=3, H=128, I=64, E=1, k=1, e_lo=-8, e_hi=-3)
    inp = synthetic.moe_inputs_host(cfg)
    y, sm, h = run_oracle(inp, cfg, want_h=True)
    _, acc, _ = oracle.mx_linear(inp["x"], inp["wgu"][0], inp["sgu"][0], 3, 128, 128)
    g, u = acc[:, :64].astype(np.float64), acc[:, 64:].astype(np.float64)
    hv = g / (1 + np.exp(-g)) * u
    h_ref = np.array([[oracle.bf16_rne(v) for v in row] for row in hv], np.uint16)
    assert np.array_equal(h, h_ref)
    y_ref, _, _ = oracle.mx_linear(h, inp["wd"][0], inp["sd"][0], 3, 64, 128)
    assert np.array_equal(y, y_ref)  # gate = 1 exactly when k = 1


def test_gate_up_terms_are_the_dense_layer_dot_products():
    """The gate_up terms the oracle reports (g, u before SwiGLU and their sums of |x w|)
    are, slot by slot, the pinned dense layer's fp32 dot products and bound terms over the
    routed expert's gate and up rows, and the h it returns with them is moe_tokens' h."""
    cfg = tiny_cfg(7, T=4, H=128, I=64, E=5, k=2, e_lo=-8, e_hi=-3)
    inp = synthetic.moe_inputs_host(cfg)
    args = (inp["x"], inp["logits"], cfg.k, inp["wgu"], inp["sgu"], inp["wd"], inp["sd"], cfg.T, cfg.H, cfg.I, cfg.E)
    y, sm, h, terms = oracle.moe_gate_up_terms(*args)
    y2, sm2, h2 = oracle.moe_tokens(*args, want_h=True)
    assert np.array_equal(y, y2) and np.array_equal(sm, sm2) and np.array_equal(h, h2)
    ids, _ = oracle.route(inp["logits"], cfg.k)
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = ids[t, j]
            _, acc, sd = oracle.mx_linear(inp["x"][t:t + 1], inp["wgu"][e], inp["sgu"][e], 1, cfg.H, 2 * cfg.I)
            r = t * cfg.k + j
            assert np.array_equal(terms["g"][r], acc[0, :cfg.I]) and np.array_equal(terms["u"][r], acc[0, cfg.I:])
            assert np.array_equal(terms["gabs"][r], sd[0, :cfg.I]) and np.array_equal(terms["uabs"][r], sd[0, cfg.I:])


def shared_cfg(seed, n_shared, E=3, k=2):
    return synthetic.MoEConfig("tiny_shared", T=3, H=128, I=64, E=E, k=k, routing="normal", e_lo=-8, e_hi=-3,
                               seed=seed, n_shared=n_shared)


def dense_mlp_acc(x, wgu, sgu, wd, sd, T, H, I):
    """The shared expert as a dense MLP from two mx_linear calls: (fp32 down outputs, h)."""
    _, acc, _ = oracle.mx_linear(x, wgu, sgu, T, H, 2 * I)
    g, u = acc[:, :I].astype(np.float64), acc[:, I:].astype(np.float64)
    hv = g / (1 + np.exp(-g)) * u
    h = np.array([[oracle.bf16_rne(v) for v in row] for row in hv], np.uint16)
    _, dacc, _ = oracle.mx_linear(h, wd, sd, T, I, H)
    return dacc, h


@pytest.mark.parametrize("n_shared", [1, 2])
def test_shared_experts_add_to_the_routed_ones(n_shared):
    """With every routed expert's codes zero (its outputs are +0), the layer is the shared
    experts' sum: one shared expert gives the dense MLP bit for bit, two identical ones
    give exactly twice its fp32 down outputs before the bf16 rounding."""
    cfg = shared_cfg(11, n_shared)
    inp = synthetic.moe_inputs_host(cfg)
    E = cfg.E
    inp["wgu"][:E] = 0
    inp["wd"][:E] = 0
    for key in ("wgu", "sgu", "wd", "sd"):
        inp[key][E + 1:] = inp[key][E]  # identical shared experts
    y, _, h = oracle.moe_tokens(inp["x"], inp["logits"], cfg.k, inp["wgu"], inp["sgu"], inp["wd"], inp["sd"],
                                cfg.T, cfg.H, cfg.I, E, want_h=True, n_shared=n_shared)
    dacc, h_ref = dense_mlp_acc(inp["x"], inp["wgu"][E], inp["sgu"][E], inp["wd"][E], inp["sd"][E], cfg.T, cfg.H,
                                cfg.I)
    kk = cfg.k + n_shared
    for s in range(n_shared):
        assert np.array_equal(h.reshape(cfg.T, kk, cfg.I)[:, cfg.k + s], h_ref)
    y_ref = np.array([[oracle.bf16_rne(n_shared * float(v)) for v in row] for row in dacc], np.uint16)
    assert np.array_equal(y, y_ref)


def test_shared_expert_slots_follow_the_routed_ones():
    """Routed experts unchanged, one shared expert added: the routed slots' h rows are
    the same as without the shared expert."""
    cfg = shared_cfg(12, 1, E=5, k=2)
    inp = synthetic.moe_inputs_host(cfg)
    _, _, h1 = oracle.moe_tokens(inp["x"], inp["logits"], cfg.k, inp["wgu"], inp["sgu"], inp["wd"], inp["sd"],
                                 cfg.T, cfg.H, cfg.I, cfg.E, want_h=True, n_shared=1)
    routed = {k_: np.ascontiguousarray(v[:cfg.E]) for k_, v in inp.items() if k_ in ("wgu", "sgu", "wd", "sd")}
    _, _, h0 = oracle.moe_tokens(inp["x"], inp["logits"], cfg.k, routed["wgu"], routed["sgu"], routed["wd"],
                                 routed["sd"], cfg.T, cfg.H, cfg.I, cfg.E, want_h=True)
    assert np.array_equal(h1.reshape(cfg.T, 3, cfg.I)[:, :2], h0.reshape(cfg.T, 2, cfg.I))


def test_identical_experts_make_routing_irrelevant():
    cfg = tiny_cfg(6, T=4, H=64, I=32, E=6, k=3)
    inp = synthetic.moe_inputs_host(cfg)
    for key in ("wgu", "sgu", "wd", "sd"):
        inp[key] = np.ascontiguousarray(np.broadcast_to(inp[key][:1], inp[key].shape))
    y1, sm1, _ = run_oracle(inp, cfg)
    inp2 = dict(inp)
    inp2["logits"] = np.ascontiguousarray(inp["logits"][:, ::-1] * np.float32(3.0))
    y2, _, _ = run_oracle(inp2, cfg)
    single = tiny_cfg(6, T=4, H=64, I=32, E=1, k=1)
    inp1 = {k_: (v[:1] if k_ in ("wgu", "sgu", "wd", "sd") else v) for k_, v in inp.items()}
    inp1["logits"] = np.zeros((4, 1), np.float32)
    y0, _, _ = run_oracle(inp1, single)
    for yy in (y1, y2):
        a, b = bf16_to_f(yy).astype(np.float64), bf16_to_f(y0).astype(np.float64)
        tol = np.array([[ulp_bf16(max(abs(p), abs(q))) for p, q in zip(ra, rb)] for ra, rb in zip(a, b)])
        assert np.all(np.abs(a - b) <= tol + 4 * U32 * sm1)


def test_nan_scale_in_inactive_expert_is_never_read():
    cfg = tiny_cfg(7, T=2, H=64, I=32, E=8, k=2)
    inp = synthetic.moe_inputs_host(cfg)
    ids, _ = oracle.route(inp["logits"], 2)
    unused = sorted(set(range(8)) - set(ids.ravel().tolist()))
    assert unused
    y0, _, _ = run_oracle(inp, cfg)
    for key in ("sgu", "sd"):
        inp[key] = inp[key].copy()
        inp[key][unused] = 255
    y1, _, _ = run_oracle(inp, cfg)
    assert np.array_equal(y0, y1)
