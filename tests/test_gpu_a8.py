"""GPU parity of the MXFP8-activation path (the AMD megakernel blog, "Bringing Ultra-Fast,
Interactive LLM Inference to AMD Instinct MI355X GPUs", section "3. Low-Precision Data Types")
against the oracle, through the C ABI.

The quantizer is bit-exact.  The GEMMs run on the scaled MFMA, which sums each group of 8
products dropping the bits more than about 14 binades below the group's largest product;
the dense bound is therefore |gpu - oracle| <= 2^-10 * sum_k |q(x) w| + ulp_bf16 (7 * 2^-14
from the instruction, the rest for fp32 accumulation on both sides).  The MoE layer keeps
the bf16 path's bound (1e-2 of sum_j gate_j sum_i |q(h)_i w_ni|).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_helpers import MOE_REL, bf16_to_f, check_bound, random_linear_shapes, say, to_dev_bf16, to_host_bits

pytestmark = pytest.mark.gpu

A8_DENSE_REL = 2.0 ** -10


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import mxfp4_weight_moe_amd  # noqa: F401  (fails loudly if the HIP library is missing)
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def mx(dev):
    import mxfp4_weight_moe_amd
    return mxfp4_weight_moe_amd


def f_to_bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).bfloat16().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ quantizer

def quant_blocks():
    """Blocks over every finite bf16 value, with largest values 1.75 and 1.99 times 2^e (the
    latter saturating), plus zero, NaN and Inf blocks and random rows."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = bf16_to_f(allb).astype(np.float64)
    rows = []
    for e in (-131, -127, -119, -118, -8, 0, 7, 100, 127):
        for mant in (1.75, 2 - 2.0 ** -7):
            ab = int(f_to_bf16_bits([mant * 2.0 ** e])[0])
            fill = allb[np.isfinite(vals) & (np.abs(vals) <= bf16_to_f([ab])[0])]
            n = (fill.size + 30) // 31
            fill = np.concatenate([fill, np.zeros(n * 31 - fill.size, np.uint16)])
            b = np.empty((n, 32), np.uint16)
            b[:, 0] = ab
            b[:, 1:] = fill.reshape(n, 31)
            rows.append(b)
    special = np.zeros((4, 32), np.uint16)
    special[1, 3] = 0x7FC0   # NaN
    special[2, 9] = 0xFF80   # -Inf
    special[3, :] = 0x8000   # -0
    rows.append(special)
    x = np.concatenate(rows)
    pad = (-x.shape[0]) % 8
    x = np.concatenate([x, np.zeros((pad, 32), np.uint16)]).reshape(-1, 256)
    rng = np.random.default_rng(9)
    extra = f_to_bf16_bits(rng.standard_normal((37, 256)) * np.exp2(rng.integers(-30, 30, (37, 1))))
    return np.concatenate([x, extra])


def test_mxfp8_quantize_bit_exact(dev, mx):
    x = quant_blocks()
    say("mxfp8 quantize", x.shape)
    codes, scales = mx.mxfp8_quantize(to_dev_bf16(x, dev))
    torch.cuda.synchronize()
    oc, os_ = oracle.mxfp8_quantize(x, x.shape[0], x.shape[1])
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


# ------------------------------------------------------------------ dense layer

def run_linear_a8(dev, mx, x, w, s):
    y = mx.mx_linear(to_dev_bf16(x, dev), torch.from_numpy(w).to(dev), torch.from_numpy(s).to(dev), act8=True)
    torch.cuda.synchronize()
    return to_host_bits(y)


@pytest.mark.parametrize("name", ["dense_t1", "dense_t4"])
def test_mx_linear_a8_configs(dev, mx, name):
    cfg = synthetic.LINEAR_CONFIGS[name]
    x, w, s = synthetic.linear_inputs(cfg)
    say("mx_linear_a8", name, cfg)
    got = run_linear_a8(dev, mx, x, w, s)
    y, _, sd = oracle.mx_linear_a8(x, w, s, cfg.T, cfg.K, cfg.N)
    worst = check_bound(got, y, sd, A8_DENSE_REL, name)
    say(f"  worst ratio {worst:.3g}")


ODD = [(1, 32, 16), (3, 64, 17), (2, 96, 40), (5, 288, 33), (16, 256, 16), (17, 512, 48), (31, 1024, 64),
       (32, 800, 80), (33, 256, 32), (64, 2048, 128), (7, 7168, 100), (4, 7200, 64), (9, 2048, 48), (2, 16384, 24)]


@pytest.mark.parametrize("T,K,N", ODD)
def test_mx_linear_a8_odd_shapes(dev, mx, T, K, N):
    cfg = synthetic.LinearConfig("odd", T=T, K=K, N=N, e_lo=-6, e_hi=2, seed=T * 11 + K + N)
    x, w, s = synthetic.linear_inputs(cfg)
    say("mx_linear_a8 odd", T, K, N)
    got = run_linear_a8(dev, mx, x, w, s)
    y, _, sd = oracle.mx_linear_a8(x, w, s, T, K, N)
    check_bound(got, y, sd, A8_DENSE_REL, f"a8 odd {T},{K},{N}")


RANDOM_LINEAR = random_linear_shapes(seed=20261205)


@pytest.mark.parametrize("T,K,N", RANDOM_LINEAR)
def test_mx_linear_a8_random_shapes(dev, mx, T, K, N):
    cfg = synthetic.LinearConfig("random", T=T, K=K, N=N, e_lo=-6, e_hi=2, seed=T * 3 + K + N)
    x, w, s = synthetic.linear_inputs(cfg)
    say("mx_linear_a8 random", T, K, N)
    got = run_linear_a8(dev, mx, x, w, s)
    y, _, sd = oracle.mx_linear_a8(x, w, s, T, K, N)
    check_bound(got, y, sd, A8_DENSE_REL, f"a8 random {T},{K},{N}")


def test_mx_linear_a8_sparse_and_one_hot(dev, mx):
    """Rows with one or a few nonzeros per block make every code and scale count: a wrong
    code moves an output by an E4M3 step, far past the bound.  A one-hot row extracts the
    weight column exactly."""
    T, K, N = 6, 512, 64
    cfg = synthetic.LinearConfig("sparse", T=T, K=K, N=N, e_lo=-6, e_hi=0, seed=21)
    x, w, s = synthetic.linear_inputs(cfg)
    x = x.copy()
    rng = np.random.default_rng(22)
    keep = np.zeros((T, K), bool)
    for t in range(T):
        for b in range(K // 32):
            keep[t, 32 * b + rng.choice(32, size=1 + t % 3, replace=False)] = True
    x[~keep] = 0
    x[0, :] = 0
    x[0, 77] = 0x3F80  # 1.0
    say("mx_linear_a8 sparse")
    got = run_linear_a8(dev, mx, x, w, s)
    y, _, sd = oracle.mx_linear_a8(x, w, s, T, K, N)
    check_bound(got, y, sd, A8_DENSE_REL, "a8 sparse")
    assert np.array_equal(got[0], y[0])


# ------------------------------------------------------------------ MoE layer

def moe_inputs(cfg, dev, host=None):
    if host is not None:
        d = {k: torch.from_numpy(v).to(dev) for k, v in host.items() if k in ("wgu", "sgu", "wd", "sd")}
        x, logits = host["x"], host["logits"]
    else:
        d = synthetic.moe_weights_device(cfg, dev)
        x, logits = synthetic.moe_activations(cfg)
    d["x"] = to_dev_bf16(x, dev)
    d["logits"] = torch.from_numpy(logits).to(dev)
    return d, x, logits


def run_moe_a8(mx, d, k, n_shared=0):
    y = mx.moe_mxfp4_forward(d["x"], d["logits"], k, d["wgu"], d["sgu"], d["wd"], d["sd"], n_shared=n_shared,
                             act8=True)
    torch.cuda.synchronize()
    return to_host_bits(y)


def oracle_moe_a8(cfg, x, logits, w, tokens=None):
    y, sm, _ = oracle.moe_tokens(x, logits, cfg.k, w["wgu"], w["sgu"], w["wd"], w["sd"], cfg.T, cfg.H, cfg.I, cfg.E,
                                 tokens=tokens, n_shared=cfg.n_shared, act8=True)
    return y, sm


TINY = [
    dict(T=1, H=1024, I=1024, E=4, k=1),
    dict(T=5, H=2048, I=1024, E=8, k=3),
    dict(T=17, H=1024, I=2048, E=4, k=2),   # two row groups
    dict(T=40, H=1024, I=1024, E=4, k=4),   # three row groups
    dict(T=9, H=1024, I=256, E=3, k=2),     # one-segment down reductions
    dict(T=20, H=2048, I=768, E=6, k=3),
    dict(T=4, H=1024, I=1024, E=6, k=2, n_shared=1),
    # both expert GEMMs in one launch: the workgroup's own sort (T = 8, 32), and the sort
    # launches' result (a shared expert at T = 24)
    dict(T=8, H=1024, I=2048, E=64, k=8),
    dict(T=32, H=1024, I=1024, E=128, k=8),
    dict(T=24, H=1024, I=1024, E=128, k=6, n_shared=1),
]


@pytest.mark.parametrize("shape", TINY, ids=[f"T{s['T']}_H{s['H']}_I{s['I']}_E{s['E']}_k{s['k']}"
                                             f"_ns{s.get('n_shared', 0)}" for s in TINY])
def test_moe_a8_tiny(dev, mx, shape):
    cfg = synthetic.MoEConfig("tiny_a8", routing="normal", e_lo=-8, e_hi=-2, seed=shape["T"] * 3 + shape["I"], **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("moe a8 tiny", shape)
    d, x, logits = moe_inputs(cfg, dev, host)
    got = run_moe_a8(mx, d, cfg.k, cfg.n_shared)
    y, sm = oracle_moe_a8(cfg, x, logits, host)
    worst = check_bound(got, y, sm, MOE_REL, f"a8 tiny {shape}")
    say(f"  worst ratio {worst:.3g}")
    assert np.array_equal(run_moe_a8(mx, d, cfg.k, cfg.n_shared), got)  # deterministic


# moe_sweep_t1: in-gate_up routing with the combine inside down; moe_sweep_t2: half-width down
FULL = [("moe_t4", None), ("moe_t32_zipf", [0, 7, 31]), ("moe_t128", [0, 100]), ("moe_tp8_t32", [0, 3, 30]),
        ("moe_shared_t1", None), ("moe_shared_t32", [0, 9, 31]), ("moe_sweep_t1", None), ("moe_sweep_t2", None)]


@pytest.mark.parametrize("name,tokens", FULL, ids=[f[0] for f in FULL])
def test_moe_a8_full_size(dev, mx, name, tokens):
    cfg = (synthetic.MOE_CONFIGS[name] if name in synthetic.MOE_CONFIGS
           else synthetic.sweep_config(int(name[len("moe_sweep_t"):])))
    say("moe a8 full", name, "tokens", tokens)
    d, x, logits = moe_inputs(cfg, dev)
    got = run_moe_a8(mx, d, cfg.k, cfg.n_shared)
    w = {k: d[k].cpu().numpy() for k in ("wgu", "sgu", "wd", "sd")}
    tok = np.arange(cfg.T, dtype=np.int32) if tokens is None else np.array(tokens, np.int32)
    y, sm = oracle_moe_a8(cfg, x, logits, w, tokens=tok)
    worst = check_bound(got[tok], y, sm, MOE_REL, name)
    say(f"  worst ratio {worst:.3g}")


@pytest.mark.parametrize("T,E,k", [(2, 16, 4), (20, 16, 4), (24, 128, 8)])
def test_moe_a8_graph_replays(dev, mx, T, E, k):
    """The MXFP8 forward captured in a HIP graph (at T = 2 its down launch also combines; at
    T = 24 over 128 experts both expert GEMMs run in one launch): every replay, with eager
    work and synchronizations between replays, gives the eager result bit for bit, and the
    workspace control words end zero."""
    cfg = synthetic.MoEConfig("graph_a8", T=T, H=1024, I=1024, E=E, k=k, routing="normal", e_lo=-8, e_hi=-2,
                              seed=40 + T)
    host = synthetic.moe_inputs_host(cfg)
    say("a8 forward graph replays, T =", T)
    d, x, logits = moe_inputs(cfg, dev, host)
    ws = mx.workspace(T, cfg.H, cfg.I, cfg.E, cfg.k, dev)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    fwd = lambda: mx.moe_mxfp4_forward(d["x"], d["logits"], cfg.k, d["wgu"], d["sgu"], d["wd"], d["sd"], out=out,
                                       ws=ws, act8=True)
    fwd()
    torch.cuda.synchronize()
    ref = to_host_bits(out)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fwd()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(out), ref), f"replay {r}"
        fwd()
        torch.cuda.synchronize()
    assert not ws[:57344].any().item()
    y, sm = oracle_moe_a8(cfg, x, logits, host)
    check_bound(ref, y, sm, MOE_REL, f"a8 graph T={T}")
