"""GPU parity: every stage of the HIP path against the CPU oracle on the same seeded inputs.

All calls go through the C ABI of libmxmoe.so (via the thin Python binding).  Sizes run
from tiny edge cases through several tiles with ragged tails to the full workload shapes
(sampled tokens where the oracle would take too long).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_helpers import (DENSE_REL, MOE_REL, bf16_to_f, check_bound, random_linear_shapes, say,
                               to_dev_bf16, to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import mxfp4_weight_moe_amd  # noqa: F401  (fails loudly if the HIP library is missing)
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def mx(dev):
    import mxfp4_weight_moe_amd
    return mxfp4_weight_moe_amd


# ------------------------------------------------------------------ decode

def expected_decode_bits(w, s, rows, K):
    v = oracle.dequant(w, s, rows, K)  # exact fp64
    return torch.from_numpy(v).float().bfloat16().view(torch.int16).numpy().view(np.uint16)


def test_dequant_all_codes_all_scales(dev, mx):
    K = 512
    w = np.tile(np.arange(256, dtype=np.uint8), (256, 1))   # row r: every byte value
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 32, axis=1)  # row r: scale byte r
    say("dequant all codes x all scales", w.shape)
    out = mx.mxfp4_dequantize(torch.from_numpy(w).to(dev), torch.from_numpy(s).to(dev))
    got = to_host_bits(out)
    want = expected_decode_bits(w, s, 256, K)
    nan_rows = np.isnan(bf16_to_f(want))
    assert np.array_equal(np.isnan(bf16_to_f(got)), nan_rows)
    assert np.array_equal(got[~nan_rows], want[~nan_rows])


def test_dequant_random_large(dev, mx):
    cfg = synthetic.LINEAR_CONFIGS["dense_t4"]
    _, w, s = synthetic.linear_inputs(cfg)
    say("dequant", w.shape)
    out = mx.mxfp4_dequantize(torch.from_numpy(w).to(dev), torch.from_numpy(s).to(dev))
    assert np.array_equal(to_host_bits(out), expected_decode_bits(w, s, cfg.N, cfg.K))


# ------------------------------------------------------------------ dense linear

def run_linear(dev, mx, x, w, s, T, K, N):
    y = mx.mx_linear(to_dev_bf16(x, dev), torch.from_numpy(w).to(dev), torch.from_numpy(s).to(dev))
    torch.cuda.synchronize()
    return to_host_bits(y)


@pytest.mark.parametrize("name", ["dense_t1", "dense_t4"])
def test_mx_linear_configs(dev, mx, name):
    cfg = synthetic.LINEAR_CONFIGS[name]
    x, w, s = synthetic.linear_inputs(cfg)
    say("mx_linear", name, cfg)
    got = run_linear(dev, mx, x, w, s, cfg.T, cfg.K, cfg.N)
    y, _, sd = oracle.mx_linear(x, w, s, cfg.T, cfg.K, cfg.N)
    worst = check_bound(got, y, sd, DENSE_REL, name)
    say(f"  worst ratio {worst:.3g}")


ODD = [(1, 32, 16), (3, 64, 17), (2, 96, 40), (5, 288, 33), (16, 256, 16), (17, 512, 48), (31, 1024, 64),
       (32, 800, 80), (33, 256, 32), (64, 2048, 128), (100, 256, 20), (7, 7168, 100), (4, 7200, 64),
       (9, 2048, 48), (12, 2560, 33), (2, 16384, 24)]


@pytest.mark.parametrize("T,K,N", ODD)
def test_mx_linear_odd_shapes(dev, mx, T, K, N):
    cfg = synthetic.LinearConfig("odd", T=T, K=K, N=N, e_lo=-6, e_hi=2, seed=T * 7 + K + N)
    x, w, s = synthetic.linear_inputs(cfg)
    say("mx_linear odd", T, K, N)
    got = run_linear(dev, mx, x, w, s, T, K, N)
    y, _, sd = oracle.mx_linear(x, w, s, T, K, N)
    check_bound(got, y, sd, DENSE_REL, f"odd {T},{K},{N}")


RANDOM_LINEAR = random_linear_shapes()


@pytest.mark.parametrize("T,K,N", RANDOM_LINEAR)
def test_mx_linear_random_shapes(dev, mx, T, K, N):
    cfg = synthetic.LinearConfig("random", T=T, K=K, N=N, e_lo=-6, e_hi=2, seed=T * 5 + K + N)
    x, w, s = synthetic.linear_inputs(cfg)
    say("mx_linear random", T, K, N)
    got = run_linear(dev, mx, x, w, s, T, K, N)
    y, _, sd = oracle.mx_linear(x, w, s, T, K, N)
    check_bound(got, y, sd, DENSE_REL, f"random {T},{K},{N}")


def test_mx_linear_edge_values(dev, mx):
    # subnormal-producing and overflowing scales, NaN scale, zero and one-hot activations
    T, K, N = 3, 256, 32
    cfg = synthetic.LinearConfig("edge", T=T, K=K, N=N, e_lo=-6, e_hi=0, seed=5)
    x, w, s = synthetic.linear_inputs(cfg)
    s = s.copy()
    s[3, :] = 255       # NaN scales: whole output column NaN
    s[4, 2] = 255       # one NaN block
    s[5, :] = 250       # large weights, finite products
    s[6, :] = 30        # tiny weights (~2^-97), normal in fp32
    x = x.copy()
    x[1, :] = 0         # zero row -> +0 outputs (except NaN columns)
    x[2, :] = 0
    x[2, 7] = 0x3F80    # one-hot row -> extracts weight column 7
    say("mx_linear edge values")
    got = run_linear(dev, mx, x, w, s, T, K, N)
    y, _, sd = oracle.mx_linear(x, w, s, T, K, N)
    check_bound(got, y, sd, DENSE_REL, "edge")
    fin = ~np.isnan(bf16_to_f(y[2]))
    assert np.array_equal(got[2][fin], y[2][fin])


@pytest.mark.parametrize("T,K", [(1, 2048), (2, 2048), (1, 7200), (2, 96)])
def test_mx_linear_edge_values_one_and_two_tokens(dev, mx, T, K):
    """The one-row-per-wave path of one and two tokens: NaN scales (a whole output column,
    one block), huge and tiny scales, and (T = 2) a one-hot row that must extract the weight
    column exactly (nibble order, scale index); K = 7200 and 96 leave ragged blocks per lane."""
    N = 48
    cfg = synthetic.LinearConfig("edge12", T=T, K=K, N=N, e_lo=-6, e_hi=0, seed=K + T)
    x, w, s = synthetic.linear_inputs(cfg)
    s = s.copy()
    s[3, :] = 255
    s[4, min(2, K // 32 - 1)] = 255
    s[5, :] = 235  # huge weights (6 * 2^108) whose sums stay finite: |x| < 4, K <= 7200 terms
    s[6, :] = 30
    x = x.copy()
    if T == 2:
        x[1, :] = 0
        x[1, 7] = 0x3F80
    say("mx_linear edge values, T =", T, "K =", K)
    got = run_linear(dev, mx, x, w, s, T, K, N)
    y, _, sd = oracle.mx_linear(x, w, s, T, K, N)
    check_bound(got, y, sd, DENSE_REL, f"edge T={T} K={K}")
    if T == 2:
        fin = ~np.isnan(bf16_to_f(y[1]))
        assert np.array_equal(got[1][fin], y[1][fin])


# ------------------------------------------------------------------ routing and sort

ROUTE_CASES = [("moe_t4", None), ("moe_t32_zipf", None), ("moe_t128", None)]


def route_logits(name):
    return synthetic.router_logits(synthetic.MOE_CONFIGS[name])


@pytest.mark.parametrize("name", ["moe_t4", "moe_t32_zipf", "moe_t128"])
def test_route_matches_oracle(dev, mx, name):
    cfg = synthetic.MOE_CONFIGS[name]
    logits = synthetic.router_logits(cfg)
    say("route", name, logits.shape)
    ids, gates = mx.moe_route_topk(torch.from_numpy(logits).to(dev), cfg.k)
    oids, ogates = oracle.route(logits, cfg.k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(gates.cpu().numpy().astype(np.float64) - ogates)) <= 1e-6


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 7, 7), (5, 64, 3), (17, 1024, 32), (256, 256, 8), (2, 65, 4)])
def test_route_edge_shapes_and_ties(dev, mx, T, E, k):
    rng = np.random.default_rng(T + E + k)
    logits = np.round(rng.standard_normal((T, E)), 1).astype(np.float32)  # many exact ties
    logits[0, :] = 0.0                                                    # all tied
    say("route ties", T, E, k)
    ids, gates = mx.moe_route_topk(torch.from_numpy(logits).to(dev), k)
    oids, ogates = oracle.route(logits, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(gates.cpu().numpy().astype(np.float64) - ogates)) <= 1e-6


def check_sort(r, o):
    """The library's sort against the oracle's: counts, offsets and sorted slots bit-exact;
    the active list a permutation of the oracle's active set (ascending there) in the order
    the library documents for its expert GEMMs (row class descending: 8 or more rows, 4-7,
    2-3, 1; expert id ascending within a class), -1 after it; num_active = {the number of
    active experts, the largest count}, the second computed here from the counts."""
    for key in ("counts", "offsets", "sorted_slots"):
        assert np.array_equal(r[key].cpu().numpy(), o[key]), key
    counts, na = o["counts"], o["num_active"]
    assert r["num_active"].cpu().tolist() == [na, int(counts.max())]
    act = r["active"].cpu().numpy()
    lib = act[:na]
    assert np.array_equal(np.sort(lib), o["active"][:na]), "active list is not a permutation of the active set"
    assert np.all(act[na:] == -1)
    cls = np.digitize(counts[lib], [2, 4, 8])
    assert np.array_equal(lib, lib[np.lexsort((lib, -cls))]), "active list not in row-class order"


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (4, 256, 8), (32, 256, 8), (128, 384, 8), (256, 1024, 32),
                                   (3, 4, 4), (9, 7, 2), (256, 8, 1)])
def test_sort_matches_oracle(dev, mx, T, E, k):
    rng = np.random.default_rng(T * 3 + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    say("sort", T, E, k)
    r = mx.moe_sort_by_expert(torch.from_numpy(ids).to(dev), E)
    check_sort(r, oracle.sort(ids, E))


# T <= 16 runs as one launch, larger T as the route and sort kernels: both paths, every
# logits-per-lane class (E <= 256, <= 512, <= 1024) of the single launch
ROUTE_SORT_CASES = [("moe_t4", 0), ("moe_t32_zipf", 0), ("moe_t128", 0), ("ties", 1), ("ties", 2), ("ties", 3),
                    ("ties", 4), ("ties", 5)]


@pytest.mark.parametrize("name,variant", ROUTE_SORT_CASES, ids=[f"{n}{v}" for n, v in ROUTE_SORT_CASES])
def test_route_sort_matches_oracle(dev, mx, name, variant):
    """The fused route + sort launch of the layer forward, bit-exact against the oracle's route then sort."""
    if name != "ties":
        cfg = synthetic.MOE_CONFIGS[name]
        logits, k = synthetic.router_logits(cfg), cfg.k
    else:
        T, E, k = [(5, 64, 3), (256, 1024, 32), (40, 300, 8), (16, 1024, 32), (16, 300, 8)][variant - 1]
        rng = np.random.default_rng(variant)
        logits = np.round(rng.standard_normal((T, E)), 1).astype(np.float32)  # many exact ties
        logits[0, :] = 0.0
        logits[-1, ::2] = -0.0
    say("route+sort", name, variant, logits.shape, k)
    ids, gates, srt = mx.moe_route_sort(torch.from_numpy(logits).to(dev), k)
    oids, ogates = oracle.route(logits, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(gates.cpu().numpy().astype(np.float64) - ogates)) <= 1e-6
    check_sort(srt, oracle.sort(oids, logits.shape[1]))


# ------------------------------------------------------------------ MoE layer

def moe_device_inputs(cfg, dev, host=None):
    """Inputs for a config: tiny configs drawn on the host, large ones on the device."""
    if host is not None:
        d = {k: torch.from_numpy(v).to(dev) for k, v in host.items() if k in ("wgu", "sgu", "wd", "sd")}
        x, logits = host["x"], host["logits"]
    else:
        d = synthetic.moe_weights_device(cfg, dev)
        x, logits = synthetic.moe_activations(cfg)
    d["x"] = to_dev_bf16(x, dev)
    d["logits"] = torch.from_numpy(logits).to(dev)
    return d, x, logits


CTL_BYTES = 57344  # MX_WORKSPACE_CTL_BYTES


def poisoned_workspace(mx, T, H, I, E, k, dev):
    """A fresh workspace: control words zero (as the ABI requires), every other byte 0xFF,
    so that any h, d or sort entry a kernel fails to write reads as NaN (or -1)."""
    ws = torch.zeros(mx.workspace_size(T, H, I, E, k), dtype=torch.uint8, device=dev)
    ws[CTL_BYTES:] = 0xFF
    return ws


def nan_like_out(shape, dev):
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)


def run_moe(mx, d, k, n_shared=0, act8=False):
    """The layer forward on a NaN-poisoned workspace into a NaN-filled y."""
    T, H = d["x"].shape
    E = d["logits"].shape[1]
    I = d["wd"].shape[2] * 2
    dev = d["x"].device
    ws = poisoned_workspace(mx, T, H, I, E + n_shared, k + n_shared, dev)
    y = mx.moe_mxfp4_forward(d["x"], d["logits"], k, d["wgu"], d["sgu"], d["wd"], d["sd"], n_shared=n_shared,
                             act8=act8, out=nan_like_out((T, H), dev), ws=ws)
    torch.cuda.synchronize()
    assert not ws[:CTL_BYTES].any().item(), "control words not left zero"
    return to_host_bits(y)


def oracle_moe(cfg, x, logits, w_host, tokens=None):
    y, sm, _ = oracle.moe_tokens(x, logits, cfg.k, w_host["wgu"], w_host["sgu"], w_host["wd"], w_host["sd"],
                                 cfg.T, cfg.H, cfg.I, cfg.E, tokens=tokens, n_shared=cfg.n_shared)
    return y, sm


TINY = [
    dict(T=1, H=1024, I=1024, E=4, k=1),
    dict(T=3, H=1024, I=1024, E=4, k=2),
    dict(T=5, H=2048, I=1024, E=8, k=3),
    dict(T=17, H=1024, I=2048, E=4, k=2),   # 17 rows on some experts: two row groups
    dict(T=40, H=1024, I=1024, E=4, k=4),   # every expert has 40 rows: three row groups
    dict(T=64, H=3072, I=1024, E=16, k=8),
    dict(T=2, H=1024, I=1024, E=300, k=8),  # most experts inactive
    dict(T=33, H=1024, I=3072, E=2, k=1),   # 33 rows on one expert
    dict(T=9, H=1024, I=1024, E=1, k=1),    # one expert, 9 rows: chunk of 4 segments
]


@pytest.mark.parametrize("shape", TINY, ids=[f"T{s['T']}_H{s['H']}_I{s['I']}_E{s['E']}_k{s['k']}" for s in TINY])
def test_moe_tiny_full_oracle(dev, mx, shape):
    cfg = synthetic.MoEConfig("tiny", routing="normal", e_lo=-8, e_hi=-2, seed=shape["T"] + shape["E"], **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("moe tiny", shape)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    got = run_moe(mx, d, cfg.k)
    y, sm = oracle_moe(cfg, x, logits, host)
    worst = check_bound(got, y, sm, MOE_REL, f"tiny {shape}")
    say(f"  worst ratio {worst:.3g}")


# the sweep points cover the launch shapes of the smallest T: T = 1 (gate_up that routes in
# every workgroup, down with the combine inside), T = 2 and 3 (half-width down because
# full-width items would need between one and two rounds of the slots), T = 16 (the largest
# in-gate_up routing)
FULL = [("moe_t4", None), ("moe_t32_zipf", None), ("moe_t128", list(range(0, 128, 8))),
        ("moe_spec_t4", None), ("moe_spec_t128", [0, 1, 2, 3, 40, 41, 126, 127]),
        ("moe_tp8_t4", None), ("moe_tp8_t32", None), ("moe_shared_t1", None), ("moe_shared_t32", [0, 9, 31]),
        ("moe_sweep_t1", None), ("moe_sweep_t2", None), ("moe_sweep_t3", None), ("moe_sweep_t16", None)]


def full_config(name):
    if name in synthetic.MOE_CONFIGS:
        return synthetic.MOE_CONFIGS[name]
    return synthetic.sweep_config(int(name[len("moe_sweep_t"):]))


@pytest.mark.parametrize("name,tokens", FULL, ids=[f[0] for f in FULL])
def test_moe_full_size(dev, mx, name, tokens):
    cfg = full_config(name)
    say("moe full", name, "tokens", tokens)
    d, x, logits = moe_device_inputs(cfg, dev)
    got = run_moe(mx, d, cfg.k, cfg.n_shared)
    w_host = {k: d[k].cpu().numpy() for k in ("wgu", "sgu", "wd", "sd")}
    tok = np.arange(cfg.T, dtype=np.int32) if tokens is None else np.array(tokens, np.int32)
    y, sm = oracle_moe(cfg, x, logits, w_host, tokens=tok)
    worst = check_bound(got[tok], y, sm, MOE_REL, name)
    say(f"  worst ratio {worst:.3g}")


@pytest.mark.parametrize("T,E,k,hot", [(256, 8, 1, [3]), (256, 2, 2, [0, 1]), (200, 64, 4, [5, 6, 7, 60]),
                                        (256, 512, 8, [0, 1, 2, 3, 4, 5, 6, 7])],
                         ids=["T256_one_expert", "T256_two_experts_k2", "T200_four_hot", "T256_E512_eight_hot"])
def test_moe_all_tokens_on_few_experts(dev, mx, T, E, k, hot):
    """Routing skewed to the extreme: every token picks the same experts, so each of them has
    T rows (up to 16 row groups) and almost every work item is an extra row group."""
    cfg = synthetic.MoEConfig("skew", T=T, H=1024, I=1024, E=E, k=k, routing="normal", e_lo=-8, e_hi=-2,
                              seed=T + E + k)
    host = synthetic.moe_inputs_host(cfg)
    logits = host["logits"].copy()
    logits[:, hot] += 40.0  # the hot experts win every token's top-k
    host["logits"] = logits
    say("moe skewed routing", T, E, k, hot)
    d, x, logits = moe_device_inputs(cfg, dev, host=host)
    got = run_moe(mx, d, cfg.k)
    y, sm = oracle_moe(cfg, x, logits, host)
    worst = check_bound(got, y, sm, MOE_REL, f"skewed {T},{E},{k}")
    say(f"  worst ratio {worst:.3g}")
    assert np.array_equal(run_moe(mx, d, cfg.k), got)  # deterministic


def random_moe_cases(n=16, seed=20261203):
    """Seeded random layer shapes over the ranges the launchers choose between: T from 1 to
    256, 1 to 1024 experts, top-1 to top-32, H and I over several multiples of 1024 and
    256, and three routing distributions (host weights kept under ~400 MB)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        H = int(rng.choice([1024, 2048, 3072]))
        I = int(rng.choice([256, 512, 768, 1024, 2048]))
        E = int(rng.choice([1, 3, 8, 16, 64, 200, 256, 384, 1024]))
        k = int(min(E, rng.choice([1, 2, 4, 6, 8, 16, 32])))
        T = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 17, 24, 32, 33, 64, 100, 128, 200, 256]))
        routing = str(rng.choice(["normal", "uniform", "zipf"]))
        if E * 1.6 * H * I > 4e8:
            continue
        cases.append(dict(T=T, H=H, I=I, E=E, k=k, routing=routing, seed=len(cases)))
    return cases


RANDOM_MOE = random_moe_cases()


@pytest.mark.parametrize("shape", RANDOM_MOE,
                         ids=[f"T{c['T']}_H{c['H']}_I{c['I']}_E{c['E']}_k{c['k']}_{c['routing']}" for c in RANDOM_MOE])
def test_moe_random_shapes(dev, mx, shape):
    cfg = synthetic.MoEConfig("random", e_lo=-8, e_hi=-2, **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("moe random shape", shape)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    got = run_moe(mx, d, cfg.k)
    T = cfg.T
    tok = None
    if T * cfg.k * cfg.H * cfg.I * 3 > 3e9:  # sampled tokens where the whole layer would be slow
        tok = np.unique(np.array([0, T // 3, T // 2, T - 1], np.int32))
    y, sm = oracle_moe(cfg, x, logits, host) if tok is None else \
        oracle.moe_tokens(x, logits, cfg.k, host["wgu"], host["sgu"], host["wd"], host["sd"], T, cfg.H, cfg.I, cfg.E,
                          tokens=tok)[:2]
    worst = check_bound(got if tok is None else got[tok], y, sm, MOE_REL, f"random {shape}")
    say(f"  worst ratio {worst:.3g}")


def expert_gemm_hooks_match(mx, d, cfg, y_fwd, dev):
    """The forward's launches as stage calls (moe_route_topk, moe_expert_gemms_from_ids on a
    poisoned workspace, moe_combine) give the forward's y bit for bit, and the launch's h
    equals moe_gate_up_swiglu's h bit for bit."""
    ids, gates = mx.moe_route_topk(d["logits"], cfg.k)
    ws = poisoned_workspace(mx, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dev)
    dd = torch.full((cfg.T * cfg.k, cfg.H), float("nan"), dtype=torch.float32, device=dev)
    h1, dd = mx.moe_expert_gemms_from_ids(d["x"], ids, d["wgu"], d["sgu"], d["wd"], d["sd"], d=dd, ws=ws)
    y1 = mx.moe_combine(dd, gates, out=nan_like_out((cfg.T, cfg.H), dev))
    _, _, srt = mx.moe_route_sort(d["logits"], cfg.k)
    h2 = mx.moe_gate_up_swiglu(d["x"], d["wgu"], d["sgu"], srt, cfg.k)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(y1), y_fwd)
    assert np.array_equal(to_host_bits(h1), to_host_bits(h2))
    assert int(ws[:CTL_BYTES].count_nonzero()) == 0


# Both expert GEMMs in one launch (moe_expert_gemms_from_ids), which the forward runs up to
# 32 tokens once min(T k, E) I / 64 >= 1536.  Shapes below that bound exercise the stage entry
# point against the forward's separate launches: E = 32 with I = 1024 gives one gate_up item
# per workgroup, so many down items start before their expert's h is complete and take the
# wait-and-reload path.  Zipf routing gives experts with two row groups; T = 6 and 12 sit on
# the bound; E = 200 and 256 give many light experts; top-16 at T = 32 (512 slots, more than
# the workgroup's own sort holds) takes the launch from the sort launches' result.
SINGLE_EXPERT_LAUNCH = [dict(T=32, H=1024, I=1024, E=32, k=8, routing="normal"),
                        dict(T=32, H=1024, I=1024, E=64, k=8, routing="zipf"),
                        dict(T=17, H=2048, I=1024, E=256, k=8, routing="normal"),
                        dict(T=24, H=1024, I=2048, E=32, k=6, routing="uniform"),
                        dict(T=32, H=1024, I=1024, E=200, k=8, routing="zipf"),
                        dict(T=6, H=1024, I=2048, E=128, k=8, routing="normal"),
                        dict(T=12, H=2048, I=1024, E=256, k=8, routing="zipf"),
                        dict(T=32, H=1024, I=1024, E=128, k=16, routing="normal")]


@pytest.mark.parametrize("shape", SINGLE_EXPERT_LAUNCH,
                         ids=[f"T{s['T']}_H{s['H']}_I{s['I']}_E{s['E']}_k{s['k']}_{s['routing']}"
                              for s in SINGLE_EXPERT_LAUNCH])
def test_moe_single_expert_launch(dev, mx, shape):
    """The forward against the oracle (every token), bit-identical to the separate stage
    launches and to the single expert launch's stage calls, and again twice in a row on one
    workspace (every path leaves its control words zero)."""
    cfg = synthetic.MoEConfig("one_launch", e_lo=-8, e_hi=-2, seed=shape["T"] * 3 + shape["E"], **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("moe single expert launch", shape)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    got = run_moe(mx, d, cfg.k)
    y, sm = oracle_moe(cfg, x, logits, host)
    worst = check_bound(got, y, sm, MOE_REL, f"single expert launch {shape}")
    say(f"  worst ratio {worst:.3g}")
    assert np.array_equal(run_hooks(mx, d, cfg.k, cfg.T), got)
    if cfg.T * cfg.k <= 256:  # the stage entry point sorts in every workgroup
        expert_gemm_hooks_match(mx, d, cfg, got, dev)
    ws = poisoned_workspace(mx, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dev)
    for _ in range(2):
        out = nan_like_out((cfg.T, cfg.H), dev)
        mx.moe_mxfp4_forward(d["x"], d["logits"], cfg.k, d["wgu"], d["sgu"], d["wd"], d["sd"], out=out, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(out), got)
    assert int(ws[:CTL_BYTES].count_nonzero()) == 0


def test_expert_gemm_hooks_full_size(dev, mx):
    """The single expert launch at T = 32, H = 7168, I = 2048, E = 256, top-8, Zipf routing
    (the launch configuration the benchmark times): the stage calls give the forward's y bit
    for bit, with h identical to the separate gate_up's."""
    cfg = synthetic.MOE_CONFIGS["moe_t32_zipf"]
    say("expert gemm hooks, full size", cfg.name)
    d, x, logits = moe_device_inputs(cfg, dev)
    expert_gemm_hooks_match(mx, d, cfg, run_moe(mx, d, cfg.k), dev)


def test_moe_small_scale_variant(dev, mx):
    cfg = synthetic.small_scale_variant(synthetic.MOE_CONFIGS["moe_t4"])
    say("moe small-scale variant")
    d, x, logits = moe_device_inputs(cfg, dev)
    got = run_moe(mx, d, cfg.k)
    w_host = {k: d[k].cpu().numpy() for k in ("wgu", "sgu", "wd", "sd")}
    y, sm = oracle_moe(cfg, x, logits, w_host)
    worst = check_bound(got, y, sm, MOE_REL, "small-scale")
    say(f"  worst ratio {worst:.3g}")


def test_moe_deterministic_and_inactive_experts_unread(dev, mx):
    """Two runs on separately NaN-poisoned workspaces give the same y, and NaN scales planted
    in every expert no token routes to change nothing."""
    cfg = synthetic.MoEConfig("det", T=8, H=1024, I=1024, E=32, k=4, routing="normal", e_lo=-8, e_hi=-2, seed=3)
    host = synthetic.moe_inputs_host(cfg)
    say("moe determinism / inactive NaN scales")
    d, x, logits = moe_device_inputs(cfg, dev, host)
    y1 = run_moe(mx, d, cfg.k)
    y2 = run_moe(mx, d, cfg.k)
    assert np.array_equal(y1, y2)
    ids, _ = oracle.route(logits, cfg.k)
    unused = sorted(set(range(cfg.E)) - set(ids.ravel().tolist()))
    assert unused
    for key in ("sgu", "sd"):
        d[key][unused] = 255
    y3 = run_moe(mx, d, cfg.k)
    assert np.array_equal(y1, y3)


# ------------------------------------------------------------------ gate_up's h against the oracle's h

H_REL = 1e-5  # the dense-output tolerance, applied to the fp32 dot products g and u


def bf16_round_f64(v):
    """Nearest bf16 (ties to even) of float64 values, as float64 (finite inputs)."""
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)  # 8 significant bits; np.round ties to even
    return np.where(v == 0, v, q)


def check_h(got_bits, ora_bits, terms, what):
    """gate_up's h against the oracle's, element by element.

    g and u are dense MXFP4 dot products: the GPU's may differ from the oracle's fp32 sums
    by the dense tolerance, H_REL * sum|x w| each.  With v = silu(g) u from the oracle's g
    and u, that allows |h_exact - v| <= dh = 1.1 dg (|u| + du) + (|silu g| + 1.1 dg) du
    plus 2^-20 |v| for the GPU's fp32 evaluation of silu (|silu'| <= 1.1).  The GPU's h
    must be the bf16 rounding of some value within dh of v.  Where dh cannot move v across
    a rounding boundary that means the oracle's h bit for bit, elsewhere one of the two
    neighbours (a flip).  Returns (flips, elements)."""
    go = bf16_to_f(got_bits).astype(np.float64)
    ho = bf16_to_f(ora_bits).astype(np.float64)
    g, u = terms["g"].astype(np.float64), terms["u"].astype(np.float64)
    fin = np.isfinite(g) & np.isfinite(u)
    assert np.array_equal(np.isnan(go[~fin]), np.isnan(ho[~fin])), f"{what}: NaN positions differ"
    assert np.array_equal(go[~fin & ~np.isnan(ho)], ho[~fin & ~np.isnan(ho)]), f"{what}: non-finite h differ"
    g, u, go, ho = g[fin], u[fin], go[fin], ho[fin]
    dg, du = H_REL * terms["gabs"][fin], H_REL * terms["uabs"][fin]
    silu = g / (1.0 + np.exp(-g))
    v = silu * u
    dh = 1.1 * dg * (np.abs(u) + du) + (np.abs(silu) + 1.1 * dg) * du + 2.0 ** -20 * np.abs(v)
    lo, hi = bf16_round_f64(v - dh), bf16_round_f64(v + dh)
    assert np.all(np.isfinite(go)), f"{what}: non-finite h where g and u are finite"
    bad = (go < lo) | (go > hi)
    if bad.any():
        i = np.nonzero(bad)[0][0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} h values outside the bound; first gpu={go[i]!r} "
                             f"oracle={ho[i]!r} v={v[i]!r} dh={dh[i]!r}")
    flips = int((go != ho).sum())
    one_value = lo == hi
    assert np.array_equal(go[one_value], ho[one_value])  # implied above; stated for the reader
    return flips, go.size, int((~one_value).sum())


def poisoned_sort(T, k, E, dev):
    """Sort output tensors filled with a value no entry point writes (every entry must be written)."""
    return {key: torch.full((n,), -7, dtype=torch.int32, device=dev)
            for key, n in (("counts", E), ("offsets", E + 1), ("sorted_slots", T * k), ("active", E),
                           ("num_active", 2))}


def gate_up_h_parity(mx, dev, cfg, d, x, logits, w_host, tokens=None, from_ids=False):
    """h from a gate_up stage entry point, on a NaN-poisoned workspace into a NaN-filled h,
    against the oracle's h of the listed tokens: moe_gate_up_swiglu after the route + sort
    entry point, or (from_ids) moe_gate_up_swiglu_from_ids after the route entry point, whose
    sort, written into poisoned tensors, must equal the oracle's."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    ws = poisoned_workspace(mx, T, H, I, E, k, dev)
    h = nan_like_out((T * k, I), dev)
    if from_ids:
        ids, gates = mx.moe_route_topk(d["logits"], k)
        _, srt = mx.moe_gate_up_swiglu_from_ids(d["x"], ids, d["wgu"], d["sgu"], h=h, sort=poisoned_sort(T, k, E, dev),
                                                ws=ws)
        torch.cuda.synchronize()
        check_sort(srt, oracle.sort(ids.cpu().numpy(), E))
    else:
        ids, gates, srt = mx.moe_route_sort(d["logits"], k)
        mx.moe_gate_up_swiglu(d["x"], d["wgu"], d["sgu"], srt, k, h=h, ws=ws)
    torch.cuda.synchronize()
    hg = to_host_bits(h)                        # row p: the slot at sorted position p
    slots = srt["sorted_slots"].cpu().numpy()
    pos = np.empty_like(slots)
    pos[slots] = np.arange(slots.size)          # sorted position of each flat slot
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    _, _, ho, terms = oracle.moe_gate_up_terms(x, logits, k, w_host["wgu"], w_host["sgu"], w_host["wd"],
                                               w_host["sd"], T, H, I, E, tokens=tok)
    flat = (tok[:, None] * k + np.arange(k)[None, :]).ravel()   # oracle row i*k + j is slot tok[i]*k + j
    return check_h(hg[pos[flat]], ho, terms, cfg.name)


H_TINY = [dict(T=1, H=1024, I=1024, E=4, k=1), dict(T=5, H=2048, I=1024, E=8, k=3),
          dict(T=40, H=1024, I=1024, E=4, k=4), dict(T=64, H=3072, I=1024, E=16, k=8),
          dict(T=20, H=2048, I=512, E=6, k=3), dict(T=2, H=1024, I=256, E=300, k=8)]


@pytest.mark.parametrize("shape", H_TINY, ids=[f"T{s['T']}_H{s['H']}_I{s['I']}_E{s['E']}_k{s['k']}" for s in H_TINY])
@pytest.mark.parametrize("scales", ["curved", "config"])
def test_gate_up_h_matches_oracle_tiny(dev, mx, shape, scales):
    """gate_up's h directly against the oracle's h: tiles of both widths, ragged and
    repeated row groups, I = 256 and 512; SiLU in its curved region (scales 2^-12..2^-6)
    and with the configs' scales."""
    e_lo, e_hi = (-12, -6) if scales == "curved" else (-6, 0)
    cfg = synthetic.MoEConfig("h_tiny", routing="normal", e_lo=e_lo, e_hi=e_hi, seed=shape["T"] * 5 + shape["E"],
                              **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("gate_up h, tiny", shape, scales)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    flips, n, wide = gate_up_h_parity(mx, dev, cfg, d, x, logits, host)
    say(f"  {flips} flips of {n} h values ({wide} within reach of a rounding boundary)")


@pytest.mark.parametrize("name,tokens", [("moe_t4", None), ("moe_t32_zipf", None), ("moe_t128", list(range(0, 128, 16)))],
                         ids=["moe_t4", "moe_t32_zipf", "moe_t128"])
def test_gate_up_h_matches_oracle_full_size(dev, mx, name, tokens):
    """The same at the full workload shapes, in the launch configuration the benchmark
    times (every routed row at T = 4 and T = 32, where the hot experts have two row groups;
    every slot of 8 tokens at T = 128)."""
    cfg = synthetic.MOE_CONFIGS[name]
    say("gate_up h, full size", name)
    d, x, logits = moe_device_inputs(cfg, dev)
    w_host = {key: d[key].cpu().numpy() for key in ("wgu", "sgu", "wd", "sd")}
    flips, n, wide = gate_up_h_parity(mx, dev, cfg, d, x, logits, w_host, tokens)
    say(f"  {flips} flips of {n} h values ({wide} within reach of a rounding boundary)")


# gate_up that sorts the slots itself (T <= 32, T k <= 256, E <= 1024): experts with two row
# groups (17 and 32 rows), I = 256 and 512, E = 1024 (four experts per thread in its count
# scan), a small T the entry point also accepts, and every expert routed by every token
FROM_IDS = [dict(T=17, H=1024, I=1024, E=4, k=4), dict(T=20, H=2048, I=512, E=6, k=3),
            dict(T=32, H=1024, I=256, E=300, k=8), dict(T=32, H=1024, I=1024, E=1024, k=8),
            dict(T=3, H=1024, I=1024, E=8, k=2), dict(T=32, H=3072, I=1024, E=2, k=2),
            dict(T=25, H=2048, I=1024, E=64, k=1)]


@pytest.mark.parametrize("shape", FROM_IDS, ids=[f"T{s['T']}_H{s['H']}_I{s['I']}_E{s['E']}_k{s['k']}" for s in FROM_IDS])
def test_gate_up_from_ids_matches_oracle(dev, mx, shape):
    """moe_gate_up_swiglu_from_ids: its sort bit-exact against the oracle's (active list in
    row-class order, -1 after it), its h against the oracle's h, and the same h bit for bit as
    moe_gate_up_swiglu after the route + sort entry point."""
    cfg = synthetic.MoEConfig("from_ids", routing="normal", e_lo=-8, e_hi=-2, seed=shape["T"] * 11 + shape["E"],
                              **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("gate_up from ids, tiny", shape)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    flips, n, wide = gate_up_h_parity(mx, dev, cfg, d, x, logits, host, from_ids=True)
    say(f"  {flips} flips of {n} h values ({wide} within reach of a rounding boundary)")
    ids, _, srt = mx.moe_route_sort(d["logits"], cfg.k)
    h_sep = mx.moe_gate_up_swiglu(d["x"], d["wgu"], d["sgu"], srt, cfg.k)
    h_ids, srt2 = mx.moe_gate_up_swiglu_from_ids(d["x"], ids, d["wgu"], d["sgu"])
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "sorted_slots", "active", "num_active"):
        assert torch.equal(srt[key], srt2[key]), key
    assert np.array_equal(to_host_bits(h_ids), to_host_bits(h_sep))


def test_gate_up_from_ids_full_size(dev, mx):
    """The same at T = 32, H = 7168, I = 2048, E = 256, top-8 with Zipf routing (the hot experts
    have two row groups), the launch the layer forward makes at that size: every routed row."""
    cfg = synthetic.MOE_CONFIGS["moe_t32_zipf"]
    say("gate_up from ids, full size", cfg.name)
    d, x, logits = moe_device_inputs(cfg, dev)
    w_host = {key: d[key].cpu().numpy() for key in ("wgu", "sgu", "wd", "sd")}
    flips, n, wide = gate_up_h_parity(mx, dev, cfg, d, x, logits, w_host, from_ids=True)
    say(f"  {flips} flips of {n} h values ({wide} within reach of a rounding boundary)")


# ------------------------------------------------------------------ NaN and Inf through active experts

@pytest.mark.parametrize("act8", [False, True], ids=["bf16", "mxfp8"])
def test_moe_nan_scale_in_active_expert(dev, mx, act8):
    """A NaN scale (0xFF) in one gate row block of a routed expert makes every output of
    the tokens routed to it NaN (through h and the down sum); one in a down row block makes
    that output column NaN for its tokens.  NaN positions must match the oracle's exactly,
    every other output stays within the bound."""
    cfg = synthetic.MoEConfig("nan_active", T=6, H=1024, I=1024, E=8, k=2, routing="normal", e_lo=-8, e_hi=-2,
                              seed=21)
    host = synthetic.moe_inputs_host(cfg)
    ids, _ = oracle.route(host["logits"], cfg.k)
    e1 = int(ids[0, 0])
    e2 = next(int(e) for e in ids.ravel() if e != e1)
    host["sgu"][e1, 5, 3] = 255
    host["sd"][e2, 100, 0] = 255
    say("moe NaN scale in active experts", e1, e2, "act8", act8)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    got = run_moe(mx, d, cfg.k, act8=act8)
    y, sm, _ = oracle.moe_tokens(x, logits, cfg.k, host["wgu"], host["sgu"], host["wd"], host["sd"], cfg.T, cfg.H,
                                 cfg.I, cfg.E, act8=act8)
    nan = np.isnan(bf16_to_f(y))
    assert nan[0].all() and not nan.all()
    check_bound(got, y, sm, MOE_REL, "NaN scale")


@pytest.mark.parametrize("act8", [False, True], ids=["bf16", "mxfp8"])
def test_moe_nan_and_inf_activation_rows(dev, mx, act8):
    """A NaN, a +Inf and a -Inf activation in three tokens' rows: their outputs become
    non-finite exactly where the oracle's do, the other tokens' outputs are unaffected."""
    cfg = synthetic.MoEConfig("nan_x", T=7, H=1024, I=1024, E=8, k=2, routing="normal", e_lo=-8, e_hi=-2, seed=22)
    host = synthetic.moe_inputs_host(cfg)
    host["x"] = host["x"].copy()
    host["x"][1, 17] = 0x7FC0   # NaN
    host["x"][4, 300] = 0x7F80  # +Inf
    host["x"][5, 3] = 0xFF80    # -Inf
    say("moe NaN / Inf activation rows, act8", act8)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    got = run_moe(mx, d, cfg.k, act8=act8)
    y, sm, _ = oracle.moe_tokens(x, logits, cfg.k, host["wgu"], host["sgu"], host["wd"], host["sd"], cfg.T, cfg.H,
                                 cfg.I, cfg.E, act8=act8)
    fin = np.isfinite(bf16_to_f(y))
    assert not fin[[1, 4, 5]].any() and fin[[0, 2, 3, 6]].all()
    check_bound(got, y, sm, MOE_REL, "NaN/Inf x")


def test_forward_with_tied_logits(dev, mx):
    """The layer forward routes in its own fused kernel: exact ties (lower expert id wins)
    and +0/-0 pairs must route as the oracle routes them."""
    cfg = synthetic.MoEConfig("ties", T=6, H=1024, I=1024, E=16, k=4, routing="normal", e_lo=-8, e_hi=-2, seed=11)
    host = synthetic.moe_inputs_host(cfg)
    rng = np.random.default_rng(5)
    logits = np.round(rng.standard_normal((cfg.T, cfg.E)), 0).astype(np.float32)  # values in a few integers
    logits[0, :] = 0.0                    # every expert tied
    logits[1, ::2] = -0.0                 # -0 ties +0
    logits[1, 1::2] = 0.0
    host["logits"] = logits
    say("moe forward, tied logits")
    d, x, lg = moe_device_inputs(cfg, dev, host)
    got = run_moe(mx, d, cfg.k)
    y, sm = oracle_moe(cfg, x, lg, host)
    worst = check_bound(got, y, sm, MOE_REL, "tied logits")
    say(f"  worst ratio {worst:.3g}")


def test_forward_maximum_sizes(dev, mx):
    """T = 256 tokens, E = 1024 experts, top-32: the largest routing the library accepts."""
    cfg = synthetic.MoEConfig("max", T=256, H=1024, I=1024, E=1024, k=32, routing="normal", e_lo=-8, e_hi=-2, seed=2)
    say("moe forward, T=256 E=1024 k=32")
    d, x, logits = moe_device_inputs(cfg, dev)
    got = run_moe(mx, d, cfg.k)
    w_host = {k: d[k].cpu().numpy() for k in ("wgu", "sgu", "wd", "sd")}
    tok = np.array([0, 1, 100, 254, 255], np.int32)
    y, sm = oracle_moe(cfg, x, logits, w_host, tokens=tok)
    worst = check_bound(got[tok], y, sm, MOE_REL, "maximum sizes")
    say(f"  worst ratio {worst:.3g}")


@pytest.mark.parametrize("shape", [dict(T=3, H=1024, I=1024, E=8, k=2), dict(T=20, H=2048, I=1024, E=16, k=4)],
                         ids=["T3", "T20"])
def test_stage_hooks_match_forward(dev, mx, shape):
    """The stage entry points (route_sort, gate_up_swiglu, down_combine) called one after another give
    the forward's y bit for bit, and both match the oracle."""
    cfg = synthetic.MoEConfig("hooks", routing="normal", e_lo=-8, e_hi=-2, seed=shape["T"] * 7, **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("stage hooks vs forward", shape)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    y_fwd = run_moe(mx, d, cfg.k)
    ids, gates, srt = mx.moe_route_sort(d["logits"], cfg.k)
    h = mx.moe_gate_up_swiglu(d["x"], d["wgu"], d["sgu"], srt, cfg.k)
    y = mx.moe_down_combine(h, gates, d["wd"], d["sd"], srt, cfg.T, cfg.k)
    torch.cuda.synchronize()
    y_hooks = to_host_bits(y)
    assert np.array_equal(y_hooks, y_fwd)
    yo, sm = oracle_moe(cfg, x, logits, host)
    worst = check_bound(y_hooks, yo, sm, MOE_REL, f"hooks {shape}")
    say(f"  worst ratio {worst:.3g}")


# ------------------------------------------------------------------ single-launch layer (T <= 16)


def run_hooks(mx, d, k, T):
    """The layer as the stage entry points compute it (separate launches)."""
    ids, gates, srt = mx.moe_route_sort(d["logits"], k)
    h = mx.moe_gate_up_swiglu(d["x"], d["wgu"], d["sgu"], srt, k)
    y = mx.moe_down_combine(h, gates, d["wd"], d["sd"], srt, T, k)
    torch.cuda.synchronize()
    return to_host_bits(y)


# the third-to-last case runs both expert GEMMs in one launch from the sort launches' result
SHARED = [dict(T=1, H=1024, I=1024, E=4, k=1, n_shared=1), dict(T=5, H=1024, I=1024, E=8, k=2, n_shared=2),
          dict(T=24, H=1024, I=1024, E=128, k=6, n_shared=1),
          dict(T=20, H=2048, I=1024, E=6, k=3, n_shared=1), dict(T=40, H=1024, I=256, E=4, k=2, n_shared=1)]


@pytest.mark.parametrize("shape", SHARED, ids=[f"T{s['T']}_E{s['E']}_k{s['k']}_ns{s['n_shared']}" for s in SHARED])
def test_moe_shared_experts(dev, mx, shape):
    """Shared experts after the routed ones (every token reads them, gate 1), against the
    oracle; at T = 40 the shared expert has three row groups."""
    cfg = synthetic.MoEConfig("shared", routing="normal", e_lo=-8, e_hi=-2, seed=shape["T"] * 17 + shape["E"], **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("moe shared experts", shape)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    got = run_moe(mx, d, cfg.k, cfg.n_shared)
    yo, sm = oracle_moe(cfg, x, logits, host)
    worst = check_bound(got, yo, sm, MOE_REL, f"shared {shape}")
    say(f"  worst ratio {worst:.3g}")
    assert np.array_equal(run_moe(mx, d, cfg.k, cfg.n_shared), got)  # deterministic


# down reductions that are not multiples of 1024 (one-segment scale runs): I = 256, 512, 768.
# The last shape has enough items (5 row-group levels x 64 experts x 8 wide quads, at least
# 4 per resident workgroup) for down's wide tiles, and experts with more than 16 rows.
NARROW = [dict(T=5, H=1024, I=256, E=8, k=2), dict(T=20, H=2048, I=512, E=6, k=3), dict(T=3, H=1024, I=768, E=4, k=4),
          dict(T=40, H=1024, I=256, E=4, k=2), dict(T=80, H=2048, I=256, E=64, k=8)]


@pytest.mark.parametrize("shape", NARROW, ids=[f"T{s['T']}_H{s['H']}_I{s['I']}_E{s['E']}_k{s['k']}" for s in NARROW])
def test_moe_narrow_intermediate(dev, mx, shape):
    """Intermediate widths that are multiples of 256 but not of 1024, as one tensor-parallel
    share of an expert: the oracle bound, bit-identical stage entry points, and the single
    launch refusing them."""
    cfg = synthetic.MoEConfig("narrow", routing="normal", e_lo=-8, e_hi=-2, seed=shape["T"] * 13 + shape["I"], **shape)
    host = synthetic.moe_inputs_host(cfg)
    say("moe narrow intermediate", shape)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    got = run_moe(mx, d, cfg.k)
    yo, sm = oracle_moe(cfg, x, logits, host)
    worst = check_bound(got, yo, sm, MOE_REL, f"narrow {shape}")
    say(f"  worst ratio {worst:.3g}")
    assert np.array_equal(run_hooks(mx, d, cfg.k, cfg.T), got)
    if cfg.T <= 16:
        with pytest.raises(ValueError):
            mx.moe_mxfp4_forward(d["x"], d["logits"], cfg.k, d["wgu"], d["sgu"], d["wd"], d["sd"], persistent=True)


FUSED_EDGES = [
    dict(T=16, H=1024, I=1024, E=64, k=8),     # 128 slots: the largest single-launch step
    dict(T=4, H=1024, I=1024, E=1024, k=32),   # 1024 experts (16 logits per lane), top-32
    dict(T=16, H=1024, I=1024, E=512, k=8),    # 8 logits per lane, mostly one row per expert
    dict(T=1, H=1024, I=1024, E=1, k=1),       # one expert, one row
    dict(T=13, H=3072, I=1024, E=3, k=2),      # 13 rows on some experts
    dict(T=16, H=1024, I=2048, E=2, k=1),      # 16 rows, a full row group, on some expert
]


@pytest.mark.parametrize("shape", FUSED_EDGES, ids=[f"T{s['T']}_H{s['H']}_I{s['I']}_E{s['E']}_k{s['k']}"
                                                    for s in FUSED_EDGES])
def test_single_launch_layer(dev, mx, shape):
    """The persistent single-launch layer: within the oracle bound, bit-identical to the
    stage entry points and to the default forward, and the workspace control words are zero
    after the call (no wait gave up)."""
    cfg = synthetic.MoEConfig("fused", routing="normal", e_lo=-8, e_hi=-2, seed=shape["T"] * 31 + shape["E"], **shape)
    say("single-launch layer", shape)
    small = cfg.E <= 64
    host = synthetic.moe_inputs_host(cfg) if small else None
    d, x, logits = moe_device_inputs(cfg, dev, host)
    ws = mx.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dev)
    y = mx.moe_mxfp4_forward(d["x"], d["logits"], cfg.k, d["wgu"], d["sgu"], d["wd"], d["sd"], ws=ws,
                             persistent=True)
    torch.cuda.synchronize()
    got = to_host_bits(y)
    assert not ws[:CTL_BYTES].any().item(), "control words not reset"
    assert np.array_equal(run_hooks(mx, d, cfg.k, cfg.T), got)
    assert np.array_equal(run_moe(mx, d, cfg.k), got)
    w_host = host if small else {key: d[key].cpu().numpy() for key in ("wgu", "sgu", "wd", "sd")}
    tok = np.arange(cfg.T, dtype=np.int32) if small else np.array([0, cfg.T // 2, cfg.T - 1], np.int32)
    yo, sm = oracle_moe(cfg, x, logits, w_host, tokens=tok)
    worst = check_bound(got[tok], yo, sm, MOE_REL, f"single-launch {shape}")
    say(f"  worst ratio {worst:.3g}")


def test_single_launch_back_to_back_sizes(dev, mx):
    """Persistent calls of different sizes on one workspace, back to back without
    synchronizing and mixed with default forwards: each persistent call finds the control
    words as the previous one left them."""
    shapes = [dict(T=16, H=1024, I=1024, E=32, k=8), dict(T=2, H=1024, I=1024, E=32, k=8),
              dict(T=7, H=1024, I=1024, E=32, k=4), dict(T=40, H=1024, I=1024, E=32, k=2),
              dict(T=1, H=1024, I=1024, E=32, k=8)]
    say("single-launch layer, back-to-back sizes")
    ws = mx.workspace(40, 1024, 1024, 32, 8, dev)
    runs = []
    for i, s in enumerate(shapes):
        cfg = synthetic.MoEConfig("b2b", routing="normal", e_lo=-8, e_hi=-2, seed=100 + i, **s)
        host = synthetic.moe_inputs_host(cfg)
        d, x, logits = moe_device_inputs(cfg, dev, host)
        y = mx.moe_mxfp4_forward(d["x"], d["logits"], cfg.k, d["wgu"], d["sgu"], d["wd"], d["sd"], ws=ws,
                                 persistent=cfg.T <= 16, check=False)
        runs.append((cfg, host, x, logits, y))
    torch.cuda.synchronize()
    assert not ws[:CTL_BYTES].any().item()
    for cfg, host, x, logits, y in runs:
        yo, sm = oracle_moe(cfg, x, logits, host)
        check_bound(to_host_bits(y), yo, sm, MOE_REL, f"back-to-back T={cfg.T}")


def test_down_launch_combine_back_to_back(dev, mx):
    """At small T the down launch also combines (the workgroup completing a column quad sums
    it).  Calls of sizes on both sides of that rule, with shared experts and MXFP8
    activations, back to back on one workspace without synchronizing: each must match the
    oracle, and the control words must end zero."""
    shapes = [dict(T=4, H=1024, I=1024, E=32, k=8), dict(T=1, H=2048, I=1024, E=8, k=2),
              dict(T=40, H=1024, I=1024, E=16, k=2), dict(T=8, H=1024, I=512, E=64, k=8),
              dict(T=2, H=1024, I=1024, E=6, k=2, n_shared=1), dict(T=16, H=1024, I=1024, E=64, k=8),
              dict(T=3, H=1024, I=1024, E=32, k=4)]
    say("down launch with its combine, back-to-back sizes")
    ws = mx.workspace(40, 2048, 1024, 65, 9, dev)
    runs = []
    for i, s_ in enumerate(shapes):
        cfg = synthetic.MoEConfig("b2b_comb", routing="normal", e_lo=-8, e_hi=-2, seed=200 + i, **s_)
        host = synthetic.moe_inputs_host(cfg)
        d, x, logits = moe_device_inputs(cfg, dev, host)
        act8 = i % 3 == 1
        y = mx.moe_mxfp4_forward(d["x"], d["logits"], cfg.k, d["wgu"], d["sgu"], d["wd"], d["sd"], ws=ws,
                                 n_shared=cfg.n_shared, act8=act8)
        runs.append((cfg, host, x, logits, y, act8))
    torch.cuda.synchronize()
    assert not ws[:CTL_BYTES].any().item()
    for cfg, host, x, logits, y, act8 in runs:
        yo, sm, _ = oracle.moe_tokens(x, logits, cfg.k, host["wgu"], host["sgu"], host["wd"], host["sd"], cfg.T,
                                      cfg.H, cfg.I, cfg.E, n_shared=cfg.n_shared, act8=act8)
        check_bound(to_host_bits(y), yo, sm, MOE_REL, f"back-to-back combine T={cfg.T} act8={act8}")


@pytest.mark.parametrize("T,persistent,E,k", [(4, True, 16, 4), (4, False, 16, 4), (20, False, 16, 4),
                                               (24, False, 128, 8)])
def test_forward_graph_replays(dev, mx, T, persistent, E, k):
    """The forward captured in a HIP graph: every replay, with eager work and
    synchronizations between replays, gives the eager result bit for bit (at T = 24 over 128
    experts: the routing launch that fills h, both expert GEMMs in one launch, the combine)."""
    cfg = synthetic.MoEConfig("graph", T=T, H=1024, I=1024, E=E, k=k, routing="normal", e_lo=-8, e_hi=-2, seed=T)
    host = synthetic.moe_inputs_host(cfg)
    say("forward graph replays, T =", T, "persistent =", persistent)
    d, x, logits = moe_device_inputs(cfg, dev, host)
    ws = mx.workspace(T, cfg.H, cfg.I, cfg.E, cfg.k, dev)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    fwd = lambda: mx.moe_mxfp4_forward(d["x"], d["logits"], cfg.k, d["wgu"], d["sgu"], d["wd"], d["sd"], out=out,
                                       ws=ws, persistent=persistent)
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
        fwd()  # eager work between replays
        torch.cuda.synchronize()
    assert not ws[:CTL_BYTES].any().item()
    yo, sm = oracle_moe(cfg, x, logits, host)
    check_bound(ref, yo, sm, MOE_REL, f"graph T={T}")


# ------------------------------------------------------------------ HBM reference kernels, streams

def test_hbm_reference_kernels(dev, mx):
    """The bandwidth yardsticks compute what they claim: the read kernel's XOR of every
    16-byte piece (bit-exact against numpy) and an exact copy, with a ragged tail."""
    n = (64 << 20) + 48
    host = np.random.default_rng(9).integers(0, 256, size=n, dtype=np.uint8)
    src = torch.from_numpy(host).to(dev)
    say("hbm read / copy", n)
    got = mx.hbm_read(src).cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host.view(np.uint32).reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)
    dst = torch.full_like(src, 0xA5)
    mx.hbm_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_workspace_cache_is_per_stream_and_streams_run_concurrently(dev, mx):
    """The binding's cached workspaces are keyed by stream, so forwards issued on two
    streams at once do not share control words: both give the single-stream result."""
    cfg = synthetic.MoEConfig("streams", T=24, H=1024, I=1024, E=16, k=4, routing="normal", e_lo=-8, e_hi=-2, seed=4)
    host = synthetic.moe_inputs_host(cfg)
    say("two streams")
    d, x, logits = moe_device_inputs(cfg, dev, host)
    ref = run_moe(mx, d, cfg.k)
    s1, s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    w1 = mx.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dev, stream=s1)
    w2 = mx.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dev, stream=s2)
    assert w1.data_ptr() != w2.data_ptr()
    assert mx.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dev, stream=s1).data_ptr() == w1.data_ptr()
    outs = []
    torch.cuda.synchronize()
    for st in (s1, s2):
        with torch.cuda.stream(st):
            ys = [mx.moe_mxfp4_forward(d["x"], d["logits"], cfg.k, d["wgu"], d["sgu"], d["wd"], d["sd"])
                  for _ in range(3)]
        outs.extend(ys)
    torch.cuda.synchronize()
    for y in outs:
        assert np.array_equal(to_host_bits(y), ref)
    assert not w1[:CTL_BYTES].any().item() and not w2[:CTL_BYTES].any().item()
