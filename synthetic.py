"""Seeded synthetic inputs for the MXFP4 linear and MoE workloads.

This module only draws random numbers with the shapes and distributions of
the workloads; it holds none of the layer's arithmetic (no decode, no routing,
no rounding).  Both the oracle side and the GPU side of the tests take their
inputs from here, and nothing else is shared between them.

Data formats produced:
  x       bf16 bit patterns (uint16): an fp32 N(0,1) draw rounded to nearest-even bf16
  codes   uint8, two 4-bit codes per byte, every byte uniform over 0..255
          (so every 4-bit code, -0 included, is uniform)
  scales  uint8 E8M0 bytes, 127 + e with e uniform over [e_lo, e_hi]
  logits  fp32 router logits

Workload shapes are those the pages use for fused-MoE kernels (H = 7168,
E = 256 or 384, top-8; "Zyphra Inference Wave 2", Figure 10) with an expert
intermediate size of 2048.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

try:  # torch is only needed for device-side generation
    import torch
except Exception:  # pragma: no cover
    torch = None


# --------------------------------------------------------------------------- configs

@dataclass(frozen=True)
class LinearConfig:
    name: str
    T: int
    K: int
    N: int
    e_lo: int
    e_hi: int
    seed: int = 0


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    routing: str  # "normal" | "zipf" | "uniform" | "spec"
    e_lo: int = -6
    e_hi: int = 0
    seed: int = 0
    zipf_s: float = 1.1
    positions: int = 1        # "spec": speculative positions per request (T = requests x positions)
    spec_sigma: float = 1.2   # "spec": spread of the per-request expert preference
    n_shared: int = 0         # always-active shared experts, after the E routed ones


LINEAR_CONFIGS = {
    # 1 token, 2048 -> 2048, scales 2^-4 .. 2^2, seed 0
    "dense_t1": LinearConfig("dense_t1", T=1, K=2048, N=2048, e_lo=-4, e_hi=2, seed=0),
    # 4 tokens (1 decode + 3 draft positions), 7168 -> 4096, scales 2^-6 .. 2^0
    "dense_t4": LinearConfig("dense_t4", T=4, K=7168, N=4096, e_lo=-6, e_hi=0, seed=0),
}

MOE_CONFIGS = {
    # 4 tokens, 256 experts, N(0,1) logits
    "moe_t4": MoEConfig("moe_t4", T=4, H=7168, I=2048, E=256, k=8, routing="normal"),
    # 32 requests x 1 position, Zipf(1.1)-skewed expert load
    "moe_t32_zipf": MoEConfig("moe_t32_zipf", T=32, H=7168, I=2048, E=256, k=8, routing="zipf"),
    # 32 requests x 4 speculative positions, 384 experts, uniform-random logits
    "moe_t128": MoEConfig("moe_t128", T=128, H=7168, I=2048, E=384, k=8, routing="uniform"),
    # the same step with the positions of each request routed alike (speculative verify)
    "moe_spec_t128": MoEConfig("moe_spec_t128", T=128, H=7168, I=2048, E=384, k=8, routing="spec", positions=4),
    # one request, 4 speculative positions
    "moe_spec_t4": MoEConfig("moe_spec_t4", T=4, H=7168, I=2048, E=256, k=8, routing="spec", positions=4),
    # one GPU's share of a layer split 8 ways by tensor parallelism: each expert's
    # intermediate width 2048 / 8 = 256 (the same routing as moe_t4 and moe_t32_zipf)
    "moe_tp8_t4": MoEConfig("moe_tp8_t4", T=4, H=7168, I=256, E=256, k=8, routing="normal"),
    "moe_tp8_t32": MoEConfig("moe_tp8_t32", T=32, H=7168, I=256, E=256, k=8, routing="zipf"),
    # 256 routed experts (top-8) and one always-active shared expert, each token reading
    # 9 experts (the GLM-5.3 layer of "Zyphra Inference Wave 2", section "Quantization")
    "moe_shared_t1": MoEConfig("moe_shared_t1", T=1, H=7168, I=2048, E=256, k=8, routing="normal", n_shared=1),
    "moe_shared_t32": MoEConfig("moe_shared_t32", T=32, H=7168, I=2048, E=256, k=8, routing="zipf", n_shared=1),
}


def sweep_config(T: int, seed: int = 0) -> MoEConfig:
    """T-sweep point with the 4-token config's distributions (E = 256, N(0,1) logits)."""
    return MoEConfig(f"moe_sweep_t{T}", T=T, H=7168, I=2048, E=256, k=8, routing="normal", seed=seed)


def small_scale_variant(cfg: MoEConfig) -> MoEConfig:
    """Parity-only variant with scales 2^-12 .. 2^-6 so |g| is O(1) and SiLU is curved."""
    return replace(cfg, name=cfg.name + "_smallscale", e_lo=-12, e_hi=-6)


# --------------------------------------------------------------------------- host (numpy) draws

def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag])))


TAG_X, TAG_LOGITS, TAG_W, TAG_S, TAG_ZIPF, TAG_SPEC = 1, 2, 3, 4, 5, 6


def bf16_bits_normal(shape, seed: int, tag: int = TAG_X) -> np.ndarray:
    """bf16 bit patterns of an N(0,1) draw: each fp32 sample rounded to the nearest bf16,
    ties to even (the samples are finite and far from the bf16 range's ends)."""
    u = _rng(seed, tag).standard_normal(size=shape, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def random_codes(rows: int, K: int, seed: int, tag: int = TAG_W) -> np.ndarray:
    """Packed 4-bit codes [rows, K/2]: uniform random bytes."""
    return _rng(seed, tag).integers(0, 256, size=(rows, K // 2), dtype=np.uint8)


def random_scales(rows: int, K: int, e_lo: int, e_hi: int, seed: int, tag: int = TAG_S) -> np.ndarray:
    """E8M0 bytes [rows, K/32] = 127 + e, e uniform over [e_lo, e_hi]."""
    return (127 + _rng(seed, tag).integers(e_lo, e_hi + 1, size=(rows, K // 32))).astype(np.uint8)


def router_logits(cfg: MoEConfig) -> np.ndarray:
    """fp32 [T, E] router logits for the config's routing distribution.

    normal : i.i.d. N(0,1)
    uniform: i.i.d. U[0,1)
    zipf   : experts ranked by a seeded permutation, rank r weighted r^-s; each
             token draws k distinct experts by weighted sampling without
             replacement, and gets N(0,1) logits plus 16 on the drawn experts
             (so the drawn set is the top-k, and the gates stay a softmax of
             N(0,1) values).
    spec   : tokens t = r * positions + p are the speculative positions of request r;
             each request draws an expert preference b_r ~ N(0, spec_sigma^2) per
             expert, shared by its positions, and each token gets b_r + N(0,1).  The
             positions of a request then route to overlapping experts: with
             spec_sigma = 1.2, a request's 4 positions route to about 1.67 times the
             distinct experts of its first 2 (11.7 against 7 on the AMD megakernel
             blog, section "Data Locality"; independent tokens give about 1.95).
    """
    T, E, k = cfg.T, cfg.E, cfg.k
    g = _rng(cfg.seed, TAG_LOGITS)
    if cfg.routing == "normal":
        return g.standard_normal(size=(T, E), dtype=np.float32)
    if cfg.routing == "uniform":
        return g.random(size=(T, E), dtype=np.float32)
    if cfg.routing == "zipf":
        z = _rng(cfg.seed, TAG_ZIPF)
        perm = z.permutation(E)
        w = np.empty(E, np.float64)
        w[perm] = (np.arange(1, E + 1, dtype=np.float64)) ** (-cfg.zipf_s)
        p = w / w.sum()
        base = g.standard_normal(size=(T, E), dtype=np.float32)
        for t in range(T):
            drawn = z.choice(E, size=k, replace=False, p=p)
            base[t, drawn] += np.float32(16.0)
        return base
    if cfg.routing == "spec":
        P = cfg.positions
        R = -(-T // P)
        b = _rng(cfg.seed, TAG_SPEC).standard_normal(size=(R, E)) * cfg.spec_sigma
        noise = g.standard_normal(size=(T, E))
        return (b[np.arange(T) // P] + noise).astype(np.float32)
    raise ValueError(cfg.routing)


def linear_inputs(cfg: LinearConfig):
    """(x bits [T,K] uint16, codes [N,K/2] uint8, scales [N,K/32] uint8)."""
    x = bf16_bits_normal((cfg.T, cfg.K), cfg.seed, TAG_X)
    w = random_codes(cfg.N, cfg.K, cfg.seed, TAG_W)
    s = random_scales(cfg.N, cfg.K, cfg.e_lo, cfg.e_hi, cfg.seed, TAG_S)
    return x, w, s


def moe_inputs_host(cfg: MoEConfig):
    """All MoE inputs on the host (small shapes only: every expert is drawn).

    Returns dict(x [T,H] u16, logits [T,E] f32, wgu [Ew,2I,H/2], sgu [Ew,2I,H/32],
    wd [Ew,H,I/2], sd [Ew,H,I/32]) as numpy arrays, Ew = E + n_shared (the shared experts
    after the routed ones).
    """
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E + cfg.n_shared
    x = bf16_bits_normal((T, H), cfg.seed, TAG_X)
    logits = router_logits(cfg)
    wgu = np.stack([random_codes(2 * I, H, cfg.seed, 1000 + 4 * e) for e in range(E)])
    sgu = np.stack([random_scales(2 * I, H, cfg.e_lo, cfg.e_hi, cfg.seed, 1001 + 4 * e) for e in range(E)])
    wd = np.stack([random_codes(H, I, cfg.seed, 1002 + 4 * e) for e in range(E)])
    sd = np.stack([random_scales(H, I, cfg.e_lo, cfg.e_hi, cfg.seed, 1003 + 4 * e) for e in range(E)])
    return dict(x=x, logits=logits, wgu=wgu, sgu=sgu, wd=wd, sd=sd)


# --------------------------------------------------------------------------- device (torch) draws

def _torch_gen(device, seed: int, tag: int):
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag) & 0x7FFFFFFFFFFFFFFF)
    return g


def device_codes(shape, seed: int, tag: int, device):
    """Uniform random code bytes drawn on `device` with torch's generator."""
    g = _torch_gen(device, seed, tag)
    return torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.uint8)


def device_scales(shape, e_lo: int, e_hi: int, seed: int, tag: int, device):
    g = _torch_gen(device, seed, tag)
    return (torch.randint(e_lo, e_hi + 1, shape, generator=g, device=device, dtype=torch.int16) + 127).to(torch.uint8)


def moe_weights_device(cfg: MoEConfig, device, layer: int = 0):
    """Full [E + n_shared, ...] MXFP4 weight tensors drawn on the device (fast for large E).

    Returns dict(wgu, sgu, wd, sd) as uint8 torch tensors on `device`.
    """
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E + cfg.n_shared
    base = 10_000 * (layer + 1)
    return dict(
        wgu=device_codes((E, 2 * I, H // 2), cfg.seed, base + 1, device),
        sgu=device_scales((E, 2 * I, H // 32), cfg.e_lo, cfg.e_hi, cfg.seed, base + 2, device),
        wd=device_codes((E, H, I // 2), cfg.seed, base + 3, device),
        sd=device_scales((E, H, I // 32), cfg.e_lo, cfg.e_hi, cfg.seed, base + 4, device),
    )


def moe_activations(cfg: MoEConfig, layer: int = 0):
    """(x bits [T,H] u16, logits [T,E] f32) on the host; per-layer seeds differ."""
    c = cfg if layer == 0 else replace(cfg, seed=cfg.seed + 7919 * layer)
    return bf16_bits_normal((c.T, c.H), c.seed, TAG_X), router_logits(c)
