"""Shared helpers of the GPU parity tests: tensor marshalling and the acceptance bounds.

Acceptance (floating point): |gpu - oracle| <= rel * scale + ulp_bf16(max(|gpu|, |oracle|))
with rel = 1e-5 and scale = sum_k |x_k w_nk| for the dense layer, rel = 1e-2 and
scale = sum_j gate_j sum_i |h_i w_ni| for the MoE layer; NaN must match NaN and +-Inf
must match exactly.  Integer outputs are compared bit for bit.
"""
import sys

import numpy as np
import torch

DENSE_REL = 1e-5
MOE_REL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_bf16(a: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(a, np.float64))
    small = a < 2.0 ** -126
    e = np.floor(np.log2(np.where(small, 1.0, a)))
    return np.where(small, 2.0 ** -133, 2.0 ** (e - 7))


def check_bound(gpu_bits, ora_bits, scale, rel, what=""):
    """Returns the worst |err| / tol ratio; asserts it is <= 1."""
    g = bf16_to_f(gpu_bits).astype(np.float64)
    o = bf16_to_f(ora_bits).astype(np.float64)
    assert g.shape == o.shape == np.shape(scale), (g.shape, o.shape, np.shape(scale))
    ng, no = np.isnan(g), np.isnan(o)
    assert np.array_equal(ng, no), f"{what}: NaN positions differ ({ng.sum()} vs {no.sum()})"
    inf = (np.isinf(g) | np.isinf(o)) & ~no
    assert np.array_equal(g[inf], o[inf]), f"{what}: Inf values differ"
    fin = ~(no | inf)
    tol = rel * np.asarray(scale, np.float64)[fin] + ulp_bf16(np.maximum(np.abs(g[fin]), np.abs(o[fin])))
    err = np.abs(g[fin] - o[fin])
    ratio = err / tol
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        bad = np.nonzero(ratio > 1.0)[0]
        raise AssertionError(f"{what}: {bad.size} of {ratio.size} outputs out of bound; worst ratio {worst:.3g}; "
                             f"first bad gpu={g[fin][bad[0]]!r} oracle={o[fin][bad[0]]!r} tol={tol[bad[0]]!r}")
    return worst


def random_linear_shapes(n=16, seed=20261204):
    """Seeded random dense-layer shapes (T, K, N): T from 1 to 64, K any multiple of 32 up to
    8192 (so partial segments and odd scale-row alignments occur), N from 1 to 3000."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        T = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 17, 24, 32, 33, 48, 64]))
        K = 32 * int(rng.integers(1, 257))
        N = int(rng.integers(1, 3001))
        out.append((T, K, N))
    return out

