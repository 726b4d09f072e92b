"""Plain CPU oracle for the MXFP4 MoE layer and the dense MXFP4 linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``mxfp4_weight_moe_amd``) never imports it, and it never imports the GPU
library: the two share no code.  The C source (``mx_oracle.c``) states every
reading of the pages it follows; this module only marshals numpy arrays into
it through ctypes.

Functions pinned by ``tests/test_oracle_*.py``:
  e2m1, e8m0, pack/unpack  -> code table, all 256 scale bytes, round trips
  mx_linear                -> one-hot extraction, exact rational sums, numpy
                              fp64 matmul at unit scale, sign/scale invariants
  route                    -> numpy lexsort, scipy softmax, k = 1
  sort                     -> numpy stable argsort + bincount
  moe_tokens               -> E = 1 reduction to the dense layer, identical-
                              expert invariance, a separately written fp64
                              brute-force MoE on tiny shapes
  e4m3, mxfp8_quantize     -> torch's float8_e4m3fn decode and cast, nearest-
                              value enumeration, scale/sign invariants
  mx_linear_a8             -> one-hot extraction, reduction to mx_linear on
                              MXFP8-representable activations, exact sums
  moe_tokens(act8=True)    -> E = 1 reduction to two mx_linear_a8 calls,
                              reduction to the bf16 layer, a brute force
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
# MXMOE_ORACLE_LIB: load another build of mx_oracle.c (the sanitizer test's)
_LIB_PATH = os.environ.get("MXMOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile mx_oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.ora_version.restype = ctypes.c_int
    lib.ora_e2m1.restype = ctypes.c_double
    lib.ora_e2m1.argtypes = [ctypes.c_int]
    lib.ora_e8m0.restype = ctypes.c_double
    lib.ora_e8m0.argtypes = [ctypes.c_int]
    lib.ora_bf16_rne.restype = ctypes.c_uint16
    lib.ora_bf16_rne.argtypes = [ctypes.c_double]
    lib.ora_pack_codes.argtypes = [P, I64, P]
    lib.ora_unpack_codes.argtypes = [P, I64, P]
    lib.ora_dequant_f64.argtypes = [P, P, I64, I64, P]
    lib.ora_mx_linear.argtypes = [P, P, P, I64, I64, I64, P, P, P, ctypes.c_int]
    lib.ora_route.argtypes = [P, I64, I64, I64, P, P]
    lib.ora_sort.argtypes = [P, I64, I64, I64, P, P, P, P, P]
    lib.ora_moe_tokens.argtypes = [P, P, I64, I64, P, P, P, P, I64, I64, I64, I64, P, I64, P, P, P, ctypes.c_int]
    lib.ora_moe_tokens_a8.argtypes = lib.ora_moe_tokens.argtypes
    lib.ora_moe_tokens_terms.argtypes = lib.ora_moe_tokens.argtypes[:-1] + [P, P, P, P, ctypes.c_int]
    lib.ora_e4m3.restype = ctypes.c_double
    lib.ora_e4m3.argtypes = [ctypes.c_int]
    lib.ora_mxfp8_quantize.argtypes = [P, I64, I64, P, P]
    lib.ora_mx_linear_a8.argtypes = lib.ora_mx_linear.argtypes
    for name in ("ora_pack_codes", "ora_unpack_codes", "ora_dequant_f64", "ora_mx_linear",
                 "ora_route", "ora_sort", "ora_moe_tokens", "ora_moe_tokens_a8", "ora_moe_tokens_terms",
                 "ora_mxfp8_quantize",
                 "ora_mx_linear_a8"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def default_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", 0)) or (os.cpu_count() or 1)


def version() -> int:
    return _load().ora_version()


def e2m1(code: int) -> float:
    return _load().ora_e2m1(int(code))


def e8m0(s: int) -> float:
    return _load().ora_e8m0(int(s))


def bf16_rne(v: float) -> int:
    """Round a float to bf16 bits (nearest, ties to even)."""
    return int(_load().ora_bf16_rne(float(v)))


def pack_codes(codes: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8).ravel()
    assert codes.size % 2 == 0
    out = np.empty(codes.size // 2, np.uint8)
    _load().ora_pack_codes(_p(codes), codes.size, _p(out))
    return out


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = _c(packed, np.uint8).ravel()
    out = np.empty(packed.size * 2, np.uint8)
    _load().ora_unpack_codes(_p(packed), out.size, _p(out))
    return out


def dequant(w: np.ndarray, s: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Exact fp64 weights [rows, K] from packed codes [rows, K/2] and scales [rows, K/32]."""
    w = _c(w, np.uint8)
    s = _c(s, np.uint8)
    assert w.size == rows * K // 2 and s.size == rows * K // 32
    out = np.empty((rows, K), np.float64)
    _load().ora_dequant_f64(_p(w), _p(s), rows, K, _p(out))
    return out


def mx_linear(x_bits: np.ndarray, w: np.ndarray, s: np.ndarray, T: int, K: int, N: int,
              nthreads: int | None = None):
    """Returns (y bf16 bits [T,N] uint16, acc fp32 [T,N], scale_d fp64 [T,N])."""
    x_bits = _c(x_bits, np.uint16)
    w = _c(w, np.uint8)
    s = _c(s, np.uint8)
    assert x_bits.size == T * K and w.size == N * K // 2 and s.size == N * K // 32
    y = np.empty((T, N), np.uint16)
    acc = np.empty((T, N), np.float32)
    sd = np.empty((T, N), np.float64)
    _load().ora_mx_linear(_p(x_bits), _p(w), _p(s), T, K, N, _p(y), _p(acc), _p(sd),
                          nthreads or default_threads())
    return y, acc, sd


def e4m3(code: int) -> float:
    """Value of an E4M3 byte (NaN for 0x7F and 0xFF)."""
    return _load().ora_e4m3(int(code))


def mxfp8_quantize(x_bits: np.ndarray, rows: int, K: int):
    """MXFP8 quantization of bf16 rows: (codes uint8 [rows,K], scales uint8 [rows,K/32])."""
    x_bits = _c(x_bits, np.uint16)
    assert x_bits.size == rows * K and K % 32 == 0
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    _load().ora_mxfp8_quantize(_p(x_bits), rows, K, _p(codes), _p(scales))
    return codes, scales


def mx_linear_a8(x_bits: np.ndarray, w: np.ndarray, s: np.ndarray, T: int, K: int, N: int,
                 nthreads: int | None = None):
    """The dense layer with MXFP8-quantized activations; returns as mx_linear, with
    scale_d = sum_k |q(x) w|."""
    x_bits = _c(x_bits, np.uint16)
    w = _c(w, np.uint8)
    s = _c(s, np.uint8)
    assert x_bits.size == T * K and w.size == N * K // 2 and s.size == N * K // 32 and K % 32 == 0
    y = np.empty((T, N), np.uint16)
    acc = np.empty((T, N), np.float32)
    sd = np.empty((T, N), np.float64)
    _load().ora_mx_linear_a8(_p(x_bits), _p(w), _p(s), T, K, N, _p(y), _p(acc), _p(sd),
                             nthreads or default_threads())
    return y, acc, sd


def route(logits: np.ndarray, k: int):
    """Returns (ids int32 [T,k], gates fp32 [T,k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    assert 1 <= k <= E
    assert np.all(np.isfinite(logits)), "router logits must be finite"
    ids = np.empty((T, k), np.int32)
    gates = np.empty((T, k), np.float32)
    _load().ora_route(_p(logits), T, E, k, _p(ids), _p(gates))
    return ids, gates


def sort(ids: np.ndarray, E: int):
    """Returns dict(counts [E], offsets [E+1], sorted_slots [T*k], active [E] (the active
    experts ascending, then -1), num_active)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_slots = np.empty(T * k, np.int32)
    active = np.empty(E, np.int32)
    na = np.zeros(1, np.int32)
    _load().ora_sort(_p(ids), T, k, E, _p(counts), _p(offsets), _p(sorted_slots), _p(active), _p(na))
    return dict(counts=counts, offsets=offsets, sorted_slots=sorted_slots, active=active,
                num_active=int(na[0]))


def moe_tokens(x_bits, logits, k, wgu, sgu, wd, sd, T, H, I, E, tokens=None, want_h=False,
               nthreads: int | None = None, n_shared: int = 0, act8: bool = False):
    """MoE forward for the listed tokens (default: all).  Each token routes to k of the E
    routed experts (softmax gates over the selected logits) and to the n_shared shared
    experts E .. E + n_shared - 1 with gate 1; the weight arrays hold E + n_shared experts.

    act8: quantize x before gate_up and h before down to MXFP8 (the GEMMs read the
    quantized values; h is still returned in bf16, scale_m uses the quantized h).

    Returns (y bf16 bits [ntok,H], scale_m fp64 [ntok,H], h bf16 bits [ntok*(k+n_shared), I]
    or None).  Weight arrays may be any contiguous uint8 arrays holding [E+n_shared, ...] tensors.
    """
    x_bits = _c(x_bits, np.uint16)
    logits = _c(logits, np.float32)
    assert x_bits.size == T * H and logits.size == T * E
    Ew = E + n_shared
    for a, n in ((wgu, Ew * 2 * I * H // 2), (sgu, Ew * 2 * I * H // 32), (wd, Ew * H * I // 2),
                 (sd, Ew * H * I // 32)):
        assert a.dtype == np.uint8 and a.flags.c_contiguous and a.size == n
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = _c(tokens, np.int32)
    ntok = tokens.size
    y = np.empty((ntok, H), np.uint16)
    sm = np.empty((ntok, H), np.float64)
    h = np.empty((ntok * (k + n_shared), I), np.uint16) if want_h else None
    fn = _load().ora_moe_tokens_a8 if act8 else _load().ora_moe_tokens
    fn(_p(x_bits), _p(logits), k, n_shared, _p(wgu), _p(sgu), _p(wd), _p(sd), T, H, I, E, _p(tokens), ntok,
       _p(y), _p(sm), _p(h) if want_h else None, nthreads or default_threads())
    return y, sm, h


def moe_gate_up_terms(x_bits, logits, k, wgu, sgu, wd, sd, T, H, I, E, tokens=None,
                      nthreads: int | None = None, n_shared: int = 0):
    """moe_tokens (bf16 activations) with the gate_up terms of every slot row.

    Returns (y, scale_m, h, terms) as moe_tokens(want_h=True) does, with terms =
    dict(g, u: fp32 [ntok*(k+n_shared), I], the dot products before SwiGLU; gabs, uabs:
    fp64, sum_K |x w| of the gate and up rows).  Row i*(k+n_shared) + j is slot j of
    token tokens[i].
    """
    x_bits = _c(x_bits, np.uint16)
    logits = _c(logits, np.float32)
    assert x_bits.size == T * H and logits.size == T * E
    Ew = E + n_shared
    for a, n in ((wgu, Ew * 2 * I * H // 2), (sgu, Ew * 2 * I * H // 32), (wd, Ew * H * I // 2),
                 (sd, Ew * H * I // 32)):
        assert a.dtype == np.uint8 and a.flags.c_contiguous and a.size == n
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = _c(tokens, np.int32)
    ntok = tokens.size
    rows = ntok * (k + n_shared)
    y = np.empty((ntok, H), np.uint16)
    sm = np.empty((ntok, H), np.float64)
    h = np.empty((rows, I), np.uint16)
    g = np.empty((rows, I), np.float32)
    u = np.empty((rows, I), np.float32)
    ga = np.empty((rows, I), np.float64)
    ua = np.empty((rows, I), np.float64)
    _load().ora_moe_tokens_terms(_p(x_bits), _p(logits), k, n_shared, _p(wgu), _p(sgu), _p(wd), _p(sd), T, H, I, E,
                                 _p(tokens), ntok, _p(y), _p(sm), _p(h), _p(g), _p(u), _p(ga), _p(ua),
                                 nthreads or default_threads())
    return y, sm, h, dict(g=g, u=u, gabs=ga, uabs=ua)
