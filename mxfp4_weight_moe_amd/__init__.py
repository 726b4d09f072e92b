"""Python binding of the mxmoe C ABI (include/mxmoe.h): MXFP4 weight-streaming MoE layer
and dense MXFP4 linear layer for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
libmxmoe.so.  PyTorch provides device memory and the current stream.  If the library is
not built, importing this package raises: there is no fallback path.

bf16 tensors are passed as their bit patterns; MXFP4 weights are uint8 code tensors
[..., rows, K/2] (element 2i in the low nibble) plus uint8 E8M0 scale tensors
[..., rows, K/32].
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxmoe.so")

MX_OK = 0
MX_MAX_TOKENS = 256
MX_MAX_EXPERTS = 1024
MX_MAX_TOPK = 32

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python mxfp4_weight_moe_amd/build.py` (hipcc, gfx950) first")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_lib.mx_version.restype = ctypes.c_int
_lib.mx_status_string.restype = ctypes.c_char_p
_lib.mx_status_string.argtypes = [ctypes.c_int]
_lib.mx_linear.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P]
_lib.mxfp4_dequantize.argtypes = [_P, _P, _I64, _I64, _P, _P]
_lib.moe_route_topk.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P]
_lib.moe_sort_by_expert.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]
_lib.moe_route_sort.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.moe_gate_up_swiglu.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P,
                                    ctypes.c_size_t, _P]
_lib.moe_gate_up_swiglu_from_ids.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P,
                                             ctypes.c_size_t, _P]
_lib.moe_down_combine.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P,
                                  ctypes.c_size_t, _P]
_lib.moe_expert_gemms_from_ids.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _P, _I64, _I64, _I64, _I64,
                                           _I64, _P, ctypes.c_size_t, _P]
_lib.moe_combine.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
_lib.moe_mxfp4_workspace_size.restype = ctypes.c_size_t
_lib.moe_mxfp4_workspace_size.argtypes = [_I64, _I64, _I64, _I64, _I64]
_lib.moe_mxfp4_forward.argtypes = [_P, _P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]
_lib.moe_mxfp4_forward_persistent.argtypes = list(_lib.moe_mxfp4_forward.argtypes)
_lib.moe_mxfp4_forward_shared.argtypes = [_P, _P, _I64, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P,
                                          ctypes.c_size_t, _P]
_lib.moe_mxfp4_forward_a8.argtypes = list(_lib.moe_mxfp4_forward_shared.argtypes)
_lib.mx_linear_a8.argtypes = list(_lib.mx_linear.argtypes)
_lib.mxfp8_quantize.argtypes = [_P, _I64, _I64, _P, _P, _P]
_lib.moe_mxfp4_forward_noalloc.argtypes = [_P, _P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
_lib.mx_hbm_read.argtypes = [_P, ctypes.c_size_t, _P, _P]
_lib.mx_hbm_copy.argtypes = [_P, _P, ctypes.c_size_t, _P]
for _n in ("mx_linear", "mxfp4_dequantize", "moe_route_topk", "moe_sort_by_expert", "moe_route_sort",
           "moe_gate_up_swiglu", "moe_down_combine", "moe_mxfp4_forward", "moe_mxfp4_forward_persistent",
           "moe_mxfp4_forward_shared", "moe_mxfp4_forward_a8", "mx_linear_a8", "mxfp8_quantize", "mx_hbm_read",
           "mx_hbm_copy", "moe_mxfp4_forward_noalloc", "moe_gate_up_swiglu_from_ids", "moe_expert_gemms_from_ids",
           "moe_combine"):
    getattr(_lib, _n).restype = ctypes.c_int

EXPORTED = ("mx_version", "mx_status_string", "mx_linear", "mxfp4_dequantize", "moe_route_topk",
            "moe_sort_by_expert", "moe_route_sort", "moe_gate_up_swiglu", "moe_down_combine",
            "moe_mxfp4_workspace_size", "moe_mxfp4_forward", "moe_mxfp4_forward_persistent",
            "moe_mxfp4_forward_shared", "moe_mxfp4_forward_a8", "mx_linear_a8", "mxfp8_quantize", "mx_hbm_read",
            "mx_hbm_copy", "moe_mxfp4_forward_noalloc", "moe_gate_up_swiglu_from_ids", "moe_expert_gemms_from_ids",
            "moe_combine")
MX_ERR_SCRATCH = -6
MX_NOALLOC_SCRATCH_BYTES = 40 << 20


class MxError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {status_string(status)} (status {status})")


def version() -> int:
    return _lib.mx_version()


def status_string(status: int) -> str:
    return _lib.mx_status_string(int(status)).decode()


def raw():
    """The ctypes handle of libmxmoe.so (for tests that call the C ABI directly)."""
    return _lib


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _raise(status: int, call: str):
    if status != MX_OK:
        if status == -2:
            raise ValueError(f"{call}: {status_string(status)}")
        raise MxError(status, call)


def mx_linear(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
              out: torch.Tensor | None = None, act8: bool = False) -> torch.Tensor:
    """y[T,N] = bf16(x[T,K] @ dequant(w)[N,K]^T), fp32 accumulation.
    act8=True: x quantized to MXFP8 first, scaled MFMA (mx_linear_a8)."""
    _check(x, "x", torch.bfloat16, 2)
    dev = x.device
    _check(w_codes, "w_codes", torch.uint8, 2, dev)
    _check(w_scales, "w_scales", torch.uint8, 2, dev)
    T, K = x.shape
    N = w_codes.shape[0]
    if w_codes.shape != (N, K // 2) or w_scales.shape != (N, K // 32) or K % 32:
        raise ValueError(f"weight shapes {tuple(w_codes.shape)}, {tuple(w_scales.shape)} do not match K={K}")
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, 2, dev)
    if out.shape != (T, N):
        raise ValueError("out has the wrong shape")
    name = "mx_linear_a8" if act8 else "mx_linear"
    st = getattr(_lib, name)(_ptr(x), _ptr(w_codes), _ptr(w_scales), _ptr(out), T, K, N, _stream(dev))
    _raise(st, name)
    return out


def hbm_read(src: torch.Tensor, xor_out: torch.Tensor | None = None, clear: bool = True) -> torch.Tensor:
    """HBM reference read of a contiguous device tensor (size a multiple of 16 bytes):
    returns int32 [4], word c = XOR of 32-bit word c of every 16-byte piece (XORed into
    xor_out, which is zeroed first unless clear=False)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    dev = src.device
    if xor_out is None:
        xor_out = torch.zeros(4, dtype=torch.int32, device=dev)
    else:
        _check(xor_out, "xor_out", torch.int32, 1, dev)
        if clear:
            xor_out.zero_()
    nbytes = src.numel() * src.element_size()
    st = _lib.mx_hbm_read(_ptr(src), nbytes, _ptr(xor_out), _stream(dev))
    _raise(st, "mx_hbm_read")
    return xor_out


def hbm_copy(dst: torch.Tensor, src: torch.Tensor) -> torch.Tensor:
    """HBM reference copy between two contiguous device tensors of the same byte size."""
    for t, n in ((dst, "dst"), (src, "src")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or dst.device != src.device:
        raise ValueError("dst and src must have the same byte size and device")
    st = _lib.mx_hbm_copy(_ptr(dst), _ptr(src), nbytes, _stream(src.device))
    _raise(st, "mx_hbm_copy")
    return dst


def mxfp8_quantize(x: torch.Tensor):
    """MXFP8 (E4M3 codes, E8M0 scales per 32) of bf16 rows: (codes uint8 [R, K], scales uint8 [R, K/32])."""
    _check(x, "x", torch.bfloat16, 2)
    dev = x.device
    R, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    codes = torch.empty((R, K), dtype=torch.uint8, device=dev)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=dev)
    st = _lib.mxfp8_quantize(_ptr(x), R, K, _ptr(codes), _ptr(scales), _stream(dev))
    _raise(st, "mxfp8_quantize")
    return codes, scales


def mxfp4_dequantize(w_codes: torch.Tensor, w_scales: torch.Tensor) -> torch.Tensor:
    """bf16 [rows, K] = E2M1(code) * 2^(s - 127), exact."""
    _check(w_codes, "w_codes", torch.uint8)
    dev = w_codes.device
    _check(w_scales, "w_scales", torch.uint8, None, dev)
    K = w_codes.shape[-1] * 2
    rows = w_codes.numel() // (K // 2)
    if w_scales.numel() != rows * (K // 32) or w_scales.shape[:-1] != w_codes.shape[:-1]:
        raise ValueError("scale tensor does not match the code tensor")
    out = torch.empty((*w_codes.shape[:-1], K), dtype=torch.bfloat16, device=dev)
    st = _lib.mxfp4_dequantize(_ptr(w_codes), _ptr(w_scales), rows, K, _ptr(out), _stream(dev))
    _raise(st, "mxfp4_dequantize")
    return out


def moe_route_topk(logits: torch.Tensor, top_k: int, ids: torch.Tensor | None = None,
                   gates: torch.Tensor | None = None):
    """(ids int32 [T,k], gates fp32 [T,k]): top-k logits (ties to lower id), softmax over them."""
    _check(logits, "router_logits", torch.float32, 2)
    dev = logits.device
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _check(ids, "ids", torch.int32, 2, dev)
    _check(gates, "gates", torch.float32, 2, dev)
    if ids.shape != (T, top_k) or gates.shape != (T, top_k):
        raise ValueError("ids / gates must be [T, top_k]")
    st = _lib.moe_route_topk(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(gates), _stream(dev))
    _raise(st, "moe_route_topk")
    return ids, gates


_SORT_KEYS = ("counts", "offsets", "sorted_slots", "active", "num_active")


def _sort_ptrs(sort: dict, dev):
    for key in _SORT_KEYS:
        _check(sort[key], key, torch.int32, 1, dev)
    return [_ptr(sort[key]) for key in _SORT_KEYS]


def _sort_out(out: dict | None, T: int, k: int, E: int, dev) -> dict:
    if out is not None:
        _sort_ptrs(out, dev)
        if (out["counts"].numel() != E or out["offsets"].numel() != E + 1 or out["sorted_slots"].numel() != T * k
                or out["active"].numel() != E or out["num_active"].numel() != 2):
            raise ValueError("sort output tensors have the wrong sizes")
        return out
    return dict(
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        sorted_slots=torch.empty(T * k, dtype=torch.int32, device=dev),
        active=torch.empty(E, dtype=torch.int32, device=dev),
        num_active=torch.empty(2, dtype=torch.int32, device=dev),
    )


def moe_sort_by_expert(ids: torch.Tensor, num_experts: int, out: dict | None = None) -> dict:
    """Counting sort of the flat slots by expert (experts ascending, slot ascending)."""
    _check(ids, "ids", torch.int32, 2)
    dev = ids.device
    T, k = ids.shape
    E = int(num_experts)
    out = _sort_out(out, T, k, E, dev)
    st = _lib.moe_sort_by_expert(_ptr(ids), T, k, E, _ptr(out["counts"]), _ptr(out["offsets"]),
                                 _ptr(out["sorted_slots"]), _ptr(out["active"]), _ptr(out["num_active"]),
                                 _stream(dev))
    _raise(st, "moe_sort_by_expert")
    return out


def moe_route_sort(logits: torch.Tensor, top_k: int, ids: torch.Tensor | None = None,
                   gates: torch.Tensor | None = None, out: dict | None = None):
    """moe_route_topk then moe_sort_by_expert in one launch: (ids, gates, sort dict)."""
    _check(logits, "router_logits", torch.float32, 2)
    dev = logits.device
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _check(ids, "ids", torch.int32, 2, dev)
    _check(gates, "gates", torch.float32, 2, dev)
    if ids.shape != (T, top_k) or gates.shape != (T, top_k):
        raise ValueError("ids / gates must be [T, top_k]")
    out = _sort_out(out, T, top_k, E, dev)
    st = _lib.moe_route_sort(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(gates), *[_ptr(out[key]) for key in _SORT_KEYS],
                             _stream(dev))
    _raise(st, "moe_route_sort")
    return ids, gates, out


def moe_gate_up_swiglu(x: torch.Tensor, W_gate_up: torch.Tensor, S_gate_up: torch.Tensor, sort: dict, top_k: int,
                       h: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Stage hook: h [T*k, I] bf16 (rows in sorted-slot order) from a moe_sort_by_expert result."""
    _check(x, "x", torch.bfloat16, 2)
    dev = x.device
    _check(W_gate_up, "W_gate_up", torch.uint8, 3, dev)
    _check(S_gate_up, "S_gate_up", torch.uint8, 3, dev)
    T, H = x.shape
    E, two_i, _ = W_gate_up.shape
    I = two_i // 2
    if W_gate_up.shape != (E, 2 * I, H // 2) or S_gate_up.shape != (E, 2 * I, H // 32):
        raise ValueError("W_gate_up / S_gate_up shapes do not match [E, 2I, H/2] / [E, 2I, H/32]")
    if h is None:
        h = torch.empty((T * top_k, I), dtype=torch.bfloat16, device=dev)
    _check(h, "h", torch.bfloat16, 2, dev)
    if ws is None:
        ws = workspace(T, H, I, E, top_k, dev)
    _check(ws, "workspace", torch.uint8, 1, dev)
    st = _lib.moe_gate_up_swiglu(_ptr(x), _ptr(W_gate_up), _ptr(S_gate_up), *_sort_ptrs(sort, dev), _ptr(h), T, H, I,
                                 E, top_k, _ptr(ws), ws.numel(), _stream(dev))
    _raise(st, "moe_gate_up_swiglu")
    return h


def moe_gate_up_swiglu_from_ids(x: torch.Tensor, ids: torch.Tensor, W_gate_up: torch.Tensor, S_gate_up: torch.Tensor,
                                h: torch.Tensor | None = None, sort: dict | None = None,
                                ws: torch.Tensor | None = None):
    """Stage hook for T <= 32: (h [T*k, I] bf16, sort dict) from the routed ids, the slots
    sorted inside the gate_up launch (the sort equals moe_sort_by_expert's)."""
    _check(x, "x", torch.bfloat16, 2)
    dev = x.device
    _check(ids, "ids", torch.int32, 2, dev)
    _check(W_gate_up, "W_gate_up", torch.uint8, 3, dev)
    _check(S_gate_up, "S_gate_up", torch.uint8, 3, dev)
    T, H = x.shape
    top_k = ids.shape[1]
    E, two_i, _ = W_gate_up.shape
    I = two_i // 2
    if ids.shape[0] != T:
        raise ValueError("ids must be [T, top_k]")
    if W_gate_up.shape != (E, 2 * I, H // 2) or S_gate_up.shape != (E, 2 * I, H // 32):
        raise ValueError("W_gate_up / S_gate_up shapes do not match [E, 2I, H/2] / [E, 2I, H/32]")
    sort = _sort_out(sort, T, top_k, E, dev)
    if h is None:
        h = torch.empty((T * top_k, I), dtype=torch.bfloat16, device=dev)
    _check(h, "h", torch.bfloat16, 2, dev)
    if ws is None:
        ws = workspace(T, H, I, E, top_k, dev)
    _check(ws, "workspace", torch.uint8, 1, dev)
    st = _lib.moe_gate_up_swiglu_from_ids(_ptr(x), _ptr(ids), _ptr(W_gate_up), _ptr(S_gate_up),
                                          *[_ptr(sort[key]) for key in _SORT_KEYS], _ptr(h), T, H, I, E, top_k,
                                          _ptr(ws), ws.numel(), _stream(dev))
    _raise(st, "moe_gate_up_swiglu_from_ids")
    return h, sort


def moe_expert_gemms_from_ids(x: torch.Tensor, ids: torch.Tensor, W_gate_up: torch.Tensor, S_gate_up: torch.Tensor,
                              W_down: torch.Tensor, S_down: torch.Tensor, h: torch.Tensor | None = None,
                              d: torch.Tensor | None = None, ws: torch.Tensor | None = None, fill_h: bool = True):
    """Stage hook for T <= 32: both expert GEMMs in one launch from the routed ids:
    (h [T*k, I] bf16 in sorted-slot order, d [T*k, H] fp32 down outputs by flat slot).
    The launch needs every element of h at 0xFFFF when it starts: fill_h=True has the call
    fill it first (one more launch); with fill_h=False the caller has done so on this stream."""
    _check(x, "x", torch.bfloat16, 2)
    dev = x.device
    _check(ids, "ids", torch.int32, 2, dev)
    for t, n in ((W_gate_up, "W_gate_up"), (S_gate_up, "S_gate_up"), (W_down, "W_down"), (S_down, "S_down")):
        _check(t, n, torch.uint8, 3, dev)
    T, H = x.shape
    top_k = ids.shape[1]
    E = W_gate_up.shape[0]
    I = W_down.shape[2] * 2
    if ids.shape[0] != T:
        raise ValueError("ids must be [T, top_k]")
    if (W_gate_up.shape != (E, 2 * I, H // 2) or S_gate_up.shape != (E, 2 * I, H // 32)
            or W_down.shape != (E, H, I // 2) or S_down.shape != (E, H, I // 32)):
        raise ValueError("expert weight shapes do not match [E, 2I, H/2], [E, 2I, H/32], [E, H, I/2], [E, H, I/32]")
    if h is None:
        h = torch.empty((T * top_k, I), dtype=torch.bfloat16, device=dev)
    if d is None:
        d = torch.empty((T * top_k, H), dtype=torch.float32, device=dev)
    _check(h, "h", torch.bfloat16, 2, dev)
    _check(d, "d", torch.float32, 2, dev)
    if h.shape != (T * top_k, I) or d.shape != (T * top_k, H):
        raise ValueError("h must be [T*top_k, I] and d [T*top_k, H]")
    if ws is None:
        ws = workspace(T, H, I, E, top_k, dev)
    _check(ws, "workspace", torch.uint8, 1, dev)
    st = _lib.moe_expert_gemms_from_ids(_ptr(x), _ptr(ids), _ptr(W_gate_up), _ptr(S_gate_up), _ptr(W_down),
                                        _ptr(S_down), _ptr(h), 0 if fill_h else 1, _ptr(d), T, H, I, E, top_k,
                                        _ptr(ws), ws.numel(), _stream(dev))
    _raise(st, "moe_expert_gemms_from_ids")
    return h, d


def moe_combine(d: torch.Tensor, gates: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Stage hook: y [T, H] bf16 = sum_j gates[t, j] d[t*k + j] (fp32, j ascending)."""
    _check(d, "d", torch.float32, 2)
    dev = d.device
    _check(gates, "gates", torch.float32, 2, dev)
    T, top_k = gates.shape
    H = d.shape[1]
    if d.shape[0] != T * top_k:
        raise ValueError("d must be [T*top_k, H] for gates [T, top_k]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, 2, dev)
    if out.shape != (T, H):
        raise ValueError("out must be [T, H]")
    _raise(_lib.moe_combine(_ptr(d), _ptr(gates), _ptr(out), T, H, top_k, _stream(dev)), "moe_combine")
    return out


def moe_down_combine(h: torch.Tensor, gates: torch.Tensor, W_down: torch.Tensor, S_down: torch.Tensor, sort: dict,
                     T: int, top_k: int, out: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Stage hook: y [T, H] bf16 from gate_up's h, the gates and the sort result."""
    _check(h, "h", torch.bfloat16, 2)
    dev = h.device
    _check(gates, "gates", torch.float32, 2, dev)
    _check(W_down, "W_down", torch.uint8, 3, dev)
    _check(S_down, "S_down", torch.uint8, 3, dev)
    E, H, half_i = W_down.shape
    I = half_i * 2
    if S_down.shape != (E, H, I // 32) or h.shape != (T * top_k, I) or gates.shape != (T, top_k):
        raise ValueError("shapes do not match h [T*k, I], gates [T, k], W_down [E, H, I/2], S_down [E, H, I/32]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, 2, dev)
    if ws is None:
        ws = workspace(T, H, I, E, top_k, dev)
    st = _lib.moe_down_combine(_ptr(h), _ptr(gates), _ptr(W_down), _ptr(S_down), *_sort_ptrs(sort, dev), _ptr(out),
                               T, H, I, E, top_k, _ptr(ws), ws.numel(), _stream(dev))
    _raise(st, "moe_down_combine")
    return out


def workspace_size(T: int, H: int, I: int, E: int, top_k: int) -> int:
    return int(_lib.moe_mxfp4_workspace_size(T, H, I, E, top_k))


_ws_cache: dict = {}


def workspace(T: int, H: int, I: int, E: int, top_k: int, device, stream=None) -> torch.Tensor:
    """A cached uint8 workspace tensor large enough for these sizes, one per (device,
    stream) -- by default the device's current stream.  Calls that share a workspace must
    not overlap in time: calls on one stream run one after another, and calls on two
    streams get two workspaces.  Allocated zero-filled: its leading control words must start
    at zero, and every call leaves them so."""
    need = workspace_size(T, H, I, E, top_k)
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    key = (dev, int(stream.cuda_stream))
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < need:
        buf = torch.zeros(need, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


# moe_mxfp4_forward_persistent: byte offset of the int32 word its bounded waits set to 1
# when they give up (sticky until cleared)
PERSISTENT_ERROR_OFFSET = 8


class MxWaitError(RuntimeError):
    """A single-launch layer's cross-workgroup wait gave up; its output is undefined."""


def take_persistent_error(ws: torch.Tensor) -> int:
    """Read and clear the single-launch layer's sticky error word in `ws` (synchronizes
    with the stream that used it)."""
    word = ws[PERSISTENT_ERROR_OFFSET:PERSISTENT_ERROR_OFFSET + 4].view(torch.int32)
    v = int(word.item())
    if v:
        word.zero_()
    return v


def raise_for_persistent_error(word: int) -> None:
    if word:
        raise MxWaitError("moe_mxfp4_forward_persistent: a cross-workgroup wait gave up (are other kernels "
                          "occupying the GPU?); the output is undefined")


def moe_mxfp4_forward(x: torch.Tensor, router_logits: torch.Tensor, top_k: int, W_gate_up: torch.Tensor,
                      S_gate_up: torch.Tensor, W_down: torch.Tensor, S_down: torch.Tensor,
                      out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                      persistent: bool = False, n_shared: int = 0, act8: bool = False,
                      check: bool = True) -> torch.Tensor:
    """y[T,H] of the MXFP4 SwiGLU MoE layer (see include/mxmoe.h for the definition).
    persistent=True runs it as one persistent launch (moe_mxfp4_forward_persistent; T <= 16);
    with check=True (and outside graph capture) the call then waits for it, reads and clears
    its sticky error word and raises MxWaitError when a wait gave up.
    n_shared > 0: the weights hold E routed + n_shared shared experts, router_logits [T, E]
    (moe_mxfp4_forward_shared).  act8=True: MXFP8 activations for both expert GEMMs
    (moe_mxfp4_forward_a8, with or without shared experts)."""
    _check(x, "x", torch.bfloat16, 2)
    dev = x.device
    _check(router_logits, "router_logits", torch.float32, 2, dev)
    for t, n in ((W_gate_up, "W_gate_up"), (S_gate_up, "S_gate_up"), (W_down, "W_down"), (S_down, "S_down")):
        _check(t, n, torch.uint8, 3, dev)
    T, H = x.shape
    E = router_logits.shape[1]
    Ew = E + n_shared
    I = W_down.shape[2] * 2
    if router_logits.shape[0] != T:
        raise ValueError("router_logits must be [T, E]")
    if (W_gate_up.shape != (Ew, 2 * I, H // 2) or S_gate_up.shape != (Ew, 2 * I, H // 32)
            or W_down.shape != (Ew, H, I // 2) or S_down.shape != (Ew, H, I // 32)):
        raise ValueError("expert weight shapes do not match [E, 2I, H/2], [E, 2I, H/32], [E, H, I/2], [E, H, I/32] "
                         "with E routed + n_shared shared experts")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, 2, dev)
    if ws is None:
        ws = workspace(T, H, I, Ew, top_k + n_shared, dev)
    _check(ws, "workspace", torch.uint8, 1, dev)
    if persistent and (n_shared or act8):
        raise ValueError("the single-launch layer has neither shared experts nor MXFP8 activations")
    if n_shared or act8:
        name = "moe_mxfp4_forward_a8" if act8 else "moe_mxfp4_forward_shared"
        st = getattr(_lib, name)(_ptr(x), _ptr(router_logits), top_k, n_shared, _ptr(W_gate_up), _ptr(S_gate_up),
                                 _ptr(W_down), _ptr(S_down), _ptr(out), T, H, I, E, _ptr(ws), ws.numel(),
                                 _stream(dev))
    else:
        name = "moe_mxfp4_forward_persistent" if persistent else "moe_mxfp4_forward"
        st = getattr(_lib, name)(_ptr(x), _ptr(router_logits), top_k, _ptr(W_gate_up), _ptr(S_gate_up),
                                 _ptr(W_down), _ptr(S_down), _ptr(out), T, H, I, E, _ptr(ws), ws.numel(),
                                 _stream(dev))
    _raise(st, name)
    if persistent and check and not torch.cuda.is_current_stream_capturing():
        raise_for_persistent_error(take_persistent_error(ws))
    return out
