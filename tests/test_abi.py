"""The C-ABI library loads without a GPU, exports exactly what include/mxmoe.h declares,
and rejects bad arguments on the host before anything is enqueued.

Every call here fails a host-side check, so no kernel is ever launched."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxmoe.h")

m = pytest.importorskip("mxfp4_weight_moe_amd")

MX_OK, MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_WORKSPACE, MX_ERR_HIP = 0, -1, -2, -3, -4, -5


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"MX_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)))


def test_exports_match_header():
    decl = declared_functions()
    assert decl == sorted(m.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == decl
    lib = m.raw()
    for name in decl:
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = '#include "mxmoe.h"\nint main(void){return mx_version() > 0 ? 0 : 1;}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.dirname(HEADER), "-x", "c", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    for st in (MX_OK, MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_WORKSPACE, MX_ERR_HIP, 7):
        assert isinstance(m.status_string(st), str) and m.status_string(st)
    assert m.version() >= 100


P = ctypes.c_void_p
A = P(1 << 20)        # aligned fake pointer (never dereferenced: every call below fails a check)
MIS = P((1 << 20) + 4)


def test_mx_linear_rejects():
    L = m.raw()
    assert L.mx_linear(None, A, A, A, 1, 64, 16, None) == MX_ERR_NULL
    assert L.mx_linear(A, A, A, A, 0, 64, 16, None) == MX_ERR_SHAPE
    assert L.mx_linear(A, A, A, A, 1, 48, 16, None) == MX_ERR_SHAPE
    assert L.mx_linear(A, A, A, A, 1, 0, 16, None) == MX_ERR_SHAPE
    assert L.mx_linear(A, A, A, A, 1, 64, 0, None) == MX_ERR_SHAPE
    assert L.mx_linear(MIS, A, A, A, 1, 64, 16, None) == MX_ERR_ALIGN
    assert L.mx_linear(A, MIS, A, A, 1, 64, 16, None) == MX_ERR_ALIGN
    assert L.mx_linear(A, A, MIS, A, 1, 256, 16, None) == MX_ERR_ALIGN
    assert L.mx_linear(A, A, A, P((1 << 20) + 2), 1, 64, 16, None) == MX_ERR_ALIGN


def test_mxfp8_entry_points_reject():
    L = m.raw()
    assert L.mx_linear_a8(None, A, A, A, 1, 64, 16, None) == MX_ERR_NULL
    assert L.mx_linear_a8(A, A, A, A, 1, 48, 16, None) == MX_ERR_SHAPE
    assert L.mx_linear_a8(A, A, A, A, 0, 64, 16, None) == MX_ERR_SHAPE
    assert L.mx_linear_a8(MIS, A, A, A, 1, 64, 16, None) == MX_ERR_ALIGN
    assert L.mx_linear_a8(A, A, MIS, A, 1, 256, 16, None) == MX_ERR_ALIGN
    assert L.mxfp8_quantize(None, 1, 32, A, A, None) == MX_ERR_NULL
    assert L.mxfp8_quantize(A, 1, 48, A, A, None) == MX_ERR_SHAPE
    assert L.mxfp8_quantize(A, 0, 32, A, A, None) == MX_ERR_SHAPE
    assert L.mxfp8_quantize(MIS, 1, 32, A, A, None) == MX_ERR_ALIGN
    assert L.mxfp8_quantize(A, 1, 32, MIS, A, None) == MX_ERR_ALIGN
    ws = m.workspace_size(4, 1024, 1024, 9, 3)

    def fwd(k=2, ns=1, T=4, E=8, H=1024, I=1024, w=A, wb=ws, x=A):
        return L.moe_mxfp4_forward_a8(x, A, k, ns, A, A, A, A, A, T, H, I, E, w, wb, None)

    assert fwd(x=None) == MX_ERR_NULL
    assert fwd(T=0) == MX_ERR_SHAPE
    assert fwd(ns=-1) == MX_ERR_SHAPE
    assert fwd(I=320) == MX_ERR_SHAPE
    assert fwd(x=MIS) == MX_ERR_ALIGN
    assert fwd(wb=ws - 1) == MX_ERR_WORKSPACE


def test_dequant_rejects():
    L = m.raw()
    assert L.mxfp4_dequantize(None, A, 1, 32, A, None) == MX_ERR_NULL
    assert L.mxfp4_dequantize(A, A, 0, 32, A, None) == MX_ERR_SHAPE
    assert L.mxfp4_dequantize(A, A, 1, 33, A, None) == MX_ERR_SHAPE
    assert L.mxfp4_dequantize(MIS, A, 1, 32, A, None) == MX_ERR_ALIGN


def test_route_and_sort_reject():
    L = m.raw()
    assert L.moe_route_topk(None, 1, 8, 2, A, A, None) == MX_ERR_NULL
    assert L.moe_route_topk(A, 0, 8, 2, A, A, None) == MX_ERR_SHAPE
    assert L.moe_route_topk(A, 257, 8, 2, A, A, None) == MX_ERR_SHAPE
    assert L.moe_route_topk(A, 1, 8, 9, A, A, None) == MX_ERR_SHAPE
    assert L.moe_route_topk(A, 1, 1025, 2, A, A, None) == MX_ERR_SHAPE
    assert L.moe_route_topk(A, 1, 64, 33, A, A, None) == MX_ERR_SHAPE
    assert L.moe_route_topk(P((1 << 20) + 2), 1, 8, 2, A, A, None) == MX_ERR_ALIGN
    assert L.moe_sort_by_expert(A, 1, 2, 8, A, A, A, A, None, None) == MX_ERR_NULL
    assert L.moe_sort_by_expert(A, 1, 0, 8, A, A, A, A, A, None) == MX_ERR_SHAPE
    assert L.moe_route_sort(A, 1, 8, 2, A, A, A, A, A, A, None, None) == MX_ERR_NULL
    assert L.moe_route_sort(A, 0, 8, 2, A, A, A, A, A, A, A, None) == MX_ERR_SHAPE
    assert L.moe_route_sort(A, 1, 8, 9, A, A, A, A, A, A, A, None) == MX_ERR_SHAPE
    assert L.moe_route_sort(P((1 << 20) + 2), 1, 8, 2, A, A, A, A, A, A, A, None) == MX_ERR_ALIGN


def test_forward_rejects():
    L = m.raw()
    ws = m.workspace_size(4, 1024, 1024, 8, 2)
    assert ws > 0 and ws % 256 == 0

    def fwd(x=A, lg=A, k=2, wgu=A, sgu=A, wd=A, sd=A, y=A, T=4, H=1024, I=1024, E=8, w=A, wb=ws):
        return L.moe_mxfp4_forward(x, lg, k, wgu, sgu, wd, sd, y, T, H, I, E, w, wb, None)

    assert fwd(x=None) == MX_ERR_NULL
    assert fwd(sd=None) == MX_ERR_NULL
    assert fwd(T=0) == MX_ERR_SHAPE
    assert fwd(T=257) == MX_ERR_SHAPE
    assert fwd(k=9) == MX_ERR_SHAPE
    assert fwd(H=320) == MX_ERR_SHAPE
    assert fwd(H=1536) == MX_ERR_SHAPE  # not a multiple of 1024
    assert fwd(I=96) == MX_ERR_SHAPE
    assert fwd(I=128) == MX_ERR_SHAPE   # below 256
    assert fwd(I=320) == MX_ERR_SHAPE   # not a multiple of 256
    # I = 256 and 768 pass the shape checks (the header's I % 256 == 0): they fail at the
    # workspace check that follows, since the workspace below is sized for I = 1024
    small = m.workspace_size(4, 1024, 256, 8, 2) - 1
    assert fwd(I=256, wb=small) == MX_ERR_WORKSPACE
    assert fwd(I=768, wb=m.workspace_size(4, 1024, 768, 8, 2) - 1) == MX_ERR_WORKSPACE
    assert fwd(H=2048, I=256, wb=m.workspace_size(4, 2048, 256, 8, 2) - 1) == MX_ERR_WORKSPACE
    assert fwd(wgu=MIS) == MX_ERR_ALIGN
    assert fwd(sgu=P((1 << 20) + 4)) == MX_ERR_ALIGN
    assert fwd(sd=P((1 << 20) + 8)) == MX_ERR_ALIGN
    assert fwd(w=None) == MX_ERR_WORKSPACE
    assert fwd(w=P((1 << 20) + 128)) == MX_ERR_WORKSPACE
    assert fwd(wb=ws - 1) == MX_ERR_WORKSPACE


def test_stage_gemm_hooks_reject():
    L = m.raw()
    ws = m.workspace_size(4, 1024, 1024, 8, 2)

    def gu(x=A, h=A, T=4, H=1024, I=1024, E=8, k=2, w=A, wb=ws):
        return L.moe_gate_up_swiglu(x, A, A, A, A, A, A, A, h, T, H, I, E, k, w, wb, None)

    assert gu(x=None) == MX_ERR_NULL
    assert gu(h=None) == MX_ERR_NULL
    assert gu(T=0) == MX_ERR_SHAPE
    assert gu(H=1536) == MX_ERR_SHAPE
    assert gu(x=MIS) == MX_ERR_ALIGN
    assert gu(w=None) == MX_ERR_WORKSPACE
    assert gu(w=P((1 << 20) + 128)) == MX_ERR_WORKSPACE
    assert gu(wb=ws - 1) == MX_ERR_WORKSPACE

    def gi(x=A, ids=A, h=A, T=4, H=1024, I=1024, E=8, k=2, w=A, wb=ws):
        return L.moe_gate_up_swiglu_from_ids(x, ids, A, A, A, A, A, A, A, h, T, H, I, E, k, w, wb, None)

    assert gi(ids=None) == MX_ERR_NULL
    assert gi(h=None) == MX_ERR_NULL
    assert gi(T=0) == MX_ERR_SHAPE
    assert gi(T=33, E=64) == MX_ERR_SHAPE  # the in-launch sort holds one 32-bit token mask per expert
    assert gi(T=32, k=9, E=64) == MX_ERR_SHAPE  # at most 256 slots
    assert gi(H=1536) == MX_ERR_SHAPE
    assert gi(ids=P((1 << 20) + 2)) == MX_ERR_ALIGN
    assert gi(x=MIS) == MX_ERR_ALIGN
    assert gi(w=None) == MX_ERR_WORKSPACE
    assert gi(wb=ws - 1) == MX_ERR_WORKSPACE

    ws32 = m.workspace_size(32, 1024, 1024, 64, 8)

    def eg(x=A, ids=A, h=A, d=A, T=32, H=1024, I=1024, E=64, k=8, w=A, wb=ws32):
        return L.moe_expert_gemms_from_ids(x, ids, A, A, A, A, h, 0, d, T, H, I, E, k, w, wb, None)

    assert eg(ids=None) == MX_ERR_NULL
    assert eg(h=None) == MX_ERR_NULL
    assert eg(d=None) == MX_ERR_NULL
    assert eg(T=0) == MX_ERR_SHAPE
    assert eg(T=33) == MX_ERR_SHAPE          # the in-launch sort holds one 32-bit token mask per expert
    assert eg(k=9) == MX_ERR_SHAPE           # at most 256 slots
    assert eg(I=768) == MX_ERR_SHAPE         # down's reduction in 4-segment scale runs
    assert eg(E=1025) == MX_ERR_SHAPE
    assert eg(H=1536) == MX_ERR_SHAPE
    assert eg(h=P((1 << 20) + 8)) == MX_ERR_ALIGN
    assert eg(d=P((1 << 20) + 4)) == MX_ERR_ALIGN
    assert eg(ids=P((1 << 20) + 2)) == MX_ERR_ALIGN
    assert eg(w=None) == MX_ERR_WORKSPACE
    assert eg(w=P((1 << 20) + 128)) == MX_ERR_WORKSPACE
    assert eg(wb=ws32 - 1) == MX_ERR_WORKSPACE

    def cb(d=A, g=A, y=A, T=4, H=1024, k=2):
        return L.moe_combine(d, g, y, T, H, k, None)

    assert cb(d=None) == MX_ERR_NULL
    assert cb(g=None) == MX_ERR_NULL
    assert cb(T=0) == MX_ERR_SHAPE
    assert cb(T=257) == MX_ERR_SHAPE
    assert cb(k=33) == MX_ERR_SHAPE
    assert cb(H=1026) == MX_ERR_SHAPE
    assert cb(d=P((1 << 20) + 8)) == MX_ERR_ALIGN
    assert cb(y=P((1 << 20) + 4)) == MX_ERR_ALIGN

    def dn(h=A, y=A, T=4, w=A, wb=ws):
        return L.moe_down_combine(h, A, A, A, A, A, A, A, A, y, T, 1024, 1024, 8, 2, w, wb, None)

    assert dn(y=None) == MX_ERR_NULL
    assert dn(T=300) == MX_ERR_SHAPE
    assert dn(w=None) == MX_ERR_WORKSPACE
    assert dn(wb=ws - 1) == MX_ERR_WORKSPACE


def test_shared_forward_rejects():
    L = m.raw()
    ws = m.workspace_size(4, 1024, 1024, 9, 3)  # E + n_shared experts, top_k + n_shared slots

    def fwd(k=2, ns=1, T=4, E=8, w=A, wb=ws, x=A):
        return L.moe_mxfp4_forward_shared(x, A, k, ns, A, A, A, A, A, T, 1024, 1024, E, w, wb, None)

    assert fwd(x=None) == MX_ERR_NULL
    assert fwd(ns=-1) == MX_ERR_SHAPE
    assert fwd(E=1024) == MX_ERR_SHAPE        # 1025 experts with the shared one
    assert fwd(k=32, E=64) == MX_ERR_SHAPE    # 33 slots per token
    assert fwd(wb=ws - 1) == MX_ERR_WORKSPACE
    assert fwd(wb=m.workspace_size(4, 1024, 1024, 8, 2)) == MX_ERR_WORKSPACE  # sized without the shared slots


def test_persistent_forward_rejects():
    L = m.raw()
    ws = m.workspace_size(16, 1024, 1024, 64, 8)

    def fwd(x=A, lg=A, k=2, wgu=A, sgu=A, wd=A, sd=A, y=A, T=4, H=1024, I=1024, E=8, w=A, wb=ws):
        return L.moe_mxfp4_forward_persistent(x, lg, k, wgu, sgu, wd, sd, y, T, H, I, E, w, wb, None)

    assert fwd(lg=None) == MX_ERR_NULL
    assert fwd(T=0) == MX_ERR_SHAPE
    assert fwd(T=17) == MX_ERR_SHAPE           # beyond the single-launch limit of 16 tokens
    assert fwd(T=16, k=9, E=64) == MX_ERR_SHAPE  # 144 > 128 routed slots
    assert fwd(T=4, k=33, E=64) == MX_ERR_SHAPE
    assert fwd(H=1536) == MX_ERR_SHAPE
    assert fwd(I=256) == MX_ERR_SHAPE          # the single launch needs I % 1024 == 0
    assert fwd(x=MIS) == MX_ERR_ALIGN
    assert fwd(w=None) == MX_ERR_WORKSPACE
    assert fwd(wb=m.workspace_size(4, 1024, 1024, 8, 2) - 1) == MX_ERR_WORKSPACE


def test_workspace_size_grows_with_tokens():
    a = m.workspace_size(1, 7168, 2048, 256, 8)
    b = m.workspace_size(128, 7168, 2048, 384, 8)
    assert 0 < a < b
    assert m.workspace_size(0, 7168, 2048, 256, 8) == 0


def test_header_states_the_checked_limits():
    """The header's stated MoE limits are the ones the library checks (above)."""
    src = open(HEADER).read()
    assert "I % 256 == 0" in src and "H % 1024 == 0" in src
    assert "I % 1024 == 0 (both" not in src


def test_hbm_reference_kernels_reject():
    L = m.raw()
    assert L.mx_hbm_read(None, 64, A, None) == MX_ERR_NULL
    assert L.mx_hbm_read(A, 0, A, None) == MX_ERR_SHAPE
    assert L.mx_hbm_read(A, 72, A, None) == MX_ERR_SHAPE
    assert L.mx_hbm_read(MIS, 64, A, None) == MX_ERR_ALIGN
    assert L.mx_hbm_copy(A, None, 64, None) == MX_ERR_NULL
    assert L.mx_hbm_copy(A, A, 8, None) == MX_ERR_SHAPE
    assert L.mx_hbm_copy(MIS, A, 64, None) == MX_ERR_ALIGN


def test_persistent_error_word_raises():
    """The binding turns the single-launch layer's sticky error word into an exception."""
    m.raise_for_persistent_error(0)
    with pytest.raises(m.MxWaitError):
        m.raise_for_persistent_error(1)
    assert m.PERSISTENT_ERROR_OFFSET == 8


def test_noalloc_forward_rejects():
    """The static-scratch forward checks its arguments like moe_mxfp4_forward and refuses
    sizes whose scratch exceeds its array, all before anything is enqueued."""
    L = m.raw()

    def fwd(x=A, k=2, T=4, H=1024, I=1024, E=8):
        return L.moe_mxfp4_forward_noalloc(x, A, k, A, A, A, A, A, T, H, I, E, None)

    assert fwd(x=None) == MX_ERR_NULL
    assert fwd(T=0) == MX_ERR_SHAPE
    assert fwd(I=320) == MX_ERR_SHAPE
    assert fwd(x=MIS) == MX_ERR_ALIGN
    assert fwd(T=256, k=32, E=1024, H=7168, I=2048) == m.MX_ERR_SCRATCH
    assert m.workspace_size(256, 7168, 2048, 1024, 32) > m.MX_NOALLOC_SCRATCH_BYTES
    assert m.status_string(m.MX_ERR_SCRATCH) != "unknown status"
