"""moe_mxfp4_forward_noalloc (scratch in a static device array, no workspace argument),
called through the C ABI, against moe_mxfp4_forward with a workspace: two calls in a row,
the second with a smaller input than the first, each bit for bit the workspace call's
result and within the oracle's MoE bound.  Also the rejection of sizes beyond the
array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_helpers import MOE_REL, check_bound, say, to_dev_bf16, to_host_bits

pytestmark = pytest.mark.gpu
CTL_BYTES = 57344  # MX_WORKSPACE_CTL_BYTES


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import mxfp4_weight_moe_amd
    return mxfp4_weight_moe_amd


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def inputs(cfg, dev, host):
    if host is None:
        d = synthetic.moe_weights_device(cfg, dev)
        x, logits = synthetic.moe_activations(cfg)
        w_host = {k: d[k].cpu().numpy() for k in ("wgu", "sgu", "wd", "sd")}
    else:
        d = {k: torch.from_numpy(host[k]).to(dev) for k in ("wgu", "sgu", "wd", "sd")}
        x, logits, w_host = host["x"], host["logits"], host
    d["x"] = to_dev_bf16(x, dev)
    d["logits"] = torch.from_numpy(logits).to(dev)
    return d, x, logits, w_host


def forward_noalloc(mx, d, k):
    T, H = d["x"].shape
    E = d["logits"].shape[1]
    I = d["wd"].shape[2] * 2
    y = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=d["x"].device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = mx.raw().moe_mxfp4_forward_noalloc(_p(d["x"]), _p(d["logits"]), k, _p(d["wgu"]), _p(d["sgu"]), _p(d["wd"]),
                                            _p(d["sd"]), _p(y), T, H, I, E, stream)
    assert st == 0, mx.status_string(st)
    return y


def forward_workspace(mx, d, k):
    T, H = d["x"].shape
    E = d["logits"].shape[1]
    I = d["wd"].shape[2] * 2
    dev = d["x"].device
    ws = torch.zeros(mx.workspace_size(T, H, I, E, k), dtype=torch.uint8, device=dev)
    ws[CTL_BYTES:] = 0xFF
    y = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
    mx.moe_mxfp4_forward(d["x"], d["logits"], k, d["wgu"], d["sgu"], d["wd"], d["sd"], out=y, ws=ws)
    return y


def test_noalloc_forward_matches_the_workspace_forward_twice(mx):
    dev = torch.device("cuda:0")
    small = synthetic.MoEConfig("noalloc_small", T=3, H=1024, I=1024, E=8, k=2, routing="normal", e_lo=-8, e_hi=-2,
                                seed=31)
    cases = [(synthetic.MOE_CONFIGS["moe_t32_zipf"], None), (small, synthetic.moe_inputs_host(small))]
    for cfg, host in cases:
        say("noalloc forward", cfg.name, "T =", cfg.T)
        d, x, logits, w_host = inputs(cfg, dev, host)
        y_na = forward_noalloc(mx, d, cfg.k)
        y_ws = forward_workspace(mx, d, cfg.k)
        torch.cuda.synchronize()
        got = to_host_bits(y_na)
        assert np.array_equal(got, to_host_bits(y_ws)), f"{cfg.name}: noalloc differs from the workspace forward"
        yo, sm, _ = oracle.moe_tokens(x, logits, cfg.k, w_host["wgu"], w_host["sgu"], w_host["wd"], w_host["sd"],
                                      cfg.T, cfg.H, cfg.I, cfg.E)
        worst = check_bound(got, yo, sm, MOE_REL, f"noalloc {cfg.name}")
        say(f"  worst ratio {worst:.3g}")
        del d


def test_noalloc_rejects_sizes_beyond_its_scratch(mx):
    L = mx.raw()
    A = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: the call fails its size check first
    need = mx.workspace_size(256, 7168, 2048, 1024, 32)
    assert need > mx.MX_NOALLOC_SCRATCH_BYTES
    assert L.moe_mxfp4_forward_noalloc(A, A, 32, A, A, A, A, A, 256, 7168, 2048, 1024, None) == mx.MX_ERR_SCRATCH
    assert mx.workspace_size(128, 7168, 2048, 384, 8) <= mx.MX_NOALLOC_SCRATCH_BYTES
