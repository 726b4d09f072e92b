"""bench.py's host-side contract, on the CPU: the one-GPU refusal, and the workload names it
times (the MoE configurations, the T sweep and the dense layer configurations)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthetic  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name", sorted(synthetic.MOE_CONFIGS))
def test_moe_workloads_resolve(name):
    assert bench.workload_config(name) is synthetic.MOE_CONFIGS[name]


@pytest.mark.parametrize("T", [1, 2, 3, 8, 16, 24, 64])
def test_sweep_workloads_resolve(T):
    cfg = bench.workload_config(f"moe_sweep_t{T}")
    assert cfg.T == T and (cfg.H, cfg.I, cfg.E, cfg.k) == (7168, 2048, 256, 8)


def test_unknown_workload_exits():
    with pytest.raises(SystemExit):
        bench.workload_config("no_such_workload")


def test_dense_workloads_are_the_dense_configurations():
    # the dense mode is chosen by name before the MoE configurations are looked up
    assert set(synthetic.LINEAR_CONFIGS) == {"dense_t1", "dense_t4"}
    c1, c4 = synthetic.LINEAR_CONFIGS["dense_t1"], synthetic.LINEAR_CONFIGS["dense_t4"]
    assert (c1.T, c1.K, c1.N) == (1, 2048, 2048) and (c4.T, c4.K, c4.N) == (4, 7168, 4096)


def test_default_workload_is_the_t32_zipf_layer(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert args.workload == "moe_t32_zipf" and args.gpus == 1
    assert args.steps > 0 and args.warmup > 0
