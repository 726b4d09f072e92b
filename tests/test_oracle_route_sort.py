"""Pins of the oracle's router (top-k + softmax over the selected logits) and
its token->expert counting sort, against numpy / scipy library routines."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synthetic


def np_topk(logits, k):
    T, E = logits.shape
    out = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))  # logit desc, id asc
        out[t] = order[:k]
    return out


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (4, 256, 8), (7, 384, 8), (5, 16, 16), (3, 5, 1)])
def test_route_matches_lexsort_and_softmax(T, E, k):
    logits = np.random.default_rng(T * E + k).standard_normal((T, E)).astype(np.float32)
    ids, gates = oracle.route(logits, k)
    assert np.array_equal(ids, np_topk(logits, k))
    ref = softmax(logits[np.arange(T)[:, None], ids].astype(np.float64), axis=1)
    assert np.allclose(gates, ref, rtol=2 ** -23, atol=0)
    assert np.all(np.abs(gates.astype(np.float64).sum(1) - 1) <= 1e-6)
    assert np.all(np.diff(gates, axis=1) <= 0)  # slots in descending-logit order


def test_route_ties_go_to_lower_id():
    logits = np.zeros((3, 10), np.float32)
    logits[0, [7, 2, 5]] = 1.0
    logits[1, :] = 0.5
    logits[2, [9, 3]] = [2.0, 2.0]
    ids, gates = oracle.route(logits, 3)
    assert ids[0].tolist() == [2, 5, 7]
    assert ids[1].tolist() == [0, 1, 2]
    assert ids[2].tolist() == [3, 9, 0]
    assert np.allclose(gates[1], 1 / 3, rtol=1e-7)


def test_route_k1_gate_is_one():
    logits = np.random.default_rng(0).standard_normal((6, 40)).astype(np.float32)
    ids, gates = oracle.route(logits, 1)
    assert np.all(gates == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))


def test_uniform_logits_config_routes():
    cfg = synthetic.MoEConfig("u", T=16, H=64, I=32, E=384, k=8, routing="uniform")
    logits = synthetic.router_logits(cfg)
    ids, _ = oracle.route(logits, 8)
    assert np.array_equal(ids, np_topk(logits, 8))


def test_zipf_generator_topk_is_drawn_set():
    cfg = synthetic.MoEConfig("z", T=32, H=64, I=32, E=256, k=8, routing="zipf")
    logits = synthetic.router_logits(cfg)
    ids, _ = oracle.route(logits, 8)
    for t in range(32):
        assert set(ids[t].tolist()) == set(np.nonzero(logits[t] > 8.0)[0].tolist())


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (4, 256, 8), (32, 256, 8), (128, 384, 8), (3, 4, 4), (9, 7, 2)])
def test_sort_matches_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    r = oracle.sort(ids, E)
    flat = ids.ravel()
    assert np.array_equal(r["sorted_slots"], np.argsort(flat, kind="stable"))
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(r["counts"], counts)
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    act = np.nonzero(counts)[0]  # the active experts, ascending
    assert r["num_active"] == act.size
    assert np.array_equal(r["active"][: act.size], act) and np.all(r["active"][act.size:] == -1)


def test_expected_active_experts_uniform():
    # E (1 - (1 - k/E)^T) distinct experts for independent uniform tokens.
    cfg = synthetic.MoEConfig("u", T=128, H=64, I=32, E=384, k=8, routing="uniform")
    ids, _ = oracle.route(synthetic.router_logits(cfg), 8)
    na = oracle.sort(ids, 384)["num_active"]
    expect = 384 * (1 - (1 - 8 / 384) ** 128)
    assert abs(na - expect) < 15
