"""The correlated speculative-verify routing workload against the numbers it is built from.

AMD megakernel blog ("Bringing Ultra-Fast, Interactive LLM Inference to AMD Instinct MI355X
GPUs"), section "4. Data Locality": a verification pass over 4 tokens of one request reads
the union of about 11.7 experts per layer, against 7 for 2 tokens.  The generator gives each
request an expert preference shared by its positions; routed with the oracle, a request's
4 positions must reach about 11.7 / 7 = 1.67 times the distinct experts of 2 positions
(independent tokens: about 1.95).  The page does not state its model's expert count or
top-k; at 128 experts and top-4 the generator also lands near the page's absolute counts.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synthetic

PAGE_RATIO = 11.7 / 7.0
REQUESTS = 600


def unions(E, k, routing, seed=5):
    cfg = synthetic.MoEConfig("spec_pin", T=REQUESTS * 4, H=64, I=32, E=E, k=k, routing=routing, positions=4,
                              seed=seed)
    ids, _ = oracle.route(synthetic.router_logits(cfg), k)
    ids = ids.reshape(REQUESTS, 4, k)
    u2 = np.mean([len(np.unique(ids[r, :2])) for r in range(REQUESTS)])
    u4 = np.mean([len(np.unique(ids[r])) for r in range(REQUESTS)])
    return u2, u4


@pytest.mark.parametrize("E", [256, 384])
def test_spec_union_ratio_matches_page(E):
    u2, u4 = unions(E, 8, "spec")
    assert abs(u4 / u2 - PAGE_RATIO) <= 0.04 * PAGE_RATIO, (u2, u4)


def test_independent_tokens_do_not_match():
    u2, u4 = unions(256, 8, "normal")
    assert u4 / u2 > 1.9  # the page's overlap comes from the shared preference, not from chance


def test_spec_absolute_unions_at_128_experts_top4():
    u2, u4 = unions(128, 4, "spec")
    assert abs(u2 - 7.0) <= 0.35 and abs(u4 - 11.7) <= 0.6, (u2, u4)


def test_spec_positions_share_a_request():
    cfg = synthetic.MOE_CONFIGS["moe_spec_t128"]
    assert cfg.T == 32 * cfg.positions and cfg.positions == 4
    lg = synthetic.router_logits(cfg)
    other = synthetic.router_logits(replace(cfg, seed=cfg.seed + 1))
    assert lg.shape == (cfg.T, cfg.E) and lg.dtype == np.float32
    assert not np.array_equal(lg, other)
    # positions of one request are correlated, positions of different requests are not
    same = np.corrcoef(lg[0], lg[1])[0, 1]
    diff = np.corrcoef(lg[0], lg[4])[0, 1]
    assert same > 0.4 and abs(diff) < 0.2


def test_activations_are_the_nearest_bf16_of_a_normal_draw():
    """x is bf16_rne(N(0,1)): the generator's rounding of each fp32 draw agrees with torch's
    round-to-nearest-even cast."""
    import torch
    b = synthetic.bf16_bits_normal((4096,), 3)
    f = synthetic._rng(3, synthetic.TAG_X).standard_normal(size=(4096,), dtype=np.float32)
    assert np.array_equal(b, torch.from_numpy(f).bfloat16().view(torch.int16).numpy().view(np.uint16))
