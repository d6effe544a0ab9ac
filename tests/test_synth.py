"""Seeded input generator and router shaping (CPU only).

Checks: bf16 rounding against torch's own float32->bfloat16 conversion (round
to nearest even); reproducibility by seed and the batch-prefix property; the
stored h files equal the oracle's h; on every workload the oracle's logits
select exactly the intended experts with all top-k gaps >= 1e-2; the hot
workload puts exactly 16 tokens on each of 32 experts; expected distinct
expert counts for the natural and Zipf workloads.
"""
import numpy as np
import pytest
import torch

from synth import gen, routing
from tests import workload


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 1, 100000), rng.normal(0, 1e-30, 1000),
                        rng.normal(0, 1e30, 1000)]).astype(np.float32)
    # exact halfway cases: 1 + 2^-8 (ties to even -> 1), 1 + 3*2^-8 (-> 1 + 2^-6)
    v = np.concatenate([v, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)])
    ours = gen.f32_to_bf16_bits(v)
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert list(ours[-3:]) == [0x3F80, 0x3F82, 0xBF80]


def test_seeded_and_batch_prefix():
    a, b = gen.draw(0), gen.draw(0)
    for key in ("x", "attn", "resid", "w_qkv", "w_o", "gain", "router_noise", "s1", "s3", "s2"):
        assert np.array_equal(getattr(a, key), getattr(b, key))
    assert np.array_equal(a.expert(3)[2], b.expert(3)[2])
    c = gen.draw(0, seed=5)
    assert not np.array_equal(a.w_qkv, c.w_qkv)
    big = gen.draw(2)
    small = gen.draw(2, batch=3)
    assert np.array_equal(big.x[:3], small.x) and np.array_equal(big.resid[:3], small.resid)
    assert small.x.shape == (3, 7168)


def test_distributions():
    r = gen.draw(1)
    w = gen.bf16_bits_to_f32(r.w_qkv).astype(np.float64)
    assert abs(w.std() - 0.02) < 5e-4 and abs(w.mean()) < 5e-4
    g = gen.bf16_bits_to_f32(r.gain).astype(np.float64)
    assert abs(g.mean() - 1.0) < 5e-3 and abs(g.std() - 0.1) < 5e-3
    assert abs(r.resid.std() - 1.0) < 0.05


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_stored_h_matches_oracle(cfg):
    raw = gen.draw(cfg)
    h = workload.oracle_h(raw)
    st = routing.stored_h(cfg)
    assert st.dtype == np.float32 and st.shape == h.shape
    assert np.max(np.abs(st - h)) <= 1e-6 * np.max(np.abs(h))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_routing_targets_and_margins(cfg):
    layer = workload.build(cfg, h_source="stored")
    out = workload.expected(layer)
    k = layer.shape.top_k
    assert np.array_equal(out["topk_idx"], layer.targets)
    gaps = workload.logit_gaps(out["logits"], k)
    assert np.all(gaps >= 1e-2), gaps.min()
    n_distinct = len(layer.touched_experts())
    if cfg == 3:
        load = layer.expert_load()
        assert sorted(load[load > 0]) == [16] * 32
    if cfg == 2:
        assert 50 <= n_distinct <= 64
    if cfg == 4:
        assert 25 <= n_distinct <= 60
    if cfg == 1:
        assert n_distinct == 8
