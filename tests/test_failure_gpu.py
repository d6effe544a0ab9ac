"""Failure behaviour of the single-launch path, forced from the host.

* An expired hand-off wait: the handle's spin limit is set to 0, so every wait
  of the persistent kernel gives up at its first unsatisfied poll and every
  kernel still finishes normally (no wait is left unbounded, nothing is made
  to fault).  The step must report status bit 0 and write NaN (topk_idx -1)
  into the outputs computed from values it did not receive; qkv and
  resid_out depend on no hand-off and must still match the oracle.  With the
  default limit restored the same handle must step correctly again.
* The 32-bit step counter's wrap: the counter is set just below 2^32 from the
  host; the steps across the wrap (the last one clears the hand-off slots)
  must match the oracle, including a batch-8 step whose tag after the wrap
  equals the tag of an earlier batch-8 step made with other inputs.
"""
import numpy as np
import pytest
import torch

from synth import device as sdev, gen, routing
from tests import parity, workload
from tests.parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_moe_amd  # noqa: F401


def _got(out):
    return {"qkv": out.qkv.cpu().numpy(), "resid_out": out.resid_out.cpu().numpy(),
            "logits": out.router_logits.cpu().numpy(), "topk_idx": out.topk_idx.cpu().numpy(),
            "topk_w": out.topk_w.cpu().numpy(), "moe_out": out.moe_out.cpu().numpy(), "h": None}


def test_expired_waits_poison_the_outputs():
    say("[wait expiry: spin limit 0, TP16 shard batch 8, single path] start")
    from decode_step_moe_amd import DecodeLayer
    layer = workload.build(2, h_source="stored")
    ref = workload.expected(layer)
    obj = DecodeLayer(sdev.config_of(layer), sdev.upload_weights(layer))
    assert obj.single_max_batch == 8
    x, attn, resid = sdev.upload_inputs(layer)
    obj.set_spin_limit(0)
    out = obj.step(x, attn, resid)
    torch.cuda.synchronize()
    st = obj.status(clear=True)
    got = _got(out)
    say(f"[wait expiry] status {st:#x}, non-finite moe_out {np.mean(~np.isfinite(got['moe_out'])):.3f}, "
        f"topk_idx -1 {np.mean(got['topk_idx'] == -1):.3f}")
    assert st & 1, "no wait expired with a spin limit of 0"
    assert not np.all(np.isfinite(got["moe_out"])), "an expired wait left moe_out finite"
    idx = got["topk_idx"]
    assert np.all((idx == -1) | ((idx >= 0) & (idx < layer.shape.n_experts)))
    assert np.all(np.isnan(got["topk_w"][idx == -1]))
    for key in ("qkv", "resid_out"):   # no hand-off feeds these
        assert parity.rel_l2(got[key], ref[key]) <= parity.OUT_REL_L2, key
        assert parity.max_abs(got[key], ref[key]) <= parity.OUT_MAX_ABS, key
    # the default limit again: the handle recovers
    obj.set_spin_limit(1 << 20)
    out = obj.step(x, attn, resid)
    torch.cuda.synchronize()
    assert obj.status() == 0
    m = parity.compare(_got(out), ref)
    assert not m["fails"], m["fails"]


def test_debug_mode_raises_on_an_expired_wait():
    say("[debug mode with spin limit 0, TP16 shard batch 1] start")
    from decode_step_moe_amd import DecodeLayer, DecodeLayerError
    layer = workload.build(1, h_source="stored")
    obj = DecodeLayer(sdev.config_of(layer), sdev.upload_weights(layer), debug=True)
    x, attn, resid = sdev.upload_inputs(layer)
    obj.step(x, attn, resid)               # default limit: no error
    obj.set_spin_limit(0)
    with pytest.raises(DecodeLayerError):
        obj.step(x, attn, resid)
    obj.set_spin_limit(1 << 20)
    obj.step(x, attn, resid)               # the status word was cleared by the raise


def test_step_counter_wraps():
    say("[step counter wrap, TP16 shard batches 8 and 1, single path] start")
    from decode_step_moe_amd import DecodeLayer
    full = workload.build(2, h_source="stored")
    ref8 = workload.expected(full)
    obj = DecodeLayer(sdev.config_of(full), sdev.upload_weights(full))
    x, attn, resid = sdev.upload_inputs(full)
    # step with tag 1 on other inputs (residual scaled): slots of all 8 tokens
    # now hold tag-1 values that are wrong for the real inputs
    junk = obj.step(x, attn, resid * 1000.0)
    torch.cuda.synchronize()
    one = routing.RoutedLayer(gen.draw(2, batch=1), full.w_router, full.targets[:1],
                              full.target_logits[:1])
    ref1 = workload.expected(one)
    x1, a1, r1 = sdev.upload_inputs(one)
    obj.set_step_counter(0xFFFFFFFD)
    for tag, (layer_x, ref, B) in zip((0xFFFFFFFE, 0xFFFFFFFF, 1, 2),
                                      [((x1, a1, r1), ref1, 1), ((x1, a1, r1), ref1, 1),
                                       ((x, attn, resid), ref8, 8), ((x, attn, resid), ref8, 8)]):
        say(f"[wrap] step with tag {tag:#x}, batch {B}")
        out = obj.step(*layer_x)
        torch.cuda.synchronize()
        m = parity.compare(_got(out), ref)
        assert not m["fails"], (hex(tag), m["fails"])
    assert obj.status() == 0
    del junk
