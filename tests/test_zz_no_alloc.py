"""decode_layer_step_noalloc (scratch in the library's static device area)
against decode_layer_step on a handle, through the C ABI: two calls in a row,
the second with a smaller batch, on the single-launch path (TP16 shard,
batches 8 then 3) and on the batched path (TP16 shard, max batch 24,
batches 24 then 17).  Both entry points run the same kernels, so the outputs
must be identical bit for bit, and they must match the oracle.
"""
import numpy as np
import pytest
import torch

from synth import device as sdev, gen, routing
from tests import parity, workload
from tests.parity import say

pytestmark = pytest.mark.gpu

KEYS = ("qkv", "resid_out", "router_logits", "topk_idx", "topk_w", "moe_out")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_moe_amd  # noqa: F401


def _prefix(full, b):
    return routing.RoutedLayer(gen.draw(2, batch=b), full.w_router, full.targets[:b], full.target_logits[:b])


@pytest.mark.parametrize("max_batch,batches,path", [(8, (8, 3), 0), (24, (24, 17), 3), (8, (8, 3), 1)])
def test_noalloc_matches_the_handle(max_batch, batches, path):
    import decode_step_moe_amd as dl
    from decode_step_moe_amd import binding
    say(f"[no-alloc vs handle, TP16 shapes, max batch {max_batch}, batches {batches}, path {path}] start")
    full = workload.build(2, batch=max_batch)
    cfg = sdev.config_of(full, max_batch, path=path)
    assert binding.scratch_bytes(cfg, 256) <= binding.noalloc_max_scratch()
    weights = sdev.upload_weights(full)
    obj = dl.DecodeLayer(cfg, weights)
    wc = binding.make_weights(cfg, weights)
    for b in batches:
        layer = _prefix(full, b)
        x, attn, resid = sdev.upload_inputs(layer)
        ref_out = obj.step(x, attn, resid)
        out = binding.alloc_outputs(cfg, b)
        for t in (out.qkv, out.resid_out, out.router_logits, out.topk_w, out.moe_out):
            t.fill_(float("nan"))
        binding.step_noalloc(cfg, wc, binding.make_io(cfg, x, attn, resid, out))
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(getattr(out, k), getattr(ref_out, k)), (b, k)
        got = {"qkv": out.qkv.cpu().numpy(), "resid_out": out.resid_out.cpu().numpy(),
               "logits": out.router_logits.cpu().numpy(), "topk_idx": out.topk_idx.cpu().numpy(),
               "topk_w": out.topk_w.cpu().numpy(), "moe_out": out.moe_out.cpu().numpy(), "h": None}
        m = parity.compare(got, workload.expected(layer))
        say(f"[no-alloc b{b}] " + ", ".join(f"{k}={v:.3e}" for k, v in m.items() if k != "fails"))
        assert not m["fails"], m["fails"]


def test_noalloc_rejects_a_configuration_beyond_its_area():
    import ctypes
    import decode_step_moe_amd as dl
    from decode_step_moe_amd import binding
    say("[no-alloc, batched path at batch 64 (TP8 shapes): too large for the static area] start")
    layer = workload.build(3, h_source="stored")
    cfg = sdev.config_of(layer, 64, path=3)
    assert binding.scratch_bytes(cfg, 256) > binding.noalloc_max_scratch()
    w = binding.Weights(*([0x1000] * 10))
    io = binding.IO(64, *([0x1000] * 10))
    rc = binding.lib().decode_layer_step_noalloc(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io), None)
    assert rc == dl.DL_ERR_UNSUPPORTED and "static area" in dl.last_error()
