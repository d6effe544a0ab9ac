"""GPU parity of the HIP layer-step against the CPU oracle, through the C ABI.

Every case prints its name before touching the GPU.  Inputs are the seeded
synthetic workloads (synth/), the expected values come from the oracle only.
Unselected experts are NaN-poisoned in every case, so an out-of-route read
shows up as a non-finite output.
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
    import decode_step_moe_amd  # noqa: F401  (raises if the library was not built)


def run_gpu(layer, with_h=True, max_batch=None, inplace=False, logits=True, layer_obj=None):
    from decode_step_moe_amd import DecodeLayer
    cfg = sdev.config_of(layer, max_batch)
    if layer_obj is None:
        w = sdev.upload_weights(layer)
        layer_obj = DecodeLayer(cfg, w)
    x, attn, resid = sdev.upload_inputs(layer)
    out = layer_obj.alloc_outputs(layer.shape.batch, with_h=with_h, with_logits=logits)
    if inplace:
        out.resid_out = resid
    layer_obj.step(x, attn, resid, out)
    torch.cuda.synchronize()
    got = {"qkv": out.qkv.cpu().numpy(), "resid_out": out.resid_out.cpu().numpy(),
           "logits": out.router_logits.cpu().numpy() if logits else None,
           "topk_idx": out.topk_idx.cpu().numpy(), "topk_w": out.topk_w.cpu().numpy(),
           "moe_out": out.moe_out.cpu().numpy(),
           "h": out.h_out.cpu().numpy() if with_h else None}
    return got, layer_obj


def check(layer, got, tag):
    ref = workload.expected(layer)
    m = parity.compare(got, ref)
    say(f"[{tag}] " + ", ".join(f"{k}={v:.3e}" for k, v in m.items() if k != "fails"))
    assert not m["fails"], f"{tag}: {m['fails']}"
    return m


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_workload_parity(cfg):
    say(f"[workload cfg={cfg} {gen.SHAPES[cfg].name}] start")
    layer = workload.build(cfg, h_source="stored")
    got, _ = run_gpu(layer)
    check(layer, got, f"cfg{cfg}")


@pytest.mark.parametrize("batch", [2, 3, 5, 13, 64])
def test_ragged_batches(batch):
    say(f"[ragged cfg=2 shapes, batch={batch}] start")
    layer = workload.build(2, batch=batch)
    got, _ = run_gpu(layer, max_batch=64)
    check(layer, got, f"ragged_b{batch}")


@pytest.mark.parametrize("top_k,shared", [(1, 256), (8, 256), (2, 0), (1, 0)])
def test_topk_and_shared_edges(top_k, shared):
    say(f"[tiny edges k={top_k} shared_ffn={shared}] start")
    layer = workload.build(0, batch=3, top_k=top_k, shared_ffn=shared)
    got, _ = run_gpu(layer)
    m = check(layer, got, f"tiny_k{top_k}_fs{shared}")
    if top_k == 1:
        assert np.all(got["topk_w"] == 1.0)
    if top_k == 8:   # k = E: every expert, weights s / sum s
        assert sorted(got["topk_idx"][0].tolist()) == list(range(8))
    assert m


def test_batch_zero_is_noop():
    say("[batch 0] start")
    from decode_step_moe_amd import IO
    layer = workload.build(0)
    got, obj = run_gpu(layer)
    io = IO(0)
    obj.step_io(io)
    torch.cuda.synchronize()


def test_inplace_residual_and_null_logits():
    say("[in-place residual, logits NULL] start")
    layer = workload.build(4, h_source="stored")
    got, _ = run_gpu(layer, inplace=True, logits=False)
    check(layer, got, "inplace")


def test_batch_equals_single_token_steps():
    say("[batch of 8 vs 8 single-token steps, cfg 4] start")
    layer = workload.build(4, h_source="stored")
    got, obj = run_gpu(layer, max_batch=8)
    x, attn, resid = sdev.upload_inputs(layer)
    for t in range(8):
        out = obj.alloc_outputs(1, with_h=False)
        obj.step(x[t:t + 1].contiguous(), attn[t:t + 1].contiguous(), resid[t:t + 1].contiguous(), out)
        torch.cuda.synchronize()
        assert out.topk_idx.cpu().numpy()[0].tolist() == got["topk_idx"][t].tolist()
        for key, ref in (("moe_out", got["moe_out"][t]), ("resid_out", got["resid_out"][t]),
                         ("qkv", got["qkv"][t])):
            v = getattr(out, key).cpu().numpy()[0]
            assert parity.max_abs(v, ref) <= 1e-5 * max(1.0, np.abs(ref).max()), key


def test_repeated_steps_are_stable_under_concurrency():
    """200 back-to-back steps with unrelated work on another stream: indices
    and every output must be bit-identical each time (the kernels are
    deterministic), which catches a hand-off read before its acquire."""
    say("[stress 200 steps, cfg 2 shapes] start")
    from decode_step_moe_amd import DecodeLayer
    layer = workload.build(2, h_source="stored")
    cfg = sdev.config_of(layer)
    obj = DecodeLayer(cfg, sdev.upload_weights(layer))
    x, attn, resid = sdev.upload_inputs(layer)
    first = obj.step(x, attn, resid)
    torch.cuda.synchronize()
    ref = {k: getattr(first, k).clone() for k in ("qkv", "resid_out", "topk_idx", "topk_w", "moe_out")}
    other = torch.cuda.Stream()
    junk = torch.randn(4096, 4096, device="cuda")
    outs = [obj.alloc_outputs(layer.shape.batch) for _ in range(4)]
    for it in range(200):
        with torch.cuda.stream(other):
            junk.mul_(1.0001)
        o = outs[it % 4]
        obj.step(x, attn, resid, o)
        if it % 4 == 3:
            torch.cuda.synchronize()
            for oo in outs:
                for k, v in ref.items():
                    assert torch.equal(getattr(oo, k), v), (it, k)
    torch.cuda.synchronize()


def test_graph_replay_matches_eager():
    say("[hip graph capture + replays, cfg 1] start")
    from decode_step_moe_amd import DecodeLayer
    layer = workload.build(1, h_source="stored")
    obj = DecodeLayer(sdev.config_of(layer), sdev.upload_weights(layer))
    x, attn, resid = sdev.upload_inputs(layer)
    eager = obj.step(x, attn, resid)
    torch.cuda.synchronize()
    out = obj.alloc_outputs(1)
    io = obj.make_io(x, attn, resid, out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm up on the capture stream
        obj.step_io(io, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        obj.step_io(io)
    for rep in range(3):
        for k in ("qkv", "resid_out", "moe_out", "topk_w"):
            getattr(out, k).fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k in ("qkv", "resid_out", "topk_idx", "topk_w", "moe_out"):
            assert torch.equal(getattr(out, k), getattr(eager, k)), (rep, k)
        obj.step(x, attn, resid)   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("scale", [1e3, 1e-3])
def test_residual_scale_extremes(scale):
    say(f"[residual scaled x{scale}, cfg 4 shapes] start")
    raw = gen.draw(4)
    raw.resid = (raw.resid * np.float32(scale)).astype(np.float32)
    layer = routing.shape_router(raw, workload.oracle_h(raw))
    got, _ = run_gpu(layer)
    ref = workload.expected(layer)
    m = parity.compare(got, ref)
    say(f"[resid x{scale}] " + ", ".join(f"{k}={v:.3e}" for k, v in m.items() if k != "fails"))
    # the residual itself is compared relative to its own size
    fails = [f for f in m["fails"] if not f.startswith("resid_out")]
    assert not fails, fails
    assert m["resid_out_rel_l2"] <= parity.OUT_REL_L2
