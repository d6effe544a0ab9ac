"""A chain of decode layers captured in one HIP graph, with and without the
cross-layer weight prefetch.

Every layer has its own weights (its own seed) and its own attention input
and output; layer i+1's residual input is layer i's residual output, on the
device, inside the graph.  Each layer's router is shaped with the oracle's h
for the residual it will really receive (the oracle's r1 of the previous
layer rounded to fp32, as the GPU hands it on), so every layer's top-k keeps
its margins.  The graph is replayed several times with eager steps in
between; every replay must match the oracle layer by layer, and the chain
with prefetch must equal the chain without it bit for bit (the prefetch
changes where the next layer's weights are read from, never the results).
"""
import numpy as np
import pytest
import torch

from synth import device as sdev, gen, routing
from tests import parity, workload
from tests.parity import say

pytestmark = pytest.mark.gpu

KEYS = ("qkv", "resid_out", "topk_idx", "topk_w", "moe_out")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_moe_amd  # noqa: F401


def chain_layers(cfg, n_layers):
    """Routed layers whose residual inputs chain through the oracle."""
    layers, expected = [], []
    resid = None
    for i in range(n_layers):
        raw = gen.draw(cfg, seed=100 + 17 * cfg + i)
        if resid is not None:
            raw.resid = resid
        layer = routing.shape_router(raw, workload.oracle_h(raw))
        exp = workload.expected(layer)
        layers.append(layer)
        expected.append(exp)
        resid = np.asarray(exp["resid_out"], np.float32)   # the fp32 residual the GPU hands on
        raw.drop_expert_cache()
    return layers, expected


def got_of(out):
    return {"qkv": out.qkv.cpu().numpy(), "resid_out": out.resid_out.cpu().numpy(),
            "logits": out.router_logits.cpu().numpy(), "topk_idx": out.topk_idx.cpu().numpy(),
            "topk_w": out.topk_w.cpu().numpy(), "moe_out": out.moe_out.cpu().numpy(), "h": None}


@pytest.mark.parametrize("cfg,n_layers", [(1, 6), (2, 4)])
def test_layer_chain_in_one_graph(cfg, n_layers):
    from decode_step_moe_amd import DecodeLayer
    say(f"[chain of {n_layers} layers, {gen.SHAPES[cfg].name}, one graph, prefetch off/on] start")
    layers, expected = chain_layers(cfg, n_layers)
    B = layers[0].shape.batch
    handles = [DecodeLayer(sdev.config_of(l), sdev.upload_weights(l)) for l in layers]
    assert all(h.single_max_batch >= B for h in handles)
    inputs = [sdev.upload_inputs(l) for l in layers]
    results = {}
    for prefetch in (False, True):
        for i, h in enumerate(handles):
            h.set_prefetch(handles[i + 1] if prefetch and i + 1 < n_layers else None)
        outs = [h.alloc_outputs(B) for h in handles]
        ios = []
        for i, h in enumerate(handles):
            x, attn, resid = inputs[i]
            r_in = resid if i == 0 else outs[i - 1].resid_out
            ios.append(h.make_io(x, attn, r_in, outs[i]))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for h, io in zip(handles, ios):
                h.step_io(io, s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for h, io in zip(handles, ios):
                h.step_io(io)
        for rep in range(4):
            for o in outs:
                o.moe_out.fill_(float("nan"))
                o.resid_out.fill_(float("nan"))
                o.topk_idx.fill_(-1)
            g.replay()
            torch.cuda.synchronize()
            for i, (o, exp) in enumerate(zip(outs, expected)):
                m = parity.compare(got_of(o), exp)
                if rep == 0:
                    say(f"[chain prefetch={prefetch} layer {i}] " +
                        ", ".join(f"{k}={v:.2e}" for k, v in m.items() if k != "fails"))
                assert not m["fails"], (prefetch, rep, i, m["fails"])
            if rep == 1:   # eager steps of the whole chain between replays
                for h, io in zip(handles, ios):
                    h.step_io(io)
                torch.cuda.synchronize()
        results[prefetch] = [{k: getattr(o, k).clone() for k in KEYS} for o in outs]
        del g
    for i in range(n_layers):
        for k in KEYS:
            assert torch.equal(results[False][i][k], results[True][i][k]), (i, k)
    for h in handles:
        assert h.status() == 0


def test_prefetch_needs_the_same_configuration():
    from decode_step_moe_amd import DecodeLayer, DecodeLayerError, DL_ERR_INVALID_ARG
    say("[prefetch between layers of different shapes is refused] start")
    a = workload.build(0, h_source="stored")
    b = workload.build(0, top_k=1)
    ha = DecodeLayer(sdev.config_of(a), sdev.upload_weights(a))
    hb = DecodeLayer(sdev.config_of(b), sdev.upload_weights(b))
    with pytest.raises(DecodeLayerError) as ei:
        ha.set_prefetch(hb)
    assert ei.value.code == DL_ERR_INVALID_ARG
    ha.set_prefetch(None)
