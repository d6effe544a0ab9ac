"""A decode loop captured once as a HIP graph and replayed: each step of a
TP16 shard runs the attention core (speculative verify, 1 request x 8
tokens, appending to and reading the FP8 cache) and then the MoE layer step
on the attention's bf16 output, as a serving loop would chain them.

Between replays only device buffers change, by copies on the stream: the
step's queries, keys and values, the layer's input rows and residual, and
the past length (advanced by the step's 8 tokens).  Every replay is checked
against the oracles run on the same state: the cache codes bit-exact, the
attention output within the attention gates, its bf16 copy the fp32 output
rounded to nearest even, and the layer's outputs within the layer gates (the
layer oracle takes the attention's bf16 output as its attn input).  The
router is shaped once for the 24 token rows of the three steps, from the
oracle's attention outputs, so that every step's top-k has its margins.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import attention_ref as aref
from synth import attn_gen, device as sdev, gen, routing
from tests import parity, workload
from tests.parity import say
from tests.test_attention_gpu import Dev, check_out

pytestmark = pytest.mark.gpu

STEPS, T, C, PAST0 = 3, 8, 2048, 1000


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_moe_amd  # noqa: F401  (raises if the library was not built)


def test_attention_and_layer_steps_replayed_in_one_graph():
    from decode_step_moe_amd import DecodeLayer
    from decode_step_moe_amd import attention as at
    say("[decode loop: attention + layer step in one graph, TP16 shard, 1 x 8 tokens] start")
    # attention inputs of every step; the cache and scales are those of step 0
    steps = [attn_gen.draw(1, T, 4, 1, C, PAST0 + T * k, PAST0 + T * k, seed=300 + k) for k in range(STEPS)]
    st0 = steps[0]
    kc, vc = st0.k_cache, st0.v_cache
    want_att = []
    for k, s in enumerate(steps):
        out, kc, vc = aref.decode_attention(s.q, s.k_new, s.v_new, kc, vc, s.past_len, st0.k_scale,
                                            st0.v_scale, st0.softmax_scale)
        want_att.append((out, kc, vc))
    # the layer, its router shaped for all 24 token rows at once
    s24 = dataclasses.replace(gen.SHAPES[2], name="tp16_decode_loop_24", batch=STEPS * T)
    raw24 = gen.draw_shape(s24, seed=2)
    raw24.attn = np.concatenate([gen.f32_to_bf16_bits(o.astype(np.float32)).reshape(T, -1)
                                 for o, _, _ in want_att])
    layer24 = routing.shape_router(raw24, workload.oracle_h(raw24))
    h = DecodeLayer(sdev.config_of(layer24, max_batch=T), sdev.upload_weights(layer24))

    dev = Dev(st0, max_past=PAST0 + T * (STEPS - 1), with_bf16=True)
    x = torch.empty(T, s24.hidden, dtype=torch.bfloat16, device="cuda")
    resid = torch.empty(T, s24.hidden, device="cuda")
    res = h.alloc_outputs(T, with_h=True)
    io = h.make_io(x, dev.out_bf16.view(T, -1), resid, res)

    def load_step(k):   # device copies on the current stream, as a serving loop would make
        s = steps[k]
        dev.q.copy_(sdev.bf16_tensor(s.q, "cuda"))
        dev.k_new.copy_(sdev.bf16_tensor(s.k_new, "cuda"))
        dev.v_new.copy_(sdev.bf16_tensor(s.v_new, "cuda"))
        dev.past.fill_(int(s.past_len[0]))
        x.copy_(sdev.bf16_tensor(raw24.x[T * k:T * (k + 1)], "cuda"))
        resid.copy_(sdev.f32_tensor(raw24.resid[T * k:T * (k + 1)], "cuda"))

    load_step(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        at.step_io(dev.cfg, dev.io, side)
        h.step_io(io, side)
    torch.cuda.synchronize()   # capture runs nothing: the cache still holds step 0's past

    for k in range(STEPS):
        load_step(k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert h.status() == 0
        out, got_k, got_v = dev.results()
        want_out, want_k, want_v = want_att[k]
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v), f"step {k}: cache codes differ"
        check_out(f"loop step {k} attention", out, want_out)
        ob = dev.out_bf16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(ob, torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        # the layer oracle on the attention's own bf16 output
        raw8 = dataclasses.replace(raw24, shape=dataclasses.replace(s24, batch=T), x=raw24.x[T * k:T * (k + 1)],
                                   attn=ob.reshape(T, -1), resid=raw24.resid[T * k:T * (k + 1)])
        layer8 = routing.RoutedLayer(raw8, layer24.w_router, layer24.targets[T * k:T * (k + 1)],
                                     layer24.target_logits[T * k:T * (k + 1)])
        got = {"qkv": res.qkv.cpu().numpy(), "resid_out": res.resid_out.cpu().numpy(),
               "logits": res.router_logits.cpu().numpy(), "topk_idx": res.topk_idx.cpu().numpy(),
               "topk_w": res.topk_w.cpu().numpy(), "moe_out": res.moe_out.cpu().numpy(),
               "h": res.h_out.cpu().numpy()}
        m = parity.compare(got, workload.expected(layer8))
        say(f"[loop step {k} layer] " + ", ".join(f"{n}={v:.3e}" for n, v in m.items() if n != "fails"))
        assert not m["fails"], (k, m["fails"])
