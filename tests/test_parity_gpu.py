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


AUTO, MULTI, SINGLE, BATCHED = 0, 1, 2, 3
PATH_NAMES = {AUTO: "auto", MULTI: "multi", SINGLE: "single", BATCHED: "batched"}
PATHS = [AUTO, MULTI, BATCHED]


def used_single(obj, batch, path):
    return path in (AUTO, SINGLE) and batch <= obj.single_max_batch


def used_name(obj, batch, path):
    if used_single(obj, batch, path):
        return "single"
    return "multi" if path == MULTI else "batched"


def run_gpu(layer, with_h=True, max_batch=None, inplace=False, logits=True, layer_obj=None,
            path=AUTO):
    from decode_step_moe_amd import DecodeLayer
    cfg = sdev.config_of(layer, max_batch, path=path)
    if layer_obj is None:
        w = sdev.upload_weights(layer)
        layer_obj = DecodeLayer(cfg, w)
    x, attn, resid = sdev.upload_inputs(layer)
    out = layer_obj.alloc_outputs(layer.shape.batch, with_h=with_h, with_logits=logits)
    if inplace:
        out.resid_out = resid
    layer_obj.step(x, attn, resid, out)
    torch.cuda.synchronize()
    assert layer_obj.status() == 0, "a single-launch hand-off wait expired"
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


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_workload_parity(cfg, path):
    say(f"[workload cfg={cfg} {gen.SHAPES[cfg].name} path={PATH_NAMES[path]}] start")
    layer = workload.build(cfg, h_source="stored")
    got, obj = run_gpu(layer, path=path)
    single = used_single(obj, layer.shape.batch, path)
    # batches up to 8 take the single-launch path under AUTO at these shapes
    assert single == (path == AUTO and layer.shape.batch <= 8), (obj.single_max_batch, layer.shape.batch)
    check(layer, got, f"cfg{cfg}_{used_name(obj, layer.shape.batch, path)}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("batch", [2, 3, 5, 13, 17, 64])
def test_ragged_batches(batch, path):
    say(f"[ragged cfg=2 shapes, batch={batch} path={PATH_NAMES[path]}] start")
    layer = workload.build(2, batch=batch)
    got, obj = run_gpu(layer, max_batch=64, path=path)
    check(layer, got, f"ragged_b{batch}_{used_name(obj, batch, path)}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("top_k,shared", [(1, 256), (8, 256), (2, 0), (1, 0)])
def test_topk_and_shared_edges(top_k, shared, path):
    say(f"[tiny edges k={top_k} shared_ffn={shared} path={PATH_NAMES[path]}] start")
    layer = workload.build(0, batch=3, top_k=top_k, shared_ffn=shared)
    got, obj = run_gpu(layer, path=path)
    assert used_single(obj, 3, path) == (path == AUTO)
    m = check(layer, got, f"tiny_k{top_k}_fs{shared}_{PATH_NAMES[path]}")
    if top_k == 1:
        assert np.all(got["topk_w"] == 1.0)
    if top_k == 8:   # k = E: every expert, weights s / sum s
        assert sorted(got["topk_idx"][0].tolist()) == list(range(8))
    assert m


@pytest.mark.parametrize("path", PATHS)
def test_exact_logit_ties(path):
    """Exact logit ties, made by duplicating router rows of the batch-1 TP16
    shard: one inside the top-k and one across its boundary.  Equal logits
    rank by expert id, lower first, and the boundary tie keeps the lower id."""
    import dataclasses
    say(f"[exact logit ties, TP16 shard batch 1, path={PATH_NAMES[path]}] start")
    base = workload.build(1, h_source="stored")
    k = base.shape.top_k
    order = np.argsort(-workload.expected(base)["logits"][0], kind="stable")
    picked = set(order[:k].tolist())
    free = [e for e in range(base.shape.n_experts) if e not in picked]
    r_in, r_edge = int(order[2]), int(order[k - 2])
    d_in = free[0]
    lower = [e for e in free[1:] if e < r_edge]
    d_edge = lower[0] if lower else free[1]
    wr = base.w_router.copy()
    wr[d_in] = wr[r_in]
    wr[d_edge] = wr[r_edge]
    layer = dataclasses.replace(base, w_router=wr)
    ref = workload.expected(layer)
    idx = ref["topk_idx"][0].tolist()
    assert d_in in idx and r_in in idx and idx.index(min(d_in, r_in)) + 1 == idx.index(max(d_in, r_in))
    assert (min(d_edge, r_edge) in idx) and (max(d_edge, r_edge) not in idx)
    layer = dataclasses.replace(layer, targets=np.asarray(ref["topk_idx"], np.int32))
    got, obj = run_gpu(layer, path=path)
    check(layer, got, f"ties_{used_name(obj, 1, path)}")


@pytest.mark.parametrize("case", ["ties_over_waves", "all_equal", "k10", "k11"])
def test_one_token_topk_over_waves(case):
    """Batch 1, TP16 shard (384 experts) on the single launch, which spreads
    the token's candidates one per lane over six waves and merges the six pick
    lists on one wave.  Cases: eleven equal maximal logits in six 64-expert
    ranges (the eight lowest ids win); all 384 logits equal (ids 0..7); k = 10,
    the largest k whose six lists fit one wave; k = 11, one wave per token."""
    import dataclasses
    say(f"[one-token top-k over waves, TP16 shard batch 1, {case}] start")
    if case in ("k10", "k11"):
        layer = workload.build(1, h_source="stored", top_k=int(case[1:]))
        got, obj = run_gpu(layer)
        assert used_single(obj, 1, AUTO)
        check(layer, got, f"one_token_{case}")
        return
    base = workload.build(1, h_source="stored")
    k = base.shape.top_k
    wr = base.w_router.copy()
    if case == "ties_over_waves":
        top = int(np.argmax(workload.expected(base)["logits"][0]))
        group = [e for e in (1, 3, 64, 65, 70, 129, 190, 250, 300, 383) if e != top]
        wr[group] = wr[top]
        want = sorted(group + [top])[:k]
    else:
        wr[:] = wr[0]
        want = list(range(k))
    layer = dataclasses.replace(base, w_router=wr)
    ref = workload.expected(layer)
    assert ref["topk_idx"][0].tolist() == want
    layer = dataclasses.replace(layer, targets=np.asarray(ref["topk_idx"], np.int32))
    got, obj = run_gpu(layer)
    assert used_single(obj, 1, AUTO)
    check(layer, got, f"one_token_{case}")


def test_batch_zero_is_noop():
    say("[batch 0] start")
    from decode_step_moe_amd import IO
    layer = workload.build(0)
    got, obj = run_gpu(layer)
    io = IO(0)
    obj.step_io(io)
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", PATHS)
def test_inplace_residual_and_null_logits(path):
    say(f"[in-place residual, logits NULL, path={PATH_NAMES[path]}] start")
    layer = workload.build(4, h_source="stored")
    got, _ = run_gpu(layer, inplace=True, logits=False, path=path)
    check(layer, got, "inplace")


def test_single_path_refuses_a_larger_batch():
    """DL_PATH_SINGLE with a batch above its limit fails on the host; nothing runs."""
    say("[forced single path, batch above its limit] start")
    from decode_step_moe_amd import DecodeLayerError, DL_ERR_UNSUPPORTED
    layer = workload.build(2, batch=13)
    got, obj = run_gpu(workload.build(2, batch=5), max_batch=64, path=SINGLE)
    assert obj.single_max_batch == 8
    x, attn, resid = sdev.upload_inputs(layer)
    with pytest.raises(DecodeLayerError) as ei:
        obj.step(x, attn, resid)
    assert ei.value.code == DL_ERR_UNSUPPORTED


def test_single_path_alternating_batches():
    """One handle, single-launch path, batch sizes changing from step to step:
    every step's hand-off values carry a fresh tag, so values left by an
    earlier (larger) step are never taken for this step's."""
    say("[single path, batches 8,1,5,8,2,1 on one handle] start")
    from decode_step_moe_amd import DecodeLayer
    full = workload.build(2, batch=8)
    obj = DecodeLayer(sdev.config_of(full, 8), sdev.upload_weights(full))
    for b in (8, 1, 5, 8, 2, 1):
        # the batch-8 router gives every prefix token its target logits exactly
        layer = routing.RoutedLayer(gen.draw(2, batch=b), full.w_router, full.targets[:b],
                                    full.target_logits[:b])
        got, _ = run_gpu(layer, layer_obj=obj)
        assert used_single(obj, b, AUTO)
        check(layer, got, f"alternating_b{b}")


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


@pytest.mark.parametrize("cfg,path", [(2, AUTO), (3, AUTO), (2, BATCHED)])
def test_repeated_steps_are_stable_under_concurrency(cfg, path):
    """1000 back-to-back steps with unrelated work on another stream: indices
    and every output must be bit-identical each time (the kernels are
    deterministic), which catches a hand-off read before its acquire.  The
    single-launch path (batch 8) and the batched path (batch 64 with hot
    experts on the matrix cores, and batch 8) each run it; the first
    mismatching step ends the test."""
    from decode_step_moe_amd import DecodeLayer
    layer = workload.build(cfg, h_source="stored")
    obj = DecodeLayer(sdev.config_of(layer, path=path), sdev.upload_weights(layer))
    B = layer.shape.batch
    say(f"[stress 1000 steps, cfg {cfg} batch {B}, {used_name(obj, B, path)} path] start")
    assert used_single(obj, B, path) == (cfg == 2 and path == AUTO)
    x, attn, resid = sdev.upload_inputs(layer)
    first = obj.step(x, attn, resid)
    torch.cuda.synchronize()
    got = {k: getattr(first, k).cpu().numpy() for k in ("qkv", "resid_out", "topk_idx", "topk_w", "moe_out")}
    got["logits"] = first.router_logits.cpu().numpy()
    check(layer, got, f"stress_first_cfg{cfg}")
    ref = {k: getattr(first, k).clone() for k in ("qkv", "resid_out", "topk_idx", "topk_w", "moe_out")}
    other = torch.cuda.Stream()
    junk = torch.randn(4096, 4096, device="cuda")
    outs = [obj.alloc_outputs(B) for _ in range(4)]
    for it in range(1000):
        with torch.cuda.stream(other):
            junk.mul_(1.0001)
        o = outs[it % 4]
        obj.step(x, attn, resid, o)
        if it % 4 == 3:
            torch.cuda.synchronize()
            for oo in outs:
                for k, v in ref.items():
                    assert torch.equal(getattr(oo, k), v), (it, k)
                    getattr(oo, k).fill_(-1)
    torch.cuda.synchronize()
    assert obj.status() == 0


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


@pytest.mark.parametrize("path", PATHS)
def test_graph_replay_many_steps(path):
    """A graph holding two steps (different copies of the inputs), replayed
    10 times with eager steps in between: the single-launch path's step
    counter lives on the device, so replays use fresh tags."""
    say(f"[graph of 2 steps x 10 replays, cfg 2, path={PATH_NAMES[path]}] start")
    from decode_step_moe_amd import DecodeLayer
    layer = workload.build(2, h_source="stored")
    obj = DecodeLayer(sdev.config_of(layer, path=path), sdev.upload_weights(layer))
    x, attn, resid = sdev.upload_inputs(layer)
    eager = obj.step(x, attn, resid)
    torch.cuda.synchronize()
    outs = [obj.alloc_outputs(8) for _ in range(2)]
    ios = [obj.make_io(x, attn, resid, o) for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        obj.step_io(ios[0], s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        obj.step_io(ios[0])
        obj.step_io(ios[1])
    for rep in range(10):
        for o in outs:
            o.moe_out.fill_(float("nan"))
            o.topk_idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            for k in ("qkv", "resid_out", "topk_idx", "topk_w", "moe_out"):
                assert torch.equal(getattr(o, k), getattr(eager, k)), (rep, k)
        if rep % 3 == 0:
            obj.step(x, attn, resid)
            torch.cuda.synchronize()
    assert obj.status() == 0


def test_batched_graph_replay_hot_experts():
    """The batched path at batch 64 (hot experts, every routed contraction on
    MFMA) captured in a graph with another step, replayed with eager steps
    in between: every replay equals the eager result bit for bit."""
    say("[graph of 2 batched steps x 6 replays, cfg 3] start")
    from decode_step_moe_amd import DecodeLayer
    layer = workload.build(3, h_source="stored")
    obj = DecodeLayer(sdev.config_of(layer), sdev.upload_weights(layer))
    assert not used_single(obj, 64, AUTO)
    x, attn, resid = sdev.upload_inputs(layer)
    eager = obj.step(x, attn, resid)
    torch.cuda.synchronize()
    outs = [obj.alloc_outputs(64) for _ in range(2)]
    ios = [obj.make_io(x, attn, resid, o) for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        obj.step_io(ios[0], s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        obj.step_io(ios[0])
        obj.step_io(ios[1])
    for rep in range(6):
        for o in outs:
            o.moe_out.fill_(float("nan"))
            o.qkv.fill_(float("nan"))
            o.topk_idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            for k in ("qkv", "resid_out", "topk_idx", "topk_w", "moe_out"):
                assert torch.equal(getattr(o, k), getattr(eager, k)), (rep, k)
        if rep % 2 == 0:
            obj.step(x, attn, resid)
            torch.cuda.synchronize()


def test_batched_path_batches_change_on_one_handle():
    """One batched-path handle stepping batches 64, 9, 33, 1, 64: the lists
    and partial sums of a larger step never leak into a smaller one."""
    say("[batched path, batches 64,9,33,1,64 on one handle] start")
    from decode_step_moe_amd import DecodeLayer
    full = workload.build(2, batch=64)
    obj = DecodeLayer(sdev.config_of(full, 64, path=BATCHED), sdev.upload_weights(full))
    for b in (64, 9, 33, 1, 64):
        layer = routing.RoutedLayer(gen.draw(2, batch=b), full.w_router, full.targets[:b],
                                    full.target_logits[:b])
        got, _ = run_gpu(layer, layer_obj=obj)
        check(layer, got, f"batched_b{b}")


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


_EXPECTED = {}


def _skewed(batch):
    key = ("skewed", batch)
    if key not in _EXPECTED:
        raw = gen.draw(3, batch=batch, routing="skewed")
        layer = routing.shape_router(raw, workload.oracle_h(raw))
        _EXPECTED[key] = (layer, workload.expected(layer))
    return _EXPECTED[key]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("batch", [64, 33])
def test_skewed_expert_loads(batch, path):
    """TP8 shard shapes (ffn 256) with routed experts holding 1, 9, 15, 16,
    17, 31, 32, 33, 48 and 64 tokens (clipped to the batch): both sides of the
    16-token matrix-core threshold, a partial second 16-token chunk, two or
    more full chunks, and an expert every token picked."""
    say(f"[skewed expert loads, TP8 shapes, batch={batch} path={PATH_NAMES[path]}] start")
    layer, ref = _skewed(batch)
    loads = layer.expert_load()
    say(f"[skewed b{batch}] loads: " + ",".join(str(v) for v in sorted(loads[loads > 0].tolist(), reverse=True)[:12]))
    got, obj = run_gpu(layer, path=path)
    m = parity.compare(got, ref)
    tag = f"skewed_b{batch}_{used_name(obj, batch, path)}"
    say(f"[{tag}] " + ", ".join(f"{k}={v:.3e}" for k, v in m.items() if k != "fails"))
    assert not m["fails"], f"{tag}: {m['fails']}"


@pytest.mark.parametrize("path", PATHS)
def test_saturating_logits(path):
    """Router logits shifted per token by +-30, +-60, +90, -100 and -200
    (batch 8, TP16 shard): the sigmoid saturates at 1 or underflows fp32
    (below about -87), and the renormalised weights must still match the
    oracle's."""
    say(f"[saturating logits, TP16 shard batch 8, path={PATH_NAMES[path]}] start")
    raw = gen.draw(2)
    shift = np.array([30.0, -30.0, 60.0, -60.0, 90.0, -100.0, 0.0, -200.0])
    layer = routing.shape_router(raw, workload.oracle_h(raw), shift=shift)
    ref = workload.expected(layer)
    assert np.all(np.abs(ref["logits"].max(axis=1) - shift) < 8.0)
    got, obj = run_gpu(layer, path=path)
    assert np.all(np.isfinite(got["topk_w"]))
    check(layer, got, f"saturating_{used_name(obj, 8, path)}")


@pytest.mark.parametrize("path", PATHS)
def test_negative_and_zero_gain(path):
    """RMSNorm gain drawn N(0, 1) (about half negative) with some entries
    exactly zero and some exactly -1 (speculative-verify shapes, Zipf routing)."""
    say(f"[negative / zero gain, spec-verify shapes, path={PATH_NAMES[path]}] start")
    raw = gen.draw(4)
    g = gen.rng(1234, 7).normal(0.0, 1.0, size=raw.shape.hidden).astype(np.float32)
    g[::97] = 0.0
    g[5::101] = -1.0
    raw.gain = gen.f32_to_bf16_bits(g)
    assert np.mean(gen.bf16_bits_to_f32(raw.gain) < 0) > 0.4
    layer = routing.shape_router(raw, workload.oracle_h(raw))
    got, obj = run_gpu(layer, path=path)
    check(layer, got, f"neg_gain_{used_name(obj, 8, path)}")
