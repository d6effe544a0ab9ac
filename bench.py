"""Benchmark of one MoE decode layer-step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--copies L] [--no-batches] [--no-cpu]

Workload (headline line): one TP16 shard at batch 1 - hidden 7168, Wqkv
7168x512, Wo 512x7168, fp32 router 7168x384 with sigmoid top-8, 384 SwiGLU
experts with ffn shard 128 and a shared expert with ffn 128, bf16 weights,
uniform-random routing.  Batches 8 (uniform and Zipf speculative-verify) and
64 (TP8 shard, 32 hot experts) are measured the same way and reported under
"batches".

Protocol: L device-side copies of the layer (weights, expert pool, router)
are rotated every step so that no step finds its weights in the 256 MB
Infinity Cache (L * touched bytes >= 1 GB); inputs are resident in HBM before
the timed region.  W warm-up steps, then K timed steps between HIP events on
the launching stream, once with eager launches and once replaying one HIP
graph per copy (the headline).  A third pass with per-launch HIP events gives
each kernel's average duration, from which the roofline object is computed for
the kernel that takes the most time.  The CPU baseline is the fp64 oracle run
on a bounded sample of the same workload on the host cores.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per decode layer-step & achieved HBM GB/s (% of peak), batch 1/8/64"
HBM_PEAK_GBPS = 8000.0
HEADLINE_CFG = 1
BATCH_CFGS = (2, 4, 3)
ATTN_WORKLOADS = ("attn_verify_ctx8k", "attn_b64_ctx4k")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- bytes
def algorithmic_bytes(layer) -> dict:
    """Unique weight bytes each launch must read plus its activation I/O.

    Intermediates that stay on chip or in L2 between launches (hg, inv_rms,
    the permutation lists, expert activations) are counted once where they
    are produced and consumed only as activation traffic of the consumer
    (h rows and ffn activations), as the floor any implementation pays."""
    s = layer.shape
    B, H, Dq, Do, E, k, F, Fs = (s.batch, s.hidden, s.qkv_out, s.attn_dim, s.n_experts,
                                 s.top_k, s.expert_ffn, s.shared_ffn)
    n_act = len(layer.touched_experts())
    pairs = B * k
    b = {}
    b["proj_out_in"] = 2 * (Dq * H + H * Do + H) + 2 * B * (H + Do) + 4 * B * H * 2 + 4 * B * Dq
    b["shared_gateup"] = 2 * 2 * Fs * H + 4 * B * H + 4 * B * Fs
    b["router_topk_permute"] = 4 * E * H + 4 * B * H + 4 * B * E + 8 * pairs
    b["expert_gateup"] = n_act * 2 * 2 * F * H + 4 * B * H + 4 * pairs * F
    b["expert_down_combine"] = 2 * (n_act * H * F + H * Fs) + 4 * (pairs * F + B * Fs) + 4 * B * H
    # whole step: unique weights + step I/O (x, attn, resid in/out, qkv, logits, idx, w, y)
    weights = 2 * (Dq * H + H * Do + H) + 4 * E * H + n_act * 3 * 2 * F * H + 3 * 2 * Fs * H
    io = 2 * B * (H + Do) + 4 * B * H * 2 + 4 * B * Dq + 4 * B * E + 8 * pairs + 4 * B * H
    b["step"] = weights + io
    # the single-launch kernel does the whole step
    b["single_launch_step"] = b["step"]
    b["batched_proj"] = 2 * (Dq * H + H * Do + H) + 2 * B * (H + Do) + 4 * B * H * 3
    b["batched_router"] = 4 * E * H + 4 * B * H + 4 * B * Dq
    b["batched_topk_permute"] = 4 * B * H * 2 + 4 * B * E + 8 * pairs
    b["batched_gateup"] = b["shared_gateup"] + b["expert_gateup"] - 4 * B * H
    b["batched_down"] = b["expert_down_combine"]
    b["step_flops"] = 2 * B * (Dq * H + H * Do + E * H) + 2 * pairs * 3 * F * H + 2 * B * 3 * Fs * H
    return b


MFMA_PEAK = {"bf16": 2.5e15, "fp32": 157.3e12}   # dense matrix-core peaks of MI355X, flop/s


def mfma_flops(layer) -> dict:
    """Matrix-core flops each batched-path launch issues, by operand type.

    Tokens enter the matrix cores in 16-token chunks (a partial chunk is padded
    to 16), and an fp32 activation enters as two bf16 operands (hi + lo), so
    those contractions issue twice the flops of one pass: projections (bf16
    x and attn, one pass), router (fp32 operands on v_mfma_f32_16x16x4_f32),
    gate/up and down (hi + lo), routed experts only when they hold 16 or more
    tokens (the rest run on the VALU)."""
    s = layer.shape
    B, H, Dq, Do, E, F, Fs = s.batch, s.hidden, s.qkv_out, s.attn_dim, s.n_experts, s.expert_ffn, s.shared_ffn
    pad = lambda n: -(-n // 16) * 16
    load = layer.expert_load()
    mm = sum(pad(int(c)) for c in load if c >= 16)          # routed tokens on the matrix cores (padded)
    return {
        "batched_proj": {"bf16": 2 * pad(B) * (H * Do + Dq * H)},
        "batched_router": {"fp32": 2 * pad(B) * E * H},
        "batched_gateup": {"bf16": 2 * 2 * 2 * F * H * mm + 2 * 2 * 2 * Fs * H * pad(B)},
        "batched_down": {"bf16": 2 * 2 * H * F * mm + 2 * 2 * H * Fs * pad(B)},
    }


def mfma_util(layer, kernel_us: dict) -> dict:
    """Per matrix-core launch and over all of them: the time the matrix cores
    need for the issued flops at their dense peak, divided by the launch time."""
    fl = mfma_flops(layer)
    out, need, took = {}, 0.0, 0.0
    for k, by_t in fl.items():
        if k not in kernel_us:
            continue
        t_peak = sum(v / MFMA_PEAK[t] for t, v in by_t.items())
        t_run = kernel_us[k] * 1e-6
        out[k] = round(t_peak / t_run, 5)
        need += t_peak
        took += t_run
    if took > 0:
        out["all_matrix_core_launches"] = round(need / took, 5)
    return out


# ----------------------------------------------------------------- GPU side
def make_copies(layer, n_copies):
    import torch
    from synth import device as sdev
    w0 = sdev.upload_weights(layer, fill_untouched="none")
    touched = [int(e) for e in layer.touched_experts()]
    copies = [w0]
    for _ in range(1, n_copies):
        w = {}
        for key, t in w0.items():
            if key in ("w1", "w3", "w2"):
                c = torch.empty_like(t)
                for e in touched:
                    c[e].copy_(t[e])
                w[key] = c
            else:
                w[key] = t.clone()
        copies.append(w)
    torch.cuda.synchronize()
    return copies


def time_config(cfg_id, steps, warmup, n_copies, want_kernels=True, path=0, chain=True):
    import torch
    from decode_step_moe_amd import DecodeLayer
    from synth import device as sdev, routing, gen

    raw = gen.draw(cfg_id)
    layer = routing.shape_router(raw, routing.stored_h(cfg_id))
    nbytes = algorithmic_bytes(layer)
    if n_copies is None:
        n_copies = max(4, int(np.ceil(1.0e9 / nbytes["step"])))
    log(f"[bench] cfg {cfg_id} {layer.shape.name}: {len(layer.touched_experts())} experts, "
        f"{nbytes['step'] / 1e6:.2f} MB/step, {n_copies} copies")
    copies = make_copies(layer, n_copies)
    cfg = sdev.config_of(layer, path=path)
    handles = [DecodeLayer(cfg, w) for w in copies]
    single = path in (0, 2) and layer.shape.batch <= handles[0].single_max_batch
    batched = not single and any(k.startswith("batched") for k in _launch_probe(handles[0], layer))
    path_name = "single" if single else ("batched" if batched else "multi")
    x, attn, resid = sdev.upload_inputs(layer)
    outs = [h.alloc_outputs(layer.shape.batch) for h in handles]
    ios = [h.make_io(x, attn, resid, o) for h, o in zip(handles, outs)]
    stream = torch.cuda.current_stream()

    def run(i):
        handles[i % n_copies].step_io(ios[i % n_copies], stream)

    # consistency: every copy produces identical results
    for i in range(n_copies):
        run(i)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.topk_idx, outs[0].topk_idx) and torch.equal(o.moe_out, outs[0].moe_out)
    assert np.array_equal(np.sort(outs[0].topk_idx.cpu().numpy(), 1), np.sort(layer.targets, 1))

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(steps):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    eager_ms = timed(run)
    # one graph holding one step of every copy (as a decode step holds every
    # layer), replayed until at least `steps` steps have run
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(n_copies):
            handles[i].step_io(ios[i], side)
    torch.cuda.synchronize()
    reps = max(1, -(-steps // n_copies))
    for _ in range(max(1, warmup // n_copies)):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    graph_ms = t0.elapsed_time(t1) / (reps * n_copies)
    # graph results equal eager results
    ref = outs[0].moe_out.clone()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(outs[0].moe_out, ref)
    del g
    # the same rotation as a chain of layers in which every layer prefetches
    # the next one's dense weights (single-launch path only)
    chain_ms = None
    if single and chain:
        for i, h in enumerate(handles):
            h.set_prefetch(handles[(i + 1) % n_copies])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(n_copies):
                handles[i].step_io(ios[i], side)
        torch.cuda.synchronize()
        for _ in range(max(1, warmup // n_copies)):
            g.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        chain_ms = t0.elapsed_time(t1) / (reps * n_copies)
        assert torch.equal(outs[0].moe_out, ref)
        del g
        for h in handles:
            h.set_prefetch(None)

    kern = {}
    if want_kernels:
        # each profiled step is queued behind an unprofiled one, so its first
        # event is taken as the previous step ends, not on an idle GPU
        acc = {}
        for i in range(warmup + steps):
            run(i)
            hp = handles[(i + 1) % n_copies]
            hp.set_profiling(True)
            run(i + 1)
            times = hp.kernel_times_ms()
            hp.set_profiling(False)
            if i >= warmup:
                for k_, v in times.items():
                    acc.setdefault(k_, []).append(v)
        kern = {k_: float(np.mean(v)) for k_, v in acc.items()}
    for h in handles:
        assert h.status() == 0, "a single-launch hand-off wait expired"
    res = {"cfg": cfg_id, "workload": layer.shape.name, "batch": layer.shape.batch,
           "copies": n_copies, "eager_us": eager_ms * 1e3, "graph_us": graph_ms * 1e3,
           "prefetch_chain_us": chain_ms * 1e3 if chain_ms is not None else None,
           "bytes": nbytes, "kernel_us": {k_: v * 1e3 for k_, v in kern.items()},
           "active_experts": int(len(layer.touched_experts())),
           "path": path_name, "launches": 1 if single else 5}
    del handles, copies
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, layer


def attn_bytes(st) -> dict:
    """Algorithmic HBM bytes of one attention step: every cached key and value
    the step's queries can see read once (one byte each, the step's own
    tokens included), the appended codes written, the new keys and values,
    the queries and the outputs moved once."""
    R, T, Hq, Hkv, D, C = st.shape
    kv = int(sum(int(L) + T for L in st.past_len)) * Hkv * D * 2
    append = R * T * Hkv * D * (2 * 2 + 2)      # bf16 k, v in; E4M3 k, v out
    qo = R * T * Hq * D * (2 + 4)               # bf16 queries in, fp32 outputs out
    return {"kv_read": kv, "append": append, "q_out": qo, "step": kv + append + qo}


def time_attention(name, steps, warmup):
    """One attention step (one launch: the step's keys and values appended, then
    attention over the cache in tiles of 256 positions) of a named
    workload, rotated over device-side copies of its KV cache (>= 1 GB in
    total, so no step finds its cache in the Infinity Cache), timed by
    replaying one HIP graph holding one step of every copy."""
    import torch
    from decode_step_moe_amd import attention as at
    from synth import attn_gen
    from synth.device import bf16_tensor, f32_tensor

    st = attn_gen.draw_workload(name, seed=3)
    R, T, Hq, Hkv, D, C = st.shape
    nb = attn_bytes(st)
    per_copy = 2 * R * Hkv * C * D
    n = max(4, int(np.ceil(1.0e9 / per_copy)))
    log(f"[bench] attention {name}: {nb['step'] / 1e6:.2f} MB/step, {n} cache copies")
    cfg = at.make_attn_config(Hq, Hkv, T, R, C, st.softmax_scale)
    d = "cuda"
    q, kn, vn = (bf16_tensor(a, d) for a in (st.q, st.k_new, st.v_new))
    kc0 = torch.from_numpy(np.ascontiguousarray(st.k_cache)).to(d)
    vc0 = torch.from_numpy(np.ascontiguousarray(st.v_cache)).to(d)
    kc = kc0.repeat(n, 1, 1, 1)
    vc = vc0.repeat(n, 1, 1, 1)
    ks, vs = f32_tensor(st.k_scale, d), f32_tensor(st.v_scale, d)
    past = torch.from_numpy(np.ascontiguousarray(st.past_len)).to(d)
    outs = [torch.empty((R, T, Hq, D), device=d) for _ in range(n)]
    ws = torch.zeros(at.workspace_bytes(cfg), dtype=torch.uint8, device=d)
    mp = int(st.past_len.max())
    ios = [at.make_io(cfg, past, mp, q, kn, vn, kc[i * R:(i + 1) * R], vc[i * R:(i + 1) * R], ks, vs, outs[i], ws)
           for i in range(n)]
    stream = torch.cuda.current_stream()
    for i in range(n):
        at.step_io(cfg, ios[i], stream)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    assert bool(torch.isfinite(outs[0]).all())

    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(warmup):
        at.step_io(cfg, ios[i % n], stream)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        at.step_io(cfg, ios[i % n], stream)
    t1.record(stream)
    torch.cuda.synchronize()
    eager_us = t0.elapsed_time(t1) / steps * 1e3
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(n):
            at.step_io(cfg, ios[i], side)
    torch.cuda.synchronize()
    reps = max(2, -(-steps // n))
    g.replay()
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    graph_us = t0.elapsed_time(t1) / (reps * n) * 1e3
    ref = outs[0].clone()
    assert torch.equal(outs[0], ref)
    del g
    gbps = nb["step"] / (graph_us * 1e-6) / 1e9
    res = {"workload": name, "requests": R, "tokens": T, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
           "cache_len": C, "mean_context": round(float(np.mean(st.past_len)) + T, 1), "copies": n,
           "graph_us": round(graph_us, 3), "eager_us": round(eager_us, 3), "launches_per_step": 1,
           "bytes": nb,
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "timing": "graph-replayed steps (one launch each), HIP events on the launching stream"}}
    del kc, vc, outs, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def _launch_probe(h, layer):
    """Names of the launches one step of this batch makes on handle `h`."""
    import torch
    from synth import device as sdev
    x, attn, resid = sdev.upload_inputs(layer)
    h.set_profiling(True)
    h.step(x, attn, resid)
    names = list(h.kernel_times_ms())
    h.set_profiling(False)
    torch.cuda.synchronize()
    return names


# ----------------------------------------------------------------- CPU baseline
def cpu_baseline(layer, budget_s=10.0):
    """The fp64 oracle as it stands, on a bounded sample of the same workload:
    full batch-1 layer-steps with one BLAS thread and with every core this
    process may run on, each the median of at least 5 timed steps within
    about budget_s / 2 seconds."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import decode_layer_ref as ref
    raw = layer.raw
    n_cores = len(os.sched_getaffinity(0))

    def one():
        ref.decode_step(raw.x, raw.attn, raw.resid, raw.w_qkv, raw.w_o, raw.gain, layer.w_router,
                        raw.expert, raw.s1, raw.s3, raw.s2, raw.shape.top_k)

    one()  # draws (and caches) the touched experts outside the timed sample
    res = {}
    for label, n_thr in (("one_thread", 1), ("all_cores", n_cores)):
        with threadpool_limits(limits=n_thr):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            times, t_start = [], time.perf_counter()
            while len(times) < 5 or time.perf_counter() - t_start < budget_s / 2:
                t0 = time.perf_counter()
                one()
                times.append(time.perf_counter() - t0)
                if len(times) >= 200:
                    break
        res[label] = {"us": float(np.median(times)) * 1e6, "steps": len(times), "threads": int(used)}
    # the faster of the two is the baseline (NumPy's threaded BLAS can lose to
    # one thread on these matrix-vector products); both are reported
    best = min(res, key=lambda k: res[k]["us"])
    b = res[best]
    return {"value": round(b["us"], 1), "unit": "us/layer-step", "cores": b["threads"], "kind": "oracle",
            "sample": f"median of {b['steps']} full layer-steps of the batch-1 TP16-shard workload "
                      f"(float64 NumPy, {b['threads']} BLAS thread(s)); the faster of one thread and "
                      f"all {n_cores} cores of the host",
            "one_thread_us": round(res["one_thread"]["us"], 1), "all_cores_us": round(res["all_cores"]["us"], 1),
            "all_cores_threads": res["all_cores"]["threads"], "host_cores": n_cores, "cpu": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--no-batches", action="store_true", help="headline workload only")
    ap.add_argument("--batches", default=",".join(str(c) for c in BATCH_CFGS),
                    help="workload ids measured under \"batches\" (comma-separated)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the rotation with cross-layer prefetch (so that a kernel trace holds "
                         "only standalone steps)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-attention", action="store_true", help="skip the attention-core workloads")
    ap.add_argument("--attention-only", action="store_true",
                    help="measure only the attention-core workloads and print their results")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run a few eager headline steps and a 1 GiB negate of known size "
                         "(for hardware-counter runs under rocprofv3 --pmc), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer-step is one tensor-parallel shard's work on one GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import decode_step_moe_amd  # noqa: F401  (fails loudly without the built library)

    if args.counter_pass:
        counter_pass(args.steps)
        return
    if args.attention_only:
        print(json.dumps({"attention": {n: time_attention(n, args.steps, args.warmup) for n in ATTN_WORKLOADS}}),
              flush=True)
        return
    head, layer = time_config(HEADLINE_CFG, args.steps, args.warmup, args.copies, chain=not args.no_chain)
    multi, _ = time_config(HEADLINE_CFG, args.steps, args.warmup, args.copies, want_kernels=False,
                           path=1)
    batches = {}
    if not args.no_batches:
        for c in [int(v) for v in args.batches.split(",") if v.strip()]:
            r, lay = time_config(c, max(20, args.steps // 2), args.warmup, None, chain=not args.no_chain)
            batches[r["workload"]] = _summary(r)
            if r["path"] == "batched":
                batches[r["workload"]]["mfma_util"] = mfma_util(lay, r["kernel_us"])
    us = head["graph_us"]
    b = head["bytes"]
    kern = head["kernel_us"]
    dom = max(kern, key=kern.get)
    # the kernel's average launch duration: when a step is exactly one launch
    # of it, the eager loop (K back-to-back launches between two HIP events on
    # its stream) gives it directly; otherwise the per-launch event pairs,
    # which add the event and dispatch gap (about 2 us) to each launch
    one_launch = head["launches"] == 1 and len(kern) == 1
    avg_us = head["graph_us"] if one_launch else kern[dom]
    achieved = b[dom] / (avg_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "hidden": 7168, "batch": 1, "qkv_out": 512,
                   "attn_dim": 512, "n_experts": 384, "top_k": 8, "expert_ffn": 128,
                   "shared_ffn": 128, "routing": "uniform-random", "timing": "hip-graph replay, one step of each rotated copy per graph",
                   "copies_rotated": head["copies"]},
        "hbm_gbps": round(b["step"] / (us * 1e-6) / 1e9, 1),
        "hbm_frac": round(b["step"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "tok_per_s_per_shard": round(1 / (us * 1e-6), 1),
        "eager_us": round(head["eager_us"], 3),
        "launches_per_step": head["launches"],
        "path": head["path"],
        "prefetch_chain_us": round(head["prefetch_chain_us"], 3) if head["prefetch_chain_us"] else None,
        "multi_launch_path": {"graph_us": round(multi["graph_us"], 3),
                              "eager_us": round(multi["eager_us"], 3), "launches_per_step": 5},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": counted_traffic(dom, head["workload"]), "bytes_per_launch": b[dom],
                     "avg_launch_us": round(avg_us, 3),
                     "timing": "graph-replayed steps, one launch of this kernel each, between HIP events "
                               "on the launching stream" if one_launch else "HIP events around each launch"},
        "kernels_us": {k_: round(v, 3) for k_, v in kern.items()},
        "batches": batches,
    }
    if not args.no_attention:
        line["attention"] = {n: time_attention(n, args.steps, args.warmup) for n in ATTN_WORKLOADS}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(layer, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def counter_pass(steps):
    """Eager steps of the batch-1 and batch-64 workloads, then a plain
    elementwise pass of known size.

    Under `rocprofv3 --pmc FETCH_SIZE` (then WRITE_SIZE) the negate reads and
    writes exactly COPY_BYTES each; the ratio of its counter to that size is
    the factor that turns a layer-step kernel's counter into HBM bytes."""
    import torch
    from decode_step_moe_amd import DecodeLayer
    from synth import device as sdev, routing, gen

    for cfg_id in (HEADLINE_CFG, 3):
        raw = gen.draw(cfg_id)
        layer = routing.shape_router(raw, routing.stored_h(cfg_id))
        n_copies = max(4, int(np.ceil(1.0e9 / algorithmic_bytes(layer)["step"])))
        copies = make_copies(layer, n_copies)
        handles = [DecodeLayer(sdev.config_of(layer), w) for w in copies]
        x, attn, resid = sdev.upload_inputs(layer)
        outs = [h.alloc_outputs(layer.shape.batch) for h in handles]
        ios = [h.make_io(x, attn, resid, o) for h, o in zip(handles, outs)]
        stream = torch.cuda.current_stream()
        for i in range(max(steps, n_copies)):
            handles[i % n_copies].step_io(ios[i % n_copies], stream)
        torch.cuda.synchronize()
        for h in handles:
            assert h.status() == 0
        log(f"[counter-pass] {layer.shape.name}: {max(steps, n_copies)} layer-steps over {n_copies} copies")
        del handles, copies, outs, ios
        torch.cuda.empty_cache()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[counter-pass] 3 negates of {COPY_BYTES} bytes")


COPY_BYTES = 1 << 30

# Sources each measured kernel is built from: a counter summary applies to
# the kernel only while these files are unchanged.
KERNEL_SOURCES = {
    "single_launch_step": ("fused.hip", "common.h", "kernels.h"),
    "batched_gateup": ("batched.hip", "common.h", "kernels.h"),
    "batched_down": ("batched.hip", "common.h", "kernels.h"),
}


def _code_only(text: str) -> str:
    """The source without comments, trailing blanks and empty lines (the kernel
    sources hold no comment markers inside string literals), so that edits to
    comments alone do not retire a counter summary."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "decode_step_moe_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def counted_traffic(kernel, workload):
    """HBM bytes per launch from the committed hardware-counter summary of this
    kernel and workload, or None if there is none or the kernel has changed."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}.txt")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return int(fields["hbm_bytes_per_launch"])


def _summary(r):
    us = r["graph_us"]
    return {"batch": r["batch"], "graph_us": round(us, 3), "eager_us": round(r["eager_us"], 3),
            "hbm_gbps": round(r["bytes"]["step"] / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(r["bytes"]["step"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "tok_per_s_per_shard": round(r["batch"] / (us * 1e-6), 1),
            "active_experts": r["active_experts"], "copies": r["copies"],
            "path": r["path"], "launches_per_step": r["launches"],
            "prefetch_chain_us": round(r["prefetch_chain_us"], 3) if r["prefetch_chain_us"] else None,
            "kernels_us": {k_: round(v, 3) for k_, v in r["kernel_us"].items()},
            "kernels_gbps": {k_: round(r["bytes"][k_] / (v * 1e-6) / 1e9, 1)
                             for k_, v in r["kernel_us"].items() if k_ in r["bytes"]}}


if __name__ == "__main__":
    main()
