"""GPU parity of the decode attention core (FP8 E4M3 KV cache, speculative
verify masking) against the fp64 oracle, through the C ABI.

Gates, from the kernel's arithmetic: the appended cache codes bit-exact (the
code is decided in fp32 on both sides); the outputs within max-abs 2e-3 and
relative L2 1e-4 of the oracle.  Scores are exact bf16 x bf16 products summed
in fp32 over 128 terms, P enters the P V product as bf16 hi + lo (relative
error <= 2^-16 per element) and V is exact in bf16, so the expected error is
~1e-5 relative; sums over up to 8k positions in fp32 stay well inside 1e-4.
Every output buffer starts NaN, every unused cache byte is random (NaN codes
included), so an unwritten output or a read beyond a request's positions shows.
"""
import zlib

import numpy as np
import pytest
import torch

from oracle import attention_ref as ref
from synth import attn_gen
from synth.device import bf16_tensor, f32_tensor
from tests.parity import rel_l2, say

pytestmark = pytest.mark.gpu

ATT_MAX_ABS = 2e-3
ATT_REL_L2 = 1e-4


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_moe_amd  # noqa: F401  (raises if the library was not built)


def _at():
    from decode_step_moe_amd import attention as at
    return at


class Dev:
    """One step's device buffers (outputs poisoned with NaN) and its workspace."""

    def __init__(self, st: attn_gen.AttnStep, max_tokens=None, max_requests=None, max_past=None, max_splits=0,
                 with_bf16=False):
        at = _at()
        R, T, Hq, Hkv, D, C = st.shape
        self.cfg = at.make_attn_config(Hq, Hkv, max_tokens or T, max_requests or R, C, st.softmax_scale,
                                       max_splits=max_splits)
        d = "cuda"
        self.q, self.k_new, self.v_new = (bf16_tensor(a, d) for a in (st.q, st.k_new, st.v_new))
        self.k_cache = torch.from_numpy(np.ascontiguousarray(st.k_cache)).to(d)
        self.v_cache = torch.from_numpy(np.ascontiguousarray(st.v_cache)).to(d)
        if (max_requests or R) > R:   # the cache is sized for max_requests
            pad = (max_requests - R, Hkv, C, D)
            self.k_cache = torch.cat([self.k_cache, torch.zeros(pad, dtype=torch.uint8, device=d)])
            self.v_cache = torch.cat([self.v_cache, torch.zeros(pad, dtype=torch.uint8, device=d)])
        self.k_scale, self.v_scale = f32_tensor(st.k_scale, d), f32_tensor(st.v_scale, d)
        self.past = torch.from_numpy(np.ascontiguousarray(st.past_len, np.int32)).to(d)
        self.out = torch.full((R, T, Hq, D), float("nan"), device=d)
        self.out_bf16 = torch.full((R, T, Hq, D), float("nan"), dtype=torch.bfloat16, device=d) if with_bf16 else None
        self.ws = torch.zeros(at.workspace_bytes(self.cfg), dtype=torch.uint8, device=d)
        mp = int(st.past_len.max()) if max_past is None else max_past
        self.io = at.make_io(self.cfg, self.past, mp, self.q, self.k_new, self.v_new, self.k_cache,
                             self.v_cache, self.k_scale, self.v_scale, self.out, self.ws, self.out_bf16)

    def step(self):
        _at().step_io(self.cfg, self.io)

    def results(self):
        torch.cuda.synchronize()
        return self.out.cpu().numpy(), self.k_cache.cpu().numpy(), self.v_cache.cpu().numpy()


def expect(st):
    return ref.decode_attention(st.q, st.k_new, st.v_new, st.k_cache, st.v_cache, st.past_len, st.k_scale,
                                st.v_scale, st.softmax_scale)


def check_out(name, out, want):
    assert np.isfinite(out).all(), f"{name}: non-finite outputs at {np.argwhere(~np.isfinite(out))[:4]}"
    err = float(np.abs(out - want).max())
    rl = rel_l2(out, want)
    say(f"  {name}: max-abs {err:.2e}  rel-L2 {rl:.2e}")
    assert err <= ATT_MAX_ABS and rl <= ATT_REL_L2, name


def check_caches(name, kc, vc, want_k, want_v):
    for tag, got, want in (("k", kc, want_k), ("v", vc, want_v)):
        bad = np.argwhere(got[: want.shape[0]] != want)
        assert bad.size == 0, f"{name}: {tag} cache differs at {bad[:4].tolist()} " \
                              f"(got {got[tuple(bad[0])]:#04x}, want {want[tuple(bad[0])]:#04x})"


def run_case(name, st, **kw):
    say(f"attention {name}: shape R,T,Hq,Hkv,D,C={st.shape} past={st.past_len[:8].tolist()}")
    dev = Dev(st, **kw)
    dev.step()
    out, kc, vc = dev.results()
    want, wk, wv = expect(st)
    check_caches(name, kc, vc, wk, wv)
    check_out(name, out, want)


@pytest.mark.parametrize("name,R,T,Hq,Hkv,C,lo,hi", [
    ("decode_T1", 5, 1, 4, 1, 1024, 0, 1000),
    ("verify_T8", 3, 8, 4, 1, 1200, 300, 1150),
    ("verify_T4", 4, 4, 4, 1, 700, 1, 690),
    ("gqa_16rows", 2, 4, 8, 2, 600, 100, 590),       # 4 heads per KV head x 4 tokens = one full row tile
    ("gqa_32rows", 2, 4, 16, 2, 600, 100, 590),      # 8 x 4 = 32 rows, the envelope
    ("mha_T8", 2, 8, 3, 3, 520, 0, 500),             # one query head per KV head
    ("gqa_T1_wide", 3, 1, 32, 1, 400, 10, 390),      # 32 query heads on one KV head
])
def test_parity(name, R, T, Hq, Hkv, C, lo, hi):
    run_case(name, attn_gen.draw(R, T, Hq, Hkv, C, lo, hi, seed=zlib.crc32(name.encode()) % 1000))


@pytest.mark.parametrize("name,R,T,Hq,Hkv,C,lo,hi,splits", [
    ("one_wg_12_tiles", 2, 8, 4, 1, 3000, 2700, 2990, 1),     # one workgroup loops 12 tiles, no combine
    ("splits_of_3", 3, 8, 4, 1, 3000, 1500, 2990, 5),         # 3 tiles per workgroup, ragged last split
    ("splits_32rows", 2, 4, 16, 2, 2100, 1000, 2090, 3),      # 32 rows with the prefetching loop
    ("splits_T1", 4, 1, 4, 1, 2600, 600, 2590, 2),
])
def test_multi_tile_splits(name, R, T, Hq, Hkv, C, lo, hi, splits):
    """Workgroups that take several tiles (forced through max_splits)."""
    run_case(name, attn_gen.draw(R, T, Hq, Hkv, C, lo, hi, seed=zlib.crc32(name.encode()) % 1000),
             max_splits=splits)


def test_long_context_beyond_64_tiles():
    """More tiles than partial slots: the automatic split takes 2+ tiles each."""
    st = attn_gen.draw(1, 8, 4, 1, 20480, 20000, 20470, seed=16)
    run_case("long_ctx_20k", st)


def test_chunk_boundaries():
    """Past lengths around multiples of the 256-position chunk, and zero."""
    past = [0, 1, 247, 248, 249, 255, 256, 257, 504, 511, 512, 760]
    st = attn_gen.draw(len(past), 8, 4, 1, 800, 0, 792, seed=7, past=past)
    run_case("chunk_boundaries", st)


def test_all_past_zero():
    st = attn_gen.draw(3, 8, 4, 1, 64, 0, 0, seed=8, past=[0, 0, 0])
    run_case("past_zero", st)


def test_fewer_tokens_than_max():
    """n_tokens below max_tokens, and n_requests below max_requests."""
    st = attn_gen.draw(3, 3, 4, 1, 900, 100, 880, seed=9)
    run_case("T3_of_8", st, max_tokens=8, max_requests=6)


def test_max_past_above_lengths():
    """A host bound well above the real lengths: the extra chunks return at once."""
    st = attn_gen.draw(2, 2, 4, 1, 2048, 10, 300, seed=10)
    run_case("loose_max_past", st, max_past=2040)


def test_bad_past_len_gives_nan_and_writes_nothing():
    past = [40, 200, -1, 60]          # 200 > max_past and -1: impossible lengths
    st = attn_gen.draw(4, 2, 4, 1, 256, 0, 100, seed=11, past=[40, 0, 0, 60])
    st.past_len = np.asarray(past, np.int32)
    say("attention bad_past_len: past=" + str(past))
    dev = Dev(st, max_past=100)
    dev.step()
    out, kc, vc = dev.results()
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    np.testing.assert_array_equal(kc[1:3], st.k_cache[1:3])
    np.testing.assert_array_equal(vc[1:3], st.v_cache[1:3])
    ok = [0, 3]
    want, wk, wv = ref.decode_attention(st.q[ok], st.k_new[ok], st.v_new[ok], st.k_cache[ok], st.v_cache[ok],
                                        st.past_len[ok], st.k_scale, st.v_scale, st.softmax_scale)
    check_caches("bad_past_len", kc[ok], vc[ok], wk, wv)
    check_out("bad_past_len", out[ok], want)


def _special_values() -> np.ndarray:
    """fp32 values that probe every rounding decision of the E4M3 encode at
    scale 1: every finite code's value, every midpoint between neighbours and
    one bf16 step either side of it, values past 448, tiny values, zeros."""
    vals = ref.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    def bf16_steps(x):
        b = (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.int64)
        return [((b + d).astype(np.uint32) << 16).view(np.float32) for d in (-1, 1)]
    extra = np.array([448 + 16, 470, 480, 500, 10240, 2.0 ** 127, np.inf, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -12,
                      2.0 ** -126, 0.0], np.float32)
    pos = np.concatenate([vals, mids, *bf16_steps(mids), *bf16_steps(vals[1:]), extra]).astype(np.float32)
    return np.concatenate([pos, -pos, [np.nan, -np.nan]]).astype(np.float32)


def test_quantisation_codes_bit_exact():
    """The appended codes for the rounding-decision probes (scale 1)."""
    from synth.gen import f32_to_bf16_bits
    special = _special_values()
    R, T, Hkv = 2, 8, 1
    n = R * T * Hkv * 128
    assert special.size <= n
    st = attn_gen.draw(R, T, 4, Hkv, 64, 0, 50, seed=12)
    fill = np.resize(special, n)
    bits = f32_to_bf16_bits(fill)
    assert np.array_equal(((bits.astype(np.uint32) << 16).view(np.float32) == fill) | np.isnan(fill),
                          np.ones(n, bool)), "probe values must be exact in bf16"
    st.k_new = bits.reshape(R, T, Hkv, 128)
    st.v_new = bits[::-1].copy().reshape(R, T, Hkv, 128)
    st.k_scale = np.ones(Hkv, np.float32)
    st.v_scale = np.ones(Hkv, np.float32)
    say("attention quantisation probes: %d values" % special.size)
    dev = Dev(st)
    dev.step()
    _, kc, vc = dev.results()
    wk, wv = ref.append_kv(st.k_cache, st.v_cache, st.k_new, st.v_new, st.past_len, st.k_scale, st.v_scale)
    check_caches("quantisation", kc, vc, wk, wv)


def test_decode_loop_reuses_workspace():
    """Five steps in a row on one workspace, each appending at the end of the
    previous one (the arrival counters must return to zero every step)."""
    R, T, Hq, Hkv, C = 3, 4, 4, 1, 1100
    st = attn_gen.draw(R, T, Hq, Hkv, C, 230, 260, seed=13)
    dev = Dev(st, max_past=C - T)
    kc_ref, vc_ref = st.k_cache.copy(), st.v_cache.copy()
    past = st.past_len.copy()
    for s in range(5):
        nxt = attn_gen.draw(R, T, Hq, Hkv, C, 0, 0, seed=100 + s)
        say(f"attention decode_loop step {s}: past={past.tolist()}")
        dev.q.copy_(bf16_tensor(nxt.q, "cuda"))
        dev.k_new.copy_(bf16_tensor(nxt.k_new, "cuda"))
        dev.v_new.copy_(bf16_tensor(nxt.v_new, "cuda"))
        dev.past.copy_(torch.from_numpy(past))
        dev.out.fill_(float("nan"))
        dev.step()
        out, kc, vc = dev.results()
        want, kc_ref, vc_ref = ref.decode_attention(nxt.q, nxt.k_new, nxt.v_new, kc_ref, vc_ref, past, st.k_scale,
                                                    st.v_scale, st.softmax_scale)
        check_caches(f"decode_loop_{s}", kc, vc, kc_ref, vc_ref)
        check_out(f"decode_loop_{s}", out, want)
        past = past + T


def test_graph_replays():
    """A captured step replayed with fresh inputs, eager work and syncs between."""
    st = attn_gen.draw(4, 8, 4, 1, 1100, 500, 1000, seed=14)
    dev = Dev(st)
    base_k, base_v = dev.k_cache.clone(), dev.v_cache.clone()
    g = torch.cuda.CUDAGraph()
    say("attention graph: capture")
    with torch.cuda.graph(g):
        dev.step()
    for rep in range(3):
        nxt = attn_gen.draw(4, 8, 4, 1, 1100, 0, 0, seed=200 + rep)
        dev.q.copy_(bf16_tensor(nxt.q, "cuda"))
        dev.k_new.copy_(bf16_tensor(nxt.k_new, "cuda"))
        dev.v_new.copy_(bf16_tensor(nxt.v_new, "cuda"))
        dev.k_cache.copy_(base_k)
        dev.v_cache.copy_(base_v)
        dev.out.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"attention graph: replay {rep}")
        g.replay()
        out, kc, vc = dev.results()
        want, wk, wv = ref.decode_attention(nxt.q, nxt.k_new, nxt.v_new, st.k_cache, st.v_cache, st.past_len,
                                            st.k_scale, st.v_scale, st.softmax_scale)
        check_caches(f"graph_{rep}", kc, vc, wk, wv)
        check_out(f"graph_{rep}", out, want)
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("name", sorted(attn_gen.WORKLOADS))
def test_named_workloads_full_size(name):
    """The measured workloads at their full sizes, every output checked."""
    run_case(name, attn_gen.draw_workload(name, seed=3))


def test_zero_requests_is_a_noop():
    at = _at()
    st = attn_gen.draw(1, 1, 4, 1, 64, 0, 10, seed=15)
    dev = Dev(st)
    dev.io.n_requests = 0
    dev.step()
    out, kc, _ = dev.results()
    assert np.isnan(out).all()
    np.testing.assert_array_equal(kc, st.k_cache)
    assert at.check(dev.cfg, dev.io) == 0


def test_bf16_output_feeds_the_layer_step():
    """One decode step of a TP16 shard, attention into the MoE layer on the GPU:
    8 requests x 1 token (4 query heads on 1 KV head of 128, FP8 cache,
    contexts 100..4095, so some requests run in one workgroup and others are
    split and combined) write their output also as bf16, laid out as the
    layer step's attn input [8][512]; the layer step (batch 8) then reads
    that buffer as it is.  Checks: the bf16 output is the nearest-even
    rounding of the fp32 output (torch's CPU conversion), bit for bit; the
    fp32 output is within the attention gates of the attention oracle; the
    layer's outputs are within the layer gates of the layer oracle run on
    the same attn input."""
    import dataclasses  # noqa: F401
    from decode_step_moe_amd import DecodeLayer
    from synth import device as sdev, gen, routing
    from tests import parity, workload
    say("[attention -> layer step, TP16 shard, 8 requests x 1 token] start")
    st = attn_gen.draw(8, 1, 4, 1, 4096, 100, 4095, seed=91)
    dev = Dev(st, with_bf16=True)
    dev.step()
    out, _, _ = dev.results()
    check_out("attn_to_layer", out, expect(st)[0])
    ob = dev.out_bf16.cpu()
    want_bits = torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ob.view(torch.int16).numpy(), want_bits), "bf16 output is not out rounded to nearest even"
    # the layer step on that buffer (no copy: the attention's own output tensor)
    raw = gen.draw(2)
    assert raw.attn.shape == (8, 512)
    raw.attn = ob.view(torch.int16).numpy().view(np.uint16).reshape(8, 512)
    layer = routing.shape_router(raw, workload.oracle_h(raw))
    h = DecodeLayer(sdev.config_of(layer), sdev.upload_weights(layer))
    x, _, resid = sdev.upload_inputs(layer)
    res = h.alloc_outputs(8, with_h=True)
    h.step(x, dev.out_bf16.view(8, 512), resid, res)
    torch.cuda.synchronize()
    assert h.status() == 0
    got = {"qkv": res.qkv.cpu().numpy(), "resid_out": res.resid_out.cpu().numpy(),
           "logits": res.router_logits.cpu().numpy(), "topk_idx": res.topk_idx.cpu().numpy(),
           "topk_w": res.topk_w.cpu().numpy(), "moe_out": res.moe_out.cpu().numpy(),
           "h": res.h_out.cpu().numpy()}
    m = parity.compare(got, workload.expected(layer))
    say("[attention -> layer step] " + ", ".join(f"{k}={v:.3e}" for k, v in m.items() if k != "fails"))
    assert not m["fails"], m["fails"]


def random_attention_case(i: int):
    """Seeded random shape across the attention envelope: 1-16 requests, 1-8
    tokens, 1-4 KV heads with up to 32 query rows each, caches of 8-4096
    positions with past lengths anywhere below them (zero included), forced
    split counts now and then, and the bf16 copy of the output on half."""
    g = np.random.default_rng([0xA77E, i])
    T = int(g.integers(1, 9))
    grp = int(g.integers(1, 32 // T + 1))
    Hkv = int(g.choice([1, 1, 2, 3, 4]))
    R = int(g.integers(1, 17))
    C = int(g.choice([8, 64, 255, 256, 257, 1000, 2048, 4096])) if g.random() < 0.4 else int(g.integers(8, 4097))
    C = max(C, T)
    hi = int(g.integers(0, C - T + 1))
    lo = int(g.integers(0, hi + 1))
    splits = int(g.integers(1, 9)) if g.random() < 0.3 else 0
    return dict(R=R, T=T, Hq=grp * Hkv, Hkv=Hkv, C=C, lo=lo, hi=hi, splits=splits, bf16=bool(g.random() < 0.5))


@pytest.mark.parametrize("i", range(24))
def test_random_shapes(i):
    c = random_attention_case(i)
    name = f"rand{i}_R{c['R']}_T{c['T']}_Hq{c['Hq']}_Hkv{c['Hkv']}_C{c['C']}_past{c['lo']}-{c['hi']}_s{c['splits']}"
    st = attn_gen.draw(c["R"], c["T"], c["Hq"], c["Hkv"], c["C"], c["lo"], c["hi"], seed=100 + i)
    say(f"attention {name}: start")
    dev = Dev(st, max_splits=c["splits"], with_bf16=c["bf16"])
    dev.step()
    out, kc, vc = dev.results()
    want, wk, wv = expect(st)
    check_caches(name, kc, vc, wk, wv)
    check_out(name, out, want)
    if c["bf16"]:
        b = dev.out_bf16.float().cpu().numpy()
        assert np.array_equal(b, torch.from_numpy(out).to(torch.bfloat16).float().numpy()), name
