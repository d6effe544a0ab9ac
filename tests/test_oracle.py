"""Pins for the CPU oracle (oracle/decode_layer_ref.py), CPU only.

Each pin ties the oracle to something other than itself:
  * brute force on tiny inputs with pure-Python loops and the math module
    (projections, residual, router, top-k by rank counting, SwiGLU, the whole
    step);
  * closed forms (RMSNorm of a constant row, sigmoid/SiLU at log 3 and 0);
  * invariants (unit RMS before the gain, weights sum to one, monotone
    weights, permutation equivariance, batch = single-token runs);
  * special cases that reduce to a library routine (k = 1 gives a dense
    single-expert SwiGLU computed with torch float64 on the CPU; k = E).
The mutation test at the end plants plausible mistakes in the oracle, on the
CPU, and checks that at least one pin catches each.
"""
import itertools
import math
import random

import numpy as np
import pytest
import torch

from oracle import decode_layer_ref as ref
from synth import gen


# ---------------------------------------------------------------- helpers
def rand_bf16(rng, shape, std=1.0, mean=0.0):
    return gen.f32_to_bf16_bits(rng.normal(mean, std, size=shape).astype(np.float32))


def bits_val(b):
    """Independent scalar widening: sign/exponent/mantissa of a bf16 pattern."""
    b = int(b)
    sign = -1.0 if b & 0x8000 else 1.0
    ex = (b >> 7) & 0xFF
    man = b & 0x7F
    if ex == 0:
        return sign * man * 2.0 ** (-133)
    return sign * (1.0 + man / 128.0) * 2.0 ** (ex - 127)


def py_matvec_rows(act_bits_or_vals, w_bits, act_is_bits=True):
    """out[t][j] = sum_i a[t][i] * W[j][i], pure Python."""
    a = [[bits_val(v) if act_is_bits else float(v) for v in row] for row in act_bits_or_vals]
    W = [[bits_val(v) for v in row] for row in w_bits]
    return [[math.fsum(a[t][i] * W[j][i] for i in range(len(a[t]))) for j in range(len(W))]
            for t in range(len(a))]


def py_sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z)) if z > -700 else 0.0


def py_ffn(v, w1, w3, w2):
    F = len(w1)
    u = [math.fsum(v[i] * bits_val(w1[f][i]) for i in range(len(v))) for f in range(F)]
    g = [math.fsum(v[i] * bits_val(w3[f][i]) for i in range(len(v))) for f in range(F)]
    a = [u[f] * py_sigmoid(u[f]) * g[f] for f in range(F)]
    return [math.fsum(a[f] * bits_val(w2[i][f]) for f in range(F)) for i in range(len(w2))]


def py_topk_by_rank(logits_row, k):
    """Rank counting (no sort): rank(e) = #experts strictly ahead of e."""
    l32 = [float(np.float32(v)) for v in logits_row]
    E = len(l32)
    rank = [sum(1 for o in range(E) if l32[o] > l32[e] or (l32[o] == l32[e] and o < e))
            for e in range(E)]
    chosen = [None] * k
    for e in range(E):
        if rank[e] < k:
            chosen[rank[e]] = e
    s = [py_sigmoid(logits_row[e]) for e in chosen]
    tot = math.fsum(s)
    return chosen, [v / tot for v in s]


def tiny_layer(seed=0, B=3, H=16, Dq=5, Do=6, E=4, k=2, F=8, Fs=8):
    rng = np.random.default_rng(seed)
    L = dict(
        x=rand_bf16(rng, (B, H)), attn=rand_bf16(rng, (B, Do)),
        resid=rng.normal(0, 1, (B, H)).astype(np.float32),
        w_qkv=rand_bf16(rng, (Dq, H), 0.3), w_o=rand_bf16(rng, (H, Do), 0.3),
        gain=rand_bf16(rng, (H,), 0.3, 1.0),
        w_router=rng.normal(0, 0.5, (E, H)).astype(np.float32),
        experts={e: (rand_bf16(rng, (F, H), 0.3), rand_bf16(rng, (F, H), 0.3),
                     rand_bf16(rng, (H, F), 0.3)) for e in range(E)},
        s1=rand_bf16(rng, (Fs, H), 0.3), s3=rand_bf16(rng, (Fs, H), 0.3),
        s2=rand_bf16(rng, (H, Fs), 0.3), k=k)
    return L


def run_oracle(L):
    return ref.decode_step(L["x"], L["attn"], L["resid"], L["w_qkv"], L["w_o"], L["gain"],
                           L["w_router"], lambda e: L["experts"][e], L["s1"], L["s3"], L["s2"],
                           L["k"])


def py_step(L):
    """The whole step by brute force, pure Python, written from the definitions."""
    B, H = L["resid"].shape
    qkv = py_matvec_rows(L["x"], L["w_qkv"])
    o = py_matvec_rows(L["attn"], L["w_o"])
    r1 = [[float(L["resid"][t][i]) + o[t][i] for i in range(H)] for t in range(B)]
    gain = [bits_val(v) for v in L["gain"]]
    h = []
    for t in range(B):
        ms = math.fsum(v * v for v in r1[t]) / H
        h.append([gain[i] * r1[t][i] / math.sqrt(ms + 1e-6) for i in range(H)])
    Wr = [[float(v) for v in row] for row in L["w_router"]]
    logits = [[math.fsum(h[t][i] * Wr[e][i] for i in range(H)) for e in range(len(Wr))]
              for t in range(B)]
    y, idx_all, w_all = [], [], []
    for t in range(B):
        idx, w = py_topk_by_rank(logits[t], L["k"])
        yt = py_ffn(h[t], L["s1"], L["s3"], L["s2"])
        for e, we in zip(idx, w):
            z = py_ffn(h[t], *L["experts"][e])
            yt = [yt[i] + we * z[i] for i in range(H)]
        y.append(yt)
        idx_all.append(idx)
        w_all.append(w)
    return dict(qkv=qkv, resid_out=r1, h=h, logits=logits, topk_idx=idx_all,
                topk_w=w_all, moe_out=y)


def close(a, b, rtol=1e-12, atol=1e-12):
    np.testing.assert_allclose(np.asarray(a, np.float64), np.asarray(b, np.float64),
                               rtol=rtol, atol=atol)


# ---------------------------------------------------------------- pins
def pin_bf16_widening():
    pats = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x3EAA, 0x8000, 0x4049], np.uint16)
    got = ref.bf16_to_f64(pats)
    want = [bits_val(p) for p in pats]
    assert list(got) == want
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0 ** -133


def pin_projection_bruteforce():
    rng = np.random.default_rng(1)
    x, w = rand_bf16(rng, (3, 16)), rand_bf16(rng, (5, 16), 0.3)
    close(ref.attention_input_projection(x, w), py_matvec_rows(x, w))


def pin_out_projection_residual_bruteforce():
    rng = np.random.default_rng(2)
    attn, wo = rand_bf16(rng, (3, 6)), rand_bf16(rng, (16, 6), 0.3)
    r = rng.normal(0, 1, (3, 16)).astype(np.float32)
    o = py_matvec_rows(attn, wo)
    want = [[float(r[t][i]) + o[t][i] for i in range(16)] for t in range(3)]
    close(ref.out_projection_residual(attn, wo, r), want)
    # zero attention output leaves the residual unchanged
    close(ref.out_projection_residual(np.zeros_like(attn), wo, r), r.astype(np.float64), 0, 0)


def pin_rmsnorm_closed_form():
    H = 32
    rng = np.random.default_rng(3)
    g = rand_bf16(rng, (H,), 0.3, 1.0)
    gv = np.array([bits_val(v) for v in g])
    for c in (2.5, -0.75, 1e-4, 3e-3):
        h, ms = ref.rms_norm(np.full((1, H), c), g)
        close(ms, [c * c], 1e-15, 0)
        close(h[0], gv * c / math.sqrt(c * c + 1e-6), 1e-13, 0)


def pin_rmsnorm_unit_rms_invariant():
    rng = np.random.default_rng(4)
    r1 = rng.normal(0, 1, (4, 64)) * np.array([[1.0], [1e-3], [50.0], [0.02]])
    ones = gen.f32_to_bf16_bits(np.ones(64, np.float32))
    h, ms = ref.rms_norm(r1, ones)
    rms = np.sqrt(np.mean(h * h, axis=1))
    close(rms, np.sqrt(ms / (ms + 1e-6)), 1e-13, 0)
    close(ms, [math.fsum(v * v for v in row) / 64 for row in r1], 1e-13, 0)


def pin_router_bruteforce():
    rng = np.random.default_rng(5)
    h = rng.normal(0, 1, (3, 16))
    wr = rng.normal(0, 0.5, (4, 16)).astype(np.float32)
    want = [[math.fsum(h[t][i] * float(wr[e][i]) for i in range(16)) for e in range(4)]
            for t in range(3)]
    close(ref.router_logits(h, wr), want)


def pin_sigmoid_silu_closed_forms():
    close(ref.sigmoid([0.0, math.log(3.0), -math.log(3.0)]), [0.5, 0.75, 0.25], 1e-15, 0)
    close(ref.silu([0.0, math.log(3.0), 40.0]), [0.0, 0.75 * math.log(3.0), 40.0], 1e-15, 0)
    assert abs(ref.silu([-800.0])[0]) == 0.0


def pin_topk_bruteforce_and_invariants():
    rng = np.random.default_rng(6)
    for E, k in ((8, 2), (9, 3), (5, 5), (7, 1)):
        logits = rng.normal(0, 2, (4, E))
        idx, w = ref.select_experts(logits, k)
        for t in range(4):
            bi, bw = py_topk_by_rank(list(logits[t]), k)
            assert list(idx[t]) == bi
            close(w[t], bw, 1e-14, 0)
        close(w.sum(axis=1), np.ones(4), 1e-14, 0)
        assert np.all(w > 0) and np.all(w <= 1)
        assert np.all(np.diff(w, axis=1) <= 0)
        if k == 1:
            close(w, np.ones((4, 1)), 0, 0)
        if k == E:
            s = 1 / (1 + np.exp(-logits))
            close(np.take_along_axis(s / s.sum(1, keepdims=True), idx, 1), w, 1e-14, 0)
    # ties resolve to the lower expert id; equal after float32 rounding counts as a tie
    l = np.array([[1.0, 3.0, 3.0, 2.0, 3.0 + 1e-12]])
    idx, _ = ref.select_experts(l, 3)
    assert list(idx[0]) == [1, 2, 4]


def pin_swiglu_bruteforce():
    rng = np.random.default_rng(7)
    v = rng.normal(0, 1, (2, 16))
    w1, w3, w2 = rand_bf16(rng, (8, 16), 0.3), rand_bf16(rng, (8, 16), 0.3), rand_bf16(rng, (16, 8), 0.3)
    want = [py_ffn(list(v[t]), w1, w3, w2) for t in range(2)]
    close(ref.swiglu_ffn(v, w1, w3, w2), want, 1e-12, 1e-13)


def pin_one_hot_equals_dense_expert():
    """k = 1: y - FFN_shared(h) equals a dense single-expert SwiGLU (torch f64)."""
    L = tiny_layer(seed=8, B=4, k=1)
    out = run_oracle(L)
    h = torch.tensor(out["h"], dtype=torch.float64)

    def tffn(w1, w3, w2):
        t = lambda b: torch.tensor(gen.bf16_bits_to_f32(b), dtype=torch.float64)
        return torch.nn.functional.silu(h @ t(w1).T) * (h @ t(w3).T) @ t(w2).T

    shared = tffn(L["s1"], L["s3"], L["s2"]).numpy()
    for t in range(4):
        e = int(out["topk_idx"][t][0])
        dense = tffn(*L["experts"][e]).numpy()[t]
        close(out["moe_out"][t] - shared[t], dense, 1e-11, 1e-13)
        assert out["topk_w"][t][0] == 1.0


def pin_whole_step_bruteforce():
    for seed, k in ((9, 2), (10, 3)):
        L = tiny_layer(seed=seed, k=k)
        out, want = run_oracle(L), py_step(L)
        for key in ("qkv", "resid_out", "h", "logits", "moe_out"):
            close(out[key], want[key], 1e-11, 1e-12)
        assert [list(r) for r in out["topk_idx"]] == want["topk_idx"]
        close(out["topk_w"], want["topk_w"], 1e-13, 0)


def pin_permutation_and_batch_split():
    L = tiny_layer(seed=11, B=4, k=2)
    out = run_oracle(L)
    perm = np.array([2, 0, 3, 1])
    P = dict(L)
    for key in ("x", "attn", "resid"):
        P[key] = L[key][perm]
    outp = run_oracle(P)
    for key in ("qkv", "resid_out", "logits", "moe_out"):
        close(outp[key], out[key][perm], 1e-13, 1e-14)
    for t in range(4):
        S = dict(L)
        for key in ("x", "attn", "resid"):
            S[key] = L[key][t:t + 1]
        o1 = run_oracle(S)
        for key in ("qkv", "resid_out", "logits", "moe_out"):
            close(o1[key][0], out[key][t], 1e-13, 1e-14)
        assert list(o1["topk_idx"][0]) == list(out["topk_idx"][t])


PINS = [pin_bf16_widening, pin_projection_bruteforce, pin_out_projection_residual_bruteforce,
        pin_rmsnorm_closed_form, pin_rmsnorm_unit_rms_invariant, pin_router_bruteforce,
        pin_sigmoid_silu_closed_forms, pin_topk_bruteforce_and_invariants,
        pin_swiglu_bruteforce, pin_one_hot_equals_dense_expert, pin_whole_step_bruteforce,
        pin_permutation_and_batch_split]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------- mutations
def _m_eps_outside(r1, gain_bits, eps=1e-6):
    r1 = np.asarray(r1, np.float64)
    ms = np.mean(r1 * r1, axis=1)
    return ref.bf16_to_f64(gain_bits)[None] * r1 / (np.sqrt(ms) + eps)[:, None], ms


def _m_layernorm(r1, gain_bits, eps=1e-6):
    r1 = np.asarray(r1, np.float64)
    c = r1 - r1.mean(axis=1, keepdims=True)
    ms = np.mean(c * c, axis=1)
    return ref.bf16_to_f64(gain_bits)[None] * c / np.sqrt(ms + eps)[:, None], ms


def _m_no_gain(r1, gain_bits, eps=1e-6):
    r1 = np.asarray(r1, np.float64)
    ms = np.mean(r1 * r1, axis=1)
    return r1 / np.sqrt(ms + eps)[:, None], ms


def _m_sigmoid_sign(z):
    return 1.0 / (1.0 + np.exp(np.asarray(z, np.float64)))


def _m_softmax_select(logits, k):
    l = np.asarray(logits, np.float64)
    idx = np.argsort(-l, axis=1, kind="stable")[:, :k]
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    w = np.take_along_axis(p, idx, 1)
    return idx, w / w.sum(1, keepdims=True)


def _m_no_renorm(logits, k):
    l = np.asarray(logits, np.float64)
    idx = np.argsort(-l, axis=1, kind="stable")[:, :k]
    return idx, ref.sigmoid(np.take_along_axis(l, idx, 1))


def _m_ascending(logits, k):
    l = np.asarray(logits, np.float64)
    idx = np.argsort(l, axis=1, kind="stable")[:, :k]
    s = ref.sigmoid(np.take_along_axis(l, idx, 1))
    return idx, s / s.sum(1, keepdims=True)


def _m_tie_high(logits, k):
    l = np.asarray(logits, np.float64).astype(np.float32)
    E = l.shape[1]
    idx = (E - 1 - np.argsort(-l[:, ::-1], axis=1, kind="stable"))[:, :k]
    s = ref.sigmoid(np.take_along_axis(np.asarray(logits, np.float64), idx, 1))
    return idx, s / s.sum(1, keepdims=True)


def _m_silu_on_up(v, w_gate, w_up, w_down):
    v = np.asarray(v, np.float64)
    u = v @ ref.bf16_to_f64(w_gate).T
    g = v @ ref.bf16_to_f64(w_up).T
    return (u * ref.silu(g)) @ ref.bf16_to_f64(w_down).T


def _m_relu_ffn(v, w_gate, w_up, w_down):
    v = np.asarray(v, np.float64)
    u = v @ ref.bf16_to_f64(w_gate).T
    g = v @ ref.bf16_to_f64(w_up).T
    return (np.maximum(u, 0) * g) @ ref.bf16_to_f64(w_down).T


def _m_no_shared(h, idx, w, expert, s1, s3, s2):
    return ref.__dict__["_orig_moe"](h, idx, w, expert, s1[:0], s3[:0], s2[:, :0])


def _m_unweighted(h, idx, w, expert, s1, s3, s2):
    return ref.__dict__["_orig_moe"](h, idx, np.ones_like(np.asarray(w)), expert, s1, s3, s2)


def _m_no_residual(attn_bits, w_o_bits, resid):
    return ref.bf16_to_f64(attn_bits) @ ref.bf16_to_f64(w_o_bits).T


def _m_router_bf16_h(h, w_router):
    hb = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(np.asarray(h, np.float32))).astype(np.float64)
    return hb @ np.asarray(w_router, np.float64).T


def _m_widen_truncate_sign(bits):
    b = np.asarray(bits, np.uint16) & np.uint16(0x7FFF)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


MUTATIONS = [
    ("rms_norm", _m_eps_outside), ("rms_norm", _m_layernorm), ("rms_norm", _m_no_gain),
    ("sigmoid", _m_sigmoid_sign), ("select_experts", _m_softmax_select),
    ("select_experts", _m_no_renorm), ("select_experts", _m_ascending),
    ("select_experts", _m_tie_high), ("swiglu_ffn", _m_silu_on_up),
    ("swiglu_ffn", _m_relu_ffn), ("moe_output", _m_no_shared), ("moe_output", _m_unweighted),
    ("out_projection_residual", _m_no_residual), ("router_logits", _m_router_bf16_h),
    ("bf16_to_f64", _m_widen_truncate_sign),
]


@pytest.mark.parametrize("attr,bad", MUTATIONS, ids=lambda v: getattr(v, "__name__", v))
def test_pins_catch_planted_mistake(monkeypatch, attr, bad):
    monkeypatch.setitem(ref.__dict__, "_orig_moe", ref.moe_output)
    monkeypatch.setattr(ref, attr, bad)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake in {attr}"
