"""CPU oracle for one MoE decode layer-step: plain, slow, float64 throughout.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path imports,
calls or links this file.  It may be used only by tests/, by the smoke check
in __graft_entry__.py and by the CPU-baseline leg of bench.py.  It shares no
code with the HIP kernels (no common helpers, tables or constants).

What the step computes, and where each piece is stated:

  * The step's parts and their order - attention input projection, attention
    output projection with the residual work that follows it, router scoring,
    then shared and routed experts - are those of the vLLM decode backend for
    Kimi K3 described in bigchange.ai "Kimi K3 vLLM GPU inference benchmark",
    section "Where the time was going", and in wireai.ir "vLLM's speed jump on
    NVIDIA Blackwell servers; record 842 tokens/s for Kimi K3", section "Four
    key changes behind the jump" (bullets 1-3).
  * Neither page prints a formula.  The formulas below are the textbook forms
    named by the measured workload definitions: RMSNorm with eps 1e-6 and a
    gain; an fp32 router with sigmoid scores and top-k weights renormalised
    to sum to one; SwiGLU experts with gate W1, up W3 and down W2; one
    always-on shared expert of the same shape.  Every reading taken where
    the sources are silent is listed with its function.

Data conventions (shared with the GPU path only through this description):
  bf16 tensors arrive as uint16 bit patterns and are widened exactly;
  matrices are stored [out][in] (row j of W holds the weights of output j);
  every value is converted to float64 before any arithmetic and nothing is
  rounded afterwards, except that the top-k *decision* is taken on the
  logits rounded to float32 (the precision the GPU kernel decides in).

Parity pins: every function here is pinned by tests/test_oracle.py against
brute-force loops, closed forms or invariants; see the test file for the
list.  No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

RMS_EPS = 1e-6


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64(a) -> np.ndarray:
    """float32/float64 input -> float64 (exact)."""
    return np.asarray(a, dtype=np.float64)


# --- a1: attention input projection ---------------------------------------
def attention_input_projection(x_bits, w_qkv_bits) -> np.ndarray:
    """qkv[t, j] = sum_i x[t, i] * Wqkv[j, i].

    The projection into the attention block that the wireai.ir article
    ("Four key changes behind the jump", bullet 1) gives small-batch and
    split-K kernels; the math is one dense product either way.
    """
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_qkv_bits).T


# --- a2: out-projection + residual, then RMSNorm ---------------------------
def out_projection_residual(attn_bits, w_o_bits, resid) -> np.ndarray:
    """r1[t, i] = r[t, i] + sum_j attn[t, j] * Wo[i, j].

    wireai.ir, "Four key changes behind the jump", bullet 2: the output
    projection flows straight into the residual computation.  On one
    tensor-parallel shard the cross-GPU reduction between the two is the
    identity, so the residual adds this shard's own projection.
    """
    return f64(resid) + bf16_to_f64(attn_bits) @ bf16_to_f64(w_o_bits).T


def rms_norm(r1, gain_bits, eps: float = RMS_EPS):
    """h[t, i] = g[i] * r1[t, i] / sqrt(mean_i(r1[t, i]^2) + eps).

    The "residual work that follows" the out-projection (bigchange.ai, "Where
    the time was going") read as RMSNorm with gain; eps sits inside the
    square root, there is no mean subtraction and no bias.
    Returns (h, ms) with ms[t] = mean_i r1[t, i]^2.
    """
    r1 = f64(r1)
    ms = np.mean(r1 * r1, axis=1) if r1.shape[1] else np.zeros(r1.shape[0])
    inv = 1.0 / np.sqrt(ms + eps)
    return bf16_to_f64(gain_bits)[None, :] * r1 * inv[:, None], ms


# --- a3: router, sigmoid scores, top-k, renormalisation --------------------
def router_logits(h, w_router) -> np.ndarray:
    """l[t, e] = sum_i h[t, i] * Wr[e, i] with fp32 router weights.

    wireai.ir, "Four key changes behind the jump", bullet 3 (router scores).
    The router reads the unrounded normalised hidden state h.
    """
    return f64(h) @ f64(w_router).T


def sigmoid(z) -> np.ndarray:
    z = f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def select_experts(logits, k: int):
    """Top-k experts by sigmoid score, weights renormalised to sum to one.

    Readings: the score is sigmoid(l); no score bias, scaling factor or group
    limit.  Since sigmoid is monotone, ranking by score is ranking by logit.
    The ranking is taken on the logits rounded to float32, descending, ties
    to the lower expert id.  w[t, j] = s[t, idx[t, j]] / sum_j' s[t, idx[t, j']].
    Returns (idx int64 [B][k], w float64 [B][k]).
    """
    l64 = f64(logits)
    l32 = l64.astype(np.float32)
    idx = np.argsort(-l32, axis=1, kind="stable")[:, :k]
    s = sigmoid(np.take_along_axis(l64, idx, axis=1))
    w = s / s.sum(axis=1, keepdims=True)
    return idx.astype(np.int64), w


# --- a5/a6: SwiGLU experts --------------------------------------------------
def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z)."""
    z = f64(z)
    return z * sigmoid(z)


def swiglu_ffn(v, w_gate_bits, w_up_bits, w_down_bits) -> np.ndarray:
    """FFN(v) = Wdown @ (silu(Wgate @ v) * (Wup @ v)) for each row v of `v`.

    Gate W1 [F][H], up W3 [F][H], down W2 [H][F]; SiLU on the gate branch.
    """
    v = f64(v)
    u = v @ bf16_to_f64(w_gate_bits).T
    g = v @ bf16_to_f64(w_up_bits).T
    return (silu(u) * g) @ bf16_to_f64(w_down_bits).T


def moe_output(h, idx, w, expert, s1_bits, s3_bits, s2_bits) -> np.ndarray:
    """y[t] = FFN_shared(h[t]) + sum_j w[t, j] * FFN_{idx[t, j]}(h[t]).

    Shared expert ungated (weight one) on every token; routed experts weighted
    by the renormalised router weights (wireai.ir, "Four key changes behind
    the jump", bullet 3: shared expert beside the routed experts).  This is
    the shard's partial sum: the cross-GPU reduction that follows it on a
    multi-GPU group is not part of one shard's step, and it is not added to
    the residual.  `expert(e)` returns (W1, W3, W2) bit patterns of expert e.
    """
    h = f64(h)
    B, H = h.shape
    y = np.zeros((B, H))
    if np.asarray(s1_bits).shape[0] > 0:
        y += swiglu_ffn(h, s1_bits, s3_bits, s2_bits)
    idx = np.asarray(idx)
    for e in np.unique(idx):
        rows, cols = np.nonzero(idx == e)
        w1, w3, w2 = expert(int(e))
        y[rows] += np.asarray(w)[rows, cols][:, None] * swiglu_ffn(h[rows], w1, w3, w2)
    return y


# --- the whole step ---------------------------------------------------------
def decode_step(x_bits, attn_bits, resid, w_qkv_bits, w_o_bits, gain_bits, w_router,
                expert, s1_bits, s3_bits, s2_bits, top_k: int, eps: float = RMS_EPS):
    """One decode layer-step on one shard.  Returns a dict of float64/int64 arrays:
    qkv, resid_out (r1), h, ms, logits, topk_idx, topk_w, moe_out (y)."""
    qkv = attention_input_projection(x_bits, w_qkv_bits)
    r1 = out_projection_residual(attn_bits, w_o_bits, resid)
    h, ms = rms_norm(r1, gain_bits, eps)
    logits = router_logits(h, w_router)
    idx, w = select_experts(logits, top_k)
    y = moe_output(h, idx, w, expert, s1_bits, s3_bits, s2_bits)
    return {"qkv": qkv, "resid_out": r1, "h": h, "ms": ms, "logits": logits,
            "topk_idx": idx, "topk_w": w, "moe_out": y}
