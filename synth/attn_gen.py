"""Seeded random draws for one decode-attention step (no step arithmetic).

Shapes: R requests, T query tokens per request (1 verified token plus T - 1
drafts), Hq query heads and Hkv KV heads of head size D on one shard, a
cache of C positions per request and KV head.  Distributions: query, new
keys and new values bf16 ~N(0, 1); the cache's earlier positions hold random
FP8 E4M3 codes with the exponent field in [9, 14] and random sign and
mantissa (magnitudes 4 .. 240, about N(0, 1) * 64 in scale), unused
positions hold random bytes; the per-KV-head scales are 1/64 times a factor
in [0.75, 1.25]; the past lengths are drawn in [min_past, max_past].
Streams: SeedSequence([seed, 10, sub]) with sub 0 activations, 1 cache,
2 lengths and scales.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import f32_to_bf16_bits, rng


@dataclass
class AttnStep:
    q: np.ndarray          # bf16 bits [R][T][Hq][D]
    k_new: np.ndarray      # bf16 bits [R][T][Hkv][D]
    v_new: np.ndarray      # bf16 bits [R][T][Hkv][D]
    k_cache: np.ndarray    # uint8 [R][Hkv][C][D]
    v_cache: np.ndarray    # uint8 [R][Hkv][C][D]
    past_len: np.ndarray   # int32 [R]
    k_scale: np.ndarray    # fp32 [Hkv]
    v_scale: np.ndarray    # fp32 [Hkv]
    softmax_scale: float

    @property
    def shape(self):
        R, T, Hq, D = self.q.shape
        return R, T, Hq, self.k_cache.shape[1], D, self.k_cache.shape[2]


def _codes(g, shape):
    e = g.integers(9, 15, size=shape, dtype=np.int64)
    m = g.integers(0, 8, size=shape, dtype=np.int64)
    s = g.integers(0, 2, size=shape, dtype=np.int64)
    return ((s << 7) | (e << 3) | m).astype(np.uint8)


def draw(R: int, T: int, Hq: int, Hkv: int, C: int, min_past: int, max_past: int, seed: int = 0,
         D: int = 128, past=None) -> AttnStep:
    """`past` (length R) replaces the drawn past lengths when given."""
    if max_past + T > C:
        raise ValueError("the cache cannot hold the step's tokens")
    ga, gc, gl = rng(seed, 10, 0), rng(seed, 10, 1), rng(seed, 10, 2)
    q = f32_to_bf16_bits(ga.normal(0, 1, size=(R, T, Hq, D)).astype(np.float32))
    k_new = f32_to_bf16_bits(ga.normal(0, 1, size=(R, T, Hkv, D)).astype(np.float32))
    v_new = f32_to_bf16_bits(ga.normal(0, 1, size=(R, T, Hkv, D)).astype(np.float32))
    drawn = gl.integers(min_past, max_past + 1, size=R).astype(np.int32)
    if past is None:
        past = drawn
    else:
        past = np.asarray(past, dtype=np.int32).reshape(R)
        if past.min(initial=0) < 0 or past.max(initial=0) + T > C:
            raise ValueError("past lengths outside the cache")
    k_cache = gc.integers(0, 256, size=(R, Hkv, C, D), dtype=np.int64).astype(np.uint8)
    v_cache = gc.integers(0, 256, size=(R, Hkv, C, D), dtype=np.int64).astype(np.uint8)
    for r in range(R):
        n = int(past[r])
        k_cache[r, :, :n] = _codes(gc, (Hkv, n, D))
        v_cache[r, :, :n] = _codes(gc, (Hkv, n, D))
    k_scale = (gl.uniform(0.75, 1.25, size=Hkv) / 64.0).astype(np.float32)
    v_scale = (gl.uniform(0.75, 1.25, size=Hkv) / 64.0).astype(np.float32)
    return AttnStep(q, k_new, v_new, k_cache, v_cache, past, k_scale, v_scale, float(np.float32(D ** -0.5)))


# Named attention workloads on one TP16 shard (4 query heads sharing 1 KV head
# of 128): (R requests, T tokens each, Hq, Hkv, cache_len C, min_past, max_past).
WORKLOADS = {
    # small: several chunks and a ragged tail, the oracle finishes in seconds
    "attn_small": (4, 8, 4, 1, 1024, 200, 1000),
    # speculative verify: 1 request, 1 verified token + 7 drafts, long context
    "attn_verify_ctx8k": (1, 8, 4, 1, 8192, 8184, 8184),
    # batch-64 decode: one token per request, contexts mixed over 1k .. 4k
    "attn_b64_ctx4k": (64, 1, 4, 1, 4096, 1024, 4095),
}


def draw_workload(name: str, seed: int = 0) -> AttnStep:
    R, T, Hq, Hkv, C, lo, hi = WORKLOADS[name]
    return draw(R, T, Hq, Hkv, C, lo, hi, seed=seed)
