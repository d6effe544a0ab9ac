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
         D: int = 128) -> AttnStep:
    if max_past + T > C:
        raise ValueError("the cache cannot hold the step's tokens")
    ga, gc, gl = rng(seed, 10, 0), rng(seed, 10, 1), rng(seed, 10, 2)
    q = f32_to_bf16_bits(ga.normal(0, 1, size=(R, T, Hq, D)).astype(np.float32))
    k_new = f32_to_bf16_bits(ga.normal(0, 1, size=(R, T, Hkv, D)).astype(np.float32))
    v_new = f32_to_bf16_bits(ga.normal(0, 1, size=(R, T, Hkv, D)).astype(np.float32))
    past = gl.integers(min_past, max_past + 1, size=R).astype(np.int32)
    k_cache = gc.integers(0, 256, size=(R, Hkv, C, D), dtype=np.int64).astype(np.uint8)
    v_cache = gc.integers(0, 256, size=(R, Hkv, C, D), dtype=np.int64).astype(np.uint8)
    for r in range(R):
        n = int(past[r])
        k_cache[r, :, :n] = _codes(gc, (Hkv, n, D))
        v_cache[r, :, :n] = _codes(gc, (Hkv, n, D))
    k_scale = (gl.uniform(0.75, 1.25, size=Hkv) / 64.0).astype(np.float32)
    v_scale = (gl.uniform(0.75, 1.25, size=Hkv) / 64.0).astype(np.float32)
    return AttnStep(q, k_new, v_new, k_cache, v_cache, past, k_scale, v_scale, float(np.float32(D ** -0.5)))
