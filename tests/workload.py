"""Test-side assembly of a workload: seeded draws, router shaping with the
oracle's h, and the oracle's expected outputs.  Test infrastructure."""
from __future__ import annotations

import numpy as np

from oracle import decode_layer_ref as ref
from synth import gen, routing


def oracle_h(raw) -> np.ndarray:
    r1 = ref.out_projection_residual(raw.attn, raw.w_o, raw.resid)
    return ref.rms_norm(r1, raw.gain)[0]


def build(cfg: int, seed=None, batch=None, h_source: str = "oracle", top_k=None,
          shared_ffn=None) -> routing.RoutedLayer:
    raw = gen.draw(cfg, seed, batch, top_k=top_k, shared_ffn=shared_ffn)
    h = routing.stored_h(cfg) if h_source == "stored" else oracle_h(raw)
    return routing.shape_router(raw, h)


def expected(layer: routing.RoutedLayer, w_router=None) -> dict:
    raw = layer.raw
    wr = layer.w_router if w_router is None else w_router
    return ref.decode_step(raw.x, raw.attn, raw.resid, raw.w_qkv, raw.w_o, raw.gain, wr,
                           raw.expert, raw.s1, raw.s3, raw.s2, raw.shape.top_k)


def logit_gaps(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the smallest gap among the sorted top k+1 logits."""
    srt = -np.sort(-np.asarray(logits, np.float64), axis=1)[:, : k + 1]
    return np.min(srt[:, :-1] - srt[:, 1:], axis=1)
