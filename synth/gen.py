"""Seeded random draws for one MoE decode layer-step.

Shapes follow the five workloads this library is measured on (a tiny
correctness layer, a TP16 shard at batch 1 and 8, a TP8 shard at batch 64 and
an 8-token speculative-verify step).  Distributions: bf16 weights ~N(0,0.02),
RMSNorm gain ~N(1,0.1), fp32 router noise ~N(0,0.02), bf16 activations and the
fp32 residual ~N(0,1).

Every tensor comes from its own PCG64 stream keyed by
SeedSequence([seed, stream, sub]); streams: 0 dense weights (sub = matrix id),
1 routed expert e (sub = e), 2 router noise, 3 activations, 4 routing targets.
Because each expert has its own stream, any expert can be drawn alone, so a
test never has to materialise the whole pool (2.1-4.2 GB) on the host.

bf16 values are carried as their uint16 bit patterns (no ml_dtypes here).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class LayerShape:
    name: str
    hidden: int       # H
    batch: int        # B tokens in the step
    qkv_out: int      # Dq, rows of the attention input projection
    attn_dim: int     # Do, width of the attention output fed to the out-projection
    n_experts: int    # E
    top_k: int        # k
    expert_ffn: int   # F, routed expert ffn width on this shard
    shared_ffn: int   # Fs, shared expert ffn width on this shard
    routing: str      # "natural" | "hot" | "zipf" | "skewed"


SHAPES = {
    0: LayerShape("tiny_b1", 512, 1, 768, 768, 8, 2, 256, 256, "natural"),
    1: LayerShape("tp16_shard_b1", 7168, 1, 512, 512, 384, 8, 128, 128, "natural"),
    2: LayerShape("tp16_shard_b8", 7168, 8, 512, 512, 384, 8, 128, 128, "natural"),
    3: LayerShape("tp8_shard_b64_hot", 7168, 64, 1024, 1024, 384, 8, 256, 256, "hot"),
    4: LayerShape("tp16_shard_spec_verify_1x8_zipf", 7168, 8, 512, 512, 384, 8,
                  128, 128, "zipf"),
}

# stream ids
S_DENSE, S_EXPERT, S_ROUTER, S_ACT, S_ROUTE = 0, 1, 2, 3, 4
# dense matrix ids inside stream 0
M_QKV, M_O, M_GAIN, M_S1, M_S3, M_S2 = 0, 1, 2, 3, 4, 5


def rng(seed: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, sub])))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(g: np.random.Generator, shape, mean: float, std: float) -> np.ndarray:
    return f32_to_bf16_bits(g.normal(mean, std, size=shape).astype(np.float32))


@dataclass
class RawLayer:
    """All draws of one layer-step except the router matrix (shaped later)."""
    shape: LayerShape
    seed: int
    x: np.ndarray          # bf16 bits [B][H]
    attn: np.ndarray       # bf16 bits [B][Do]
    resid: np.ndarray      # fp32 [B][H]
    w_qkv: np.ndarray      # bf16 bits [Dq][H]
    w_o: np.ndarray        # bf16 bits [H][Do]
    gain: np.ndarray       # bf16 bits [H]
    router_noise: np.ndarray  # fp32 [E][H]
    s1: np.ndarray         # bf16 bits [Fs][H]
    s3: np.ndarray         # bf16 bits [Fs][H]
    s2: np.ndarray         # bf16 bits [H][Fs]
    _expert_cache: dict = field(default_factory=dict, repr=False)

    def expert(self, e: int):
        """(w1 [F][H], w3 [F][H], w2 [H][F]) bf16 bits of routed expert e."""
        if e not in self._expert_cache:
            s = self.shape
            g = rng(self.seed, S_EXPERT, e)
            w1 = _normal_bf16(g, (s.expert_ffn, s.hidden), 0.0, 0.02)
            w3 = _normal_bf16(g, (s.expert_ffn, s.hidden), 0.0, 0.02)
            w2 = _normal_bf16(g, (s.hidden, s.expert_ffn), 0.0, 0.02)
            self._expert_cache[e] = (w1, w3, w2)
        return self._expert_cache[e]

    def drop_expert_cache(self):
        self._expert_cache.clear()


def draw(cfg: int, seed: int | None = None, batch: int | None = None,
         top_k: int | None = None, shared_ffn: int | None = None,
         routing: str | None = None) -> RawLayer:
    """Draw every tensor of workload `cfg` (default seed = cfg).

    `batch`, `top_k`, `shared_ffn` and `routing` override the workload's
    values (edge-case tests); activations for a smaller batch are the leading
    rows of the full draw, and every other tensor is drawn exactly as for the
    workload.
    """
    s = SHAPES[cfg]
    if batch is not None or top_k is not None or shared_ffn is not None or routing is not None:
        b = s.batch if batch is None else batch
        k = s.top_k if top_k is None else top_k
        fs = s.shared_ffn if shared_ffn is None else shared_ffn
        rt = s.routing if routing is None else routing
        s = LayerShape(s.name + f"_b{b}_k{k}_fs{fs}_{rt}", s.hidden, b, s.qkv_out, s.attn_dim,
                       s.n_experts, k, s.expert_ffn, fs, rt)
    return draw_shape(s, cfg if seed is None else seed)


def draw_shape(s: LayerShape, seed: int) -> RawLayer:
    """Draw every tensor of a layer of shape `s` from `seed` (any shape in the
    library's envelope, e.g. the seeded random shapes of the sweep tests)."""
    H, B = s.hidden, s.batch
    ga = rng(seed, S_ACT)
    # 64 rows are always drawn, so a smaller batch is a prefix of a larger one
    nb = max(B, 64)
    x = _normal_bf16(ga, (nb, H), 0.0, 1.0)[:B]
    attn = _normal_bf16(ga, (nb, s.attn_dim), 0.0, 1.0)[:B]
    resid = ga.normal(0.0, 1.0, size=(nb, H)).astype(np.float32)[:B]
    w_qkv = _normal_bf16(rng(seed, S_DENSE, M_QKV), (s.qkv_out, H), 0.0, 0.02)
    w_o = _normal_bf16(rng(seed, S_DENSE, M_O), (H, s.attn_dim), 0.0, 0.02)
    gain = _normal_bf16(rng(seed, S_DENSE, M_GAIN), (H,), 1.0, 0.1)
    router_noise = rng(seed, S_ROUTER).normal(0.0, 0.02, size=(s.n_experts, H)).astype(np.float32)
    if s.shared_ffn > 0:
        s1 = _normal_bf16(rng(seed, S_DENSE, M_S1), (s.shared_ffn, H), 0.0, 0.02)
        s3 = _normal_bf16(rng(seed, S_DENSE, M_S3), (s.shared_ffn, H), 0.0, 0.02)
        s2 = _normal_bf16(rng(seed, S_DENSE, M_S2), (H, s.shared_ffn), 0.0, 0.02)
    else:
        s1 = np.zeros((0, H), np.uint16)
        s3 = np.zeros((0, H), np.uint16)
        s2 = np.zeros((H, 0), np.uint16)
    return RawLayer(s, seed, np.ascontiguousarray(x), np.ascontiguousarray(attn),
                    np.ascontiguousarray(resid), w_qkv, w_o, gain, router_noise, s1, s3, s2)
