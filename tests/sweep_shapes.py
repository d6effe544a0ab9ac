"""Seeded random layer shapes across the library's envelope, for the sweep
parity tests (test infrastructure).

Each shape draws every size of the layer: hidden and attention widths (three
fifths of them meeting the batched path's tilings, the rest only the general multiple of
8), any qkv width, expert counts from 1 to 1024 with their edge values
favoured, top-k up to min(E, 64) (mostly up to 8), every routed and shared
ffn width (shared expert on or off), batches 1-64 with single-launch batches favoured, and a
routing mode.  The expert weights the oracle has to draw are kept below a
budget so that one case costs the oracle about a second.
"""
from __future__ import annotations

import numpy as np

from synth.gen import LayerShape

SWEEP_SEED = 0x5EE9
EDGE_EXPERTS = (1, 2, 3, 8, 31, 32, 33, 63, 64, 65, 255, 256, 384, 1023, 1024)
FFNS = (32, 64, 128, 256)
# routed expert weights the oracle draws per case: touched experts * 3 * F * H
DRAW_BUDGET = 80_000_000


def batched_tiling(hidden: int, attn_dim: int) -> bool:
    """The batched path's shape requirement: K splits of 4 waves x 32 for the
    projections and gate/up, 256-wide router K chunks."""
    return hidden % 512 == 0 and attn_dim % 128 == 0


def random_shape(i: int) -> LayerShape:
    g = np.random.default_rng([SWEEP_SEED, i])
    if g.random() < 0.6:
        H = 512 * int(g.integers(1, 17))          # 512 .. 8192
        Do = 128 * int(g.integers(1, 17))         # 128 .. 2048
    else:
        H = 8 * int(g.integers(2, 1025))          # 16 .. 8192
        Do = 8 * int(g.integers(1, 257))          # 8 .. 2048
    Dq = int(g.integers(1, 2049))
    E = int(g.choice(EDGE_EXPERTS)) if g.random() < 0.4 else int(g.integers(1, 1025))
    k = int(g.integers(1, min(E, 64 if g.random() < 0.4 else 8) + 1))
    F = int(g.choice(FFNS))
    Fs = 0 if g.random() < 0.3 else int(g.choice(FFNS))
    B = int(g.integers(1, 9)) if g.random() < 0.5 else int(g.integers(9, 65))
    B = max(1, min(B, H // 2))                    # h h^T of the router shaping stays invertible
    while F > 32 and min(E, B * k) * 3 * F * H > DRAW_BUDGET:
        F //= 2
    while B > 1 and min(E, B * k) * 3 * F * H > DRAW_BUDGET:
        B = max(1, B // 2)
    # hot routing draws each token's picks from 32 hot experts
    modes = ["natural", "zipf"] + (["hot"] if E >= 32 and k <= 32 else []) + (["skewed"] if E >= 256 else [])
    rt = str(g.choice(modes))
    return LayerShape(f"sweep{i}_H{H}_Dq{Dq}_Do{Do}_E{E}_k{k}_F{F}_Fs{Fs}_B{B}_{rt}",
                      H, B, Dq, Do, E, k, F, Fs, rt)


def random_single_shape(i: int) -> LayerShape:
    """A random shape inside the single-launch kernel's envelope: hidden up to
    8192, qkv width up to 8 rows per workgroup, at most 512 experts, a shared
    ffn of 0 or the routed one, and a batch within its LDS limits (B*k <= 64,
    B*E and B*k*F <= 8192, at most 8 tokens)."""
    g = np.random.default_rng([SWEEP_SEED, 1, i])
    if g.random() < 0.5:
        H = 512 * int(g.integers(1, 17))
        Do = 128 * int(g.integers(1, 17))
    else:
        H = 8 * int(g.integers(2, 1025))
        Do = 8 * int(g.integers(1, 257))
    Dq = int(g.integers(1, 2049))
    E = int(g.choice([e for e in EDGE_EXPERTS if e <= 512])) if g.random() < 0.4 else int(g.integers(1, 513))
    k = int(g.integers(1, min(E, 64 if g.random() < 0.4 else 8) + 1))
    F = int(g.choice(FFNS))
    Fs = 0 if g.random() < 0.3 else F
    bmax = min(8, 64 // k, 8192 // E, 8192 // (k * F), H // 2)
    B = int(g.integers(1, bmax + 1)) if bmax >= 1 else 1
    while F > 32 and min(E, B * k) * 3 * F * H > DRAW_BUDGET:
        F //= 2
        Fs = min(Fs, F) if Fs else 0
    modes = ["natural", "zipf"] + (["hot"] if E >= 32 and k <= 32 else []) + (["skewed"] if E >= 256 else [])
    rt = str(g.choice(modes))
    return LayerShape(f"single{i}_H{H}_Dq{Dq}_Do{Do}_E{E}_k{k}_F{F}_Fs{Fs}_B{B}_{rt}",
                      H, B, Dq, Do, E, k, F, Fs, rt)


def single_envelope(s: LayerShape) -> bool:
    """The single-launch kernel's limits at 256 workgroups."""
    return (s.hidden <= 8192 and s.qkv_out <= 8 * 256 and s.n_experts <= 512
            and s.shared_ffn in (0, s.expert_ffn) and s.batch <= 8 and s.batch * s.top_k <= 64
            and s.batch * s.n_experts <= 8192 and s.batch * s.top_k * s.expert_ffn <= 8192)


def in_envelope(s: LayerShape) -> bool:
    """The library's configuration limits (decode_layer_init's checks)."""
    return (8 <= s.hidden <= 16384 and s.hidden % 8 == 0 and 1 <= s.qkv_out <= 65536
            and 8 <= s.attn_dim <= 16384 and s.attn_dim % 8 == 0 and 1 <= s.n_experts <= 1024
            and 1 <= s.top_k <= min(s.n_experts, 64) and s.expert_ffn in FFNS
            and s.shared_ffn in (0,) + FFNS and 1 <= s.batch <= 64)
