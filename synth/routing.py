"""Router-matrix shaping: give each workload the expert routing it is meant to have.

The router's logits are l = h @ Wr.T, where h is the normalised hidden state
the layer-step produces.  Random router weights give "natural" routing (for
iid noise this is a uniformly random k-subset per token), but the top-k
indices are only comparable bit for bit between two implementations when the
k-th and (k+1)-th logits, and consecutive logits inside the top k, are
separated by a margin much larger than rounding noise.  This module therefore
picks an ordered target list T[t] of k experts per token and adds to the noise
matrix N the minimum-norm correction that moves the logits to target values L
with every gap >= DELTA:

    Wr.T = N.T + h.T (h h.T)^-1 (L - L0),   L0 = h @ N.T,

so that h @ Wr.T = L exactly in real arithmetic (B <= H makes h h.T invertible).

This is input construction, not a step of the layer: h is passed in (the
tests take it from the CPU oracle; the benchmark loads the copy stored under
synth/data/, which a committed script wrote with the oracle).

Targets per routing mode:
  natural - T[t] = the top k of L0 in order; L = L0 + DELTA*(k-j) on T[t][j].
  hot     - 32 hot experts; token t takes hot[(8*(t%4) + t//4 + j) % 32], j<8,
            which gives exactly 16 tokens to each hot expert at batch 64;
            the order inside T[t] is shuffled.
  zipf    - expert popularity proportional to rank^-1.1 over a random expert
            permutation; T[t] = k draws without replacement.
  skewed  - experts with the token counts SKEW_COUNTS (clipped to the batch),
            the rest of the B*k picks spread over other experts with 1 to 8
            tokens each; realised by giving each expert, largest count first,
            the tokens with the most free slots (ties at random), which fills
            every token's k slots exactly.  It puts routed experts on both
            sides of the 16-token matrix-core threshold and at every chunk
            shape a 64-token batch can produce (a partial second chunk, two
            full chunks, all tokens).
  For hot, zipf and skewed: L[t, T[t][j]] = max_e L0[t, e] + 0.5 + DELTA*(k-j).

shape_router(..., shift=s) adds s[t] to every logit of token t (sigmoid
saturation cases); the margins are unchanged.
"""
from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

from .gen import RawLayer, rng, S_ROUTE

DELTA = 2e-2
HOT_EXPERTS = 32
ZIPF_S = 1.1
SKEW_COUNTS = (64, 48, 33, 32, 31, 17, 16, 15, 9, 1)

_DATA = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data")
# workloads whose h is stored (default seed = workload index)
STORED_H_SEEDS = {0: 0, 1: 1, 2: 2, 3: 3, 4: 4}


def stored_h_path(cfg: int) -> str:
    return os.path.join(_DATA, f"h_cfg{cfg}_seed{STORED_H_SEEDS[cfg]}.npy")


def stored_h(cfg: int) -> np.ndarray:
    """fp32 [B][H] normalised hidden state of workload `cfg` at its default seed."""
    return np.load(stored_h_path(cfg), allow_pickle=False)


@dataclass
class RoutedLayer:
    raw: RawLayer
    w_router: np.ndarray   # fp32 [E][H]
    targets: np.ndarray    # int32 [B][k]: the intended top-k, in descending logit order
    target_logits: np.ndarray  # fp64 [B][E]

    @property
    def shape(self):
        return self.raw.shape

    def touched_experts(self) -> np.ndarray:
        return np.unique(self.targets.reshape(-1)).astype(np.int64)

    def expert_load(self) -> np.ndarray:
        return np.bincount(self.targets.reshape(-1), minlength=self.shape.n_experts)


def _hot_targets(B: int, E: int, k: int, g: np.random.Generator) -> np.ndarray:
    hot = g.choice(E, size=HOT_EXPERTS, replace=False)
    T = np.empty((B, k), np.int64)
    for t in range(B):
        start = 8 * (t % 4) + t // 4
        row = hot[[(start + j) % HOT_EXPERTS for j in range(k)]]
        T[t] = g.permutation(row)
    return T


def _zipf_targets(B: int, E: int, k: int, g: np.random.Generator) -> np.ndarray:
    perm = g.permutation(E)
    p_rank = (np.arange(1, E + 1, dtype=np.float64)) ** (-ZIPF_S)
    p = np.empty(E)
    p[perm] = p_rank / p_rank.sum()
    return np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(B)]) \
        if B > 0 else np.zeros((0, k), np.int64)


def _skewed_targets(B: int, E: int, k: int, g: np.random.Generator) -> np.ndarray:
    experts = g.permutation(E)
    counts = [min(c, B) for c in SKEW_COUNTS]
    while sum(counts) > B * k:
        counts.pop()
    load = list(zip(experts[:len(counts)].tolist(), counts))
    rest, i = B * k - sum(counts), len(counts)
    while rest > 0:
        c = int(min(rest, g.integers(1, 9), B))
        load.append((int(experts[i]), c))
        rest -= c
        i += 1
    if i > E:
        raise ValueError("not enough experts for the skewed loads")
    free = np.full(B, k)
    rows = [[] for _ in range(B)]
    for e, c in sorted(load, key=lambda ec: -ec[1]):
        order = np.lexsort((g.random(B), -free))   # most free slots first, ties at random
        for t in order[:c]:
            if free[t] == 0:
                raise ValueError("skewed loads not realisable")
            rows[t].append(e)
            free[t] -= 1
    assert np.all(free == 0)
    return np.stack([g.permutation(np.asarray(r, np.int64)) for r in rows])


def shape_router(raw: RawLayer, h: np.ndarray, shift=None) -> RoutedLayer:
    s = raw.shape
    B, E, k, H = s.batch, s.n_experts, s.top_k, s.hidden
    h = np.asarray(h, dtype=np.float64).reshape(B, H)
    N = raw.router_noise.astype(np.float64)
    if B == 0:
        return RoutedLayer(raw, raw.router_noise.copy(), np.zeros((0, k), np.int32),
                           np.zeros((0, E)))
    L0 = h @ N.T
    L = L0.copy()
    g = rng(raw.seed, S_ROUTE)
    bumps = DELTA * (k - np.arange(k))
    if s.routing == "natural":
        T = np.argsort(-L0, axis=1, kind="stable")[:, :k]
        for t in range(B):
            L[t, T[t]] += bumps
    else:
        make = {"hot": _hot_targets, "zipf": _zipf_targets, "skewed": _skewed_targets}[s.routing]
        T = make(B, E, k, g)
        for t in range(B):
            L[t, T[t]] = L0[t].max() + 0.5 + bumps
    if shift is not None:
        L += np.asarray(shift, np.float64).reshape(B, 1)
    M = np.linalg.lstsq(h @ h.T, L - L0, rcond=None)[0]      # [B][E]
    w_router = (N + M.T @ h).astype(np.float32)
    return RoutedLayer(raw, np.ascontiguousarray(w_router), T.astype(np.int32), L)
