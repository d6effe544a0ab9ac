"""Parity gates between the GPU step and the CPU oracle (test infrastructure).

Gates (the accuracy targets of this layer-step):
  topk_idx             bit-exact (the generator keeps every top-k logit gap >= 1e-2)
  router logits        per token: max_e |l_gpu - l_ref| <= 1e-4 * max_e |l_ref|
  qkv, resid_out, y    max-abs <= 2e-2 and relative L2 <= 5e-3
  topk_w               per token: max_j |w_gpu - w_ref| <= 5e-5 * max_e |l_ref| + 1e-6
                       (|dw/dl| <= 1/2 for sigmoid scores renormalised over k
                       picks, applied to the logit gate)
  h (debug output)     relative L2 <= 1e-5 (fp32 arithmetic on every path)
"""
from __future__ import annotations

import sys

import numpy as np

LOGIT_RTOL = 1e-4
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
H_REL_L2 = 1e-5


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def max_abs(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def compare(gpu: dict, ref: dict) -> dict:
    """Returns the error metrics and a list of failed gates."""
    m = {}
    fails = []
    if not np.array_equal(np.asarray(gpu["topk_idx"], np.int64), np.asarray(ref["topk_idx"], np.int64)):
        bad = np.argwhere(np.asarray(gpu["topk_idx"]) != np.asarray(ref["topk_idx"]))
        fails.append(f"topk_idx differs at {bad[:5].tolist()}")
    lref = np.asarray(ref["logits"], np.float64)
    scale = np.max(np.abs(lref), axis=1) if lref.size else np.zeros(0)
    if gpu.get("logits") is not None and lref.size:
        err = np.max(np.abs(np.asarray(gpu["logits"], np.float64) - lref), axis=1)
        m["logits_rel"] = float(np.max(err / scale))
        if np.any(err > LOGIT_RTOL * scale):
            fails.append(f"logits rel err {m['logits_rel']:.3e} > {LOGIT_RTOL}")
    if lref.size:
        werr = np.max(np.abs(np.asarray(gpu["topk_w"], np.float64) - np.asarray(ref["topk_w"])), axis=1)
        m["topk_w_abs"] = float(np.max(werr))
        if np.any(werr > 5e-5 * scale + 1e-6):
            fails.append(f"topk_w err {m['topk_w_abs']:.3e}")
    for key in ("qkv", "resid_out", "moe_out"):
        ma, rl = max_abs(gpu[key], ref[key]), rel_l2(gpu[key], ref[key])
        m[key + "_max_abs"], m[key + "_rel_l2"] = ma, rl
        if not np.all(np.isfinite(np.asarray(gpu[key]))):
            fails.append(f"{key} has non-finite values")
        if ma > OUT_MAX_ABS or rl > OUT_REL_L2:
            fails.append(f"{key}: max-abs {ma:.3e}, rel-L2 {rl:.3e}")
    if gpu.get("h") is not None:
        m["h_rel_l2"] = rel_l2(gpu["h"], ref["h"])
        if m["h_rel_l2"] > H_REL_L2:
            fails.append(f"h rel-L2 {m['h_rel_l2']:.3e}")
    m["fails"] = fails
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
