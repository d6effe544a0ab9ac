"""Upload a shaped workload to the GPU as the tensors the library consumes.

Full expert pools ([E][F][H], [E][H][F]) are allocated at their real size so
that the touched experts sit at their real addresses; only the touched
experts are filled with their drawn weights.  The rest of the pool is filled
with a bf16 NaN pattern by default: a correct step never reads an expert it
did not select, so any such read shows up as a NaN in the output.
"""
from __future__ import annotations

import numpy as np

from .routing import RoutedLayer

BF16_NAN_BITS = 0x7FC0


def bf16_tensor(bits: np.ndarray, device):
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(device)


def f32_tensor(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def upload_weights(layer: RoutedLayer, device="cuda", fill_untouched: str = "nan") -> dict:
    """Weights dict for decode_step_moe_amd.DecodeLayer.

    fill_untouched: "nan" (poison), "none" (leave the memory uninitialised).
    """
    import torch
    raw = layer.raw
    s = raw.shape
    E, F, H = s.n_experts, s.expert_ffn, s.hidden
    w = {
        "w_qkv": bf16_tensor(raw.w_qkv, device),
        "w_o": bf16_tensor(raw.w_o, device),
        "norm_gain": bf16_tensor(raw.gain, device),
        "w_router": f32_tensor(layer.w_router, device),
    }
    pools = {}
    for name, shp in (("w1", (E, F, H)), ("w3", (E, F, H)), ("w2", (E, H, F))):
        t = torch.empty(shp, dtype=torch.bfloat16, device=device)
        if fill_untouched == "nan":
            t.view(torch.int16).fill_(BF16_NAN_BITS)
        pools[name] = t
    for e in layer.touched_experts():
        w1, w3, w2 = raw.expert(int(e))
        pools["w1"][e].copy_(bf16_tensor(w1, device))
        pools["w3"][e].copy_(bf16_tensor(w3, device))
        pools["w2"][e].copy_(bf16_tensor(w2, device))
    w.update(pools)
    if s.shared_ffn > 0:
        w["s1"] = bf16_tensor(raw.s1, device)
        w["s3"] = bf16_tensor(raw.s3, device)
        w["s2"] = bf16_tensor(raw.s2, device)
    return w


def upload_inputs(layer: RoutedLayer, device="cuda"):
    raw = layer.raw
    return (bf16_tensor(raw.x, device), bf16_tensor(raw.attn, device),
            f32_tensor(raw.resid, device))


def config_of(layer: RoutedLayer, max_batch: int | None = None, eps: float = 1e-6, path: int = 0):
    from decode_step_moe_amd import make_config
    s = layer.shape
    return make_config(s.hidden, s.qkv_out, s.attn_dim, s.n_experts, s.top_k, s.expert_ffn,
                       s.shared_ffn, max_batch if max_batch is not None else max(s.batch, 1), eps,
                       path=path)
