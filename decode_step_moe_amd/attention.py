"""Thin ctypes binding of the decode attention core (include/decode_attention.h).

Argument marshalling only: dtype / shape / device / contiguity checks on the
torch tensors, then their data pointers and the current HIP stream go to the
C ABI.  The attention runs in the library's HIP kernels; there is no Python
or CPU fallback.
"""
from __future__ import annotations

import ctypes

from .binding import DL_OK, DecodeLayerError, _ptr, last_error, lib


class AttnConfig(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("max_requests", ctypes.c_int32), ("cache_len", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("max_splits", ctypes.c_int32)]


class AttnIO(ctypes.Structure):
    _fields_ = [("n_requests", ctypes.c_int32), ("n_tokens", ctypes.c_int32), ("max_past", ctypes.c_int32)] + \
               [(n, ctypes.c_void_p) for n in ("past_len", "q", "k_new", "v_new", "k_cache", "v_cache",
                                               "k_scale", "v_scale", "out", "workspace", "out_bf16")]


_done = False


def _lib():
    global _done
    L = lib()
    if not _done:
        L.decode_attention_workspace_bytes.argtypes = [ctypes.POINTER(AttnConfig)]
        L.decode_attention_workspace_bytes.restype = ctypes.c_size_t
        L.decode_attention_check.argtypes = [ctypes.POINTER(AttnConfig), ctypes.POINTER(AttnIO)]
        L.decode_attention_check.restype = ctypes.c_int
        L.decode_attention_step.argtypes = [ctypes.POINTER(AttnConfig), ctypes.POINTER(AttnIO), ctypes.c_void_p]
        L.decode_attention_step.restype = ctypes.c_int
        _done = True
    return L


def make_attn_config(n_q_heads, n_kv_heads, max_tokens, max_requests, cache_len, softmax_scale,
                     head_dim=128, max_splits=0) -> AttnConfig:
    return AttnConfig(n_q_heads, n_kv_heads, head_dim, max_tokens, max_requests, cache_len, softmax_scale,
                      max_splits)


def workspace_bytes(cfg: AttnConfig) -> int:
    return _lib().decode_attention_workspace_bytes(ctypes.byref(cfg))


def check(cfg: AttnConfig, io: AttnIO) -> int:
    return _lib().decode_attention_check(ctypes.byref(cfg), ctypes.byref(io))


def make_io(cfg: AttnConfig, past_len, max_past, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, out,
            workspace, out_bf16=None) -> AttnIO:
    """out_bf16 (optional): bf16 [R][T][Hq][D], the output rounded to bf16 in
    the decode layer step's attn layout [R*T][Hq*D]."""
    import torch
    R, T = q.shape[0], q.shape[1]
    Hq, Hkv, D, C = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.cache_len
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    return AttnIO(R, T, max_past, _ptr(past_len, torch.int32, (R,), "past_len"),
                  _ptr(q, bf, (R, T, Hq, D), "q"), _ptr(k_new, bf, (R, T, Hkv, D), "k_new"),
                  _ptr(v_new, bf, (R, T, Hkv, D), "v_new"),
                  _ptr(k_cache, u8, (cfg.max_requests, Hkv, C, D), "k_cache"),
                  _ptr(v_cache, u8, (cfg.max_requests, Hkv, C, D), "v_cache"),
                  _ptr(k_scale, f32, (Hkv,), "k_scale"), _ptr(v_scale, f32, (Hkv,), "v_scale"),
                  _ptr(out, f32, (R, T, Hq, D), "out"),
                  _ptr(workspace, u8, (workspace_bytes(cfg),), "workspace"),
                  None if out_bf16 is None else _ptr(out_bf16, bf, (R, T, Hq, D), "out_bf16"))


def step_io(cfg: AttnConfig, io: AttnIO, stream=None):
    """Enqueue one attention step (decode_attention_step) on `stream` (default: current)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = _lib().decode_attention_step(ctypes.byref(cfg), ctypes.byref(io), ctypes.c_void_p(stream.cuda_stream))
    if rc != DL_OK:
        raise DecodeLayerError(rc, last_error())
