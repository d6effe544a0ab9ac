"""Thin ctypes binding of libdecode_layer.so (include/decode_layer.h).

Argument marshalling only: dtype / shape / device / contiguity checks on the
torch tensors, then their data pointers and the current HIP stream go to the
C ABI.  Every step of the layer runs in the library's HIP kernels; there is
no Python or CPU fallback - if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdecode_layer.so")

DL_OK, DL_ERR_INVALID_ARG, DL_ERR_UNSUPPORTED, DL_ERR_HIP, DL_ERR_OOM = 0, -1, -2, -3, -4
DL_PATH_AUTO, DL_PATH_MULTI, DL_PATH_SINGLE, DL_PATH_BATCHED = 0, 1, 2, 3
_ERR_NAMES = {0: "DL_OK", -1: "DL_ERR_INVALID_ARG", -2: "DL_ERR_UNSUPPORTED", -3: "DL_ERR_HIP",
              -4: "DL_ERR_OOM"}


class DecodeLayerError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("qkv_out", ctypes.c_int32),
                ("attn_dim", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_ffn", ctypes.c_int32),
                ("shared_ffn", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("score_fn", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("path", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_qkv", "w_o", "norm_gain", "w_router", "w1", "w3", "w2", "s1", "s3", "s2")]


class IO(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32)] + [(n, ctypes.c_void_p) for n in
                ("x", "attn", "resid_in", "qkv", "resid_out", "router_logits", "topk_idx",
                 "topk_w", "moe_out", "h_out")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m decode_step_moe_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.decode_layer_init.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights),
                                        ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]
        L.decode_layer_init.restype = ctypes.c_int
        L.decode_layer_step.argtypes = [ctypes.c_void_p, ctypes.POINTER(IO), ctypes.c_void_p]
        L.decode_layer_step.restype = ctypes.c_int
        L.decode_layer_destroy.argtypes = [ctypes.c_void_p]
        L.decode_layer_destroy.restype = ctypes.c_int
        L.decode_layer_check_config.argtypes = [ctypes.POINTER(Config)]
        L.decode_layer_check_config.restype = ctypes.c_int
        L.decode_layer_check_io.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(IO)]
        L.decode_layer_check_io.restype = ctypes.c_int
        L.decode_layer_last_error.argtypes = [ctypes.c_void_p]
        L.decode_layer_last_error.restype = ctypes.c_char_p
        L.decode_layer_set_profiling.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.decode_layer_set_profiling.restype = ctypes.c_int
        L.decode_layer_kernel_times.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_int]
        L.decode_layer_kernel_times.restype = ctypes.c_int
        L.decode_layer_scratch_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int]
        L.decode_layer_scratch_bytes.restype = ctypes.c_size_t
        L.decode_layer_single_max_batch.argtypes = [ctypes.c_void_p]
        L.decode_layer_single_max_batch.restype = ctypes.c_int
        L.decode_layer_status.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32),
                                          ctypes.c_int]
        L.decode_layer_status.restype = ctypes.c_int
        L.decode_layer_set_trace.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.decode_layer_set_trace.restype = ctypes.c_int
        L.decode_layer_trace_points.argtypes = []
        L.decode_layer_trace_points.restype = ctypes.c_int
        L.decode_layer_grid.argtypes = [ctypes.c_void_p]
        L.decode_layer_grid.restype = ctypes.c_int
        L.decode_layer_set_prefetch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.decode_layer_set_prefetch.restype = ctypes.c_int
        L.decode_layer_set_spin_limit.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.decode_layer_set_spin_limit.restype = ctypes.c_int
        L.decode_layer_set_step_counter.argtypes = [ctypes.c_void_p, ctypes.c_uint32]
        L.decode_layer_set_step_counter.restype = ctypes.c_int
        # -- no-alloc entry point: begin
        L.decode_layer_step_noalloc.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights),
                                                ctypes.POINTER(IO), ctypes.c_void_p]
        L.decode_layer_step_noalloc.restype = ctypes.c_int
        L.decode_layer_noalloc_max_scratch.argtypes = []
        L.decode_layer_noalloc_max_scratch.restype = ctypes.c_size_t
        # -- no-alloc entry point: end
        _lib = L
    return _lib


def last_error(handle=None) -> str:
    return lib().decode_layer_last_error(handle).decode()


def make_config(hidden, qkv_out, attn_dim, n_experts, top_k, expert_ffn, shared_ffn, max_batch,
                rms_eps=1e-6, score_fn=0, renormalize=1, path=DL_PATH_AUTO) -> Config:
    return Config(hidden, qkv_out, attn_dim, n_experts, top_k, expert_ffn, shared_ffn, max_batch,
                  rms_eps, score_fn, renormalize, path)


def check_config(cfg: Config) -> int:
    return lib().decode_layer_check_config(ctypes.byref(cfg))


def check_io(cfg: Config, io: IO) -> int:
    return lib().decode_layer_check_io(ctypes.byref(cfg), ctypes.byref(io))


def scratch_bytes(cfg: Config, n_cu: int = 0) -> int:
    return lib().decode_layer_scratch_bytes(ctypes.byref(cfg), n_cu)


def _ptr(t, dtype, shape, name):
    import torch
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    return t.data_ptr() if t.numel() else None


def make_weights(cfg: Config, weights: dict) -> Weights:
    """The C weights block for `cfg` from a dict of GPU tensors: w_qkv, w_o,
    norm_gain, w_router, w1, w3, w2, s1, s3, s2 (bf16 except w_router fp32;
    s1/s3/s2 absent iff shared_ffn 0).  Checks dtype, shape, contiguity and
    device; the tensors are referenced, not copied."""
    import torch
    H, Dq, Do, E, F, Fs = (cfg.hidden, cfg.qkv_out, cfg.attn_dim, cfg.n_experts,
                           cfg.expert_ffn, cfg.shared_ffn)
    bf = torch.bfloat16
    return Weights(
        _ptr(weights["w_qkv"], bf, (Dq, H), "w_qkv"), _ptr(weights["w_o"], bf, (H, Do), "w_o"),
        _ptr(weights["norm_gain"], bf, (H,), "norm_gain"),
        _ptr(weights["w_router"], torch.float32, (E, H), "w_router"),
        _ptr(weights["w1"], bf, (E, F, H), "w1"), _ptr(weights["w3"], bf, (E, F, H), "w3"),
        _ptr(weights["w2"], bf, (E, H, F), "w2"),
        _ptr(weights.get("s1"), bf, (Fs, H), "s1") if Fs else None,
        _ptr(weights.get("s3"), bf, (Fs, H), "s3") if Fs else None,
        _ptr(weights.get("s2"), bf, (H, Fs), "s2") if Fs else None)


def make_io(cfg: Config, x, attn, resid_in, out) -> IO:
    """The C per-step block from GPU tensors (see DecodeLayer.make_io)."""
    import torch
    B = x.shape[0]
    bf, f32 = torch.bfloat16, torch.float32
    return IO(B, _ptr(x, bf, (B, cfg.hidden), "x"), _ptr(attn, bf, (B, cfg.attn_dim), "attn"),
              _ptr(resid_in, f32, (B, cfg.hidden), "resid_in"),
              _ptr(out.qkv, f32, (B, cfg.qkv_out), "qkv"),
              _ptr(out.resid_out, f32, (B, cfg.hidden), "resid_out"),
              _ptr(out.router_logits, f32, (B, cfg.n_experts), "router_logits"),
              _ptr(out.topk_idx, torch.int32, (B, cfg.top_k), "topk_idx"),
              _ptr(out.topk_w, f32, (B, cfg.top_k), "topk_w"),
              _ptr(out.moe_out, f32, (B, cfg.hidden), "moe_out"),
              _ptr(out.h_out, f32, (B, cfg.hidden), "h_out"))


def alloc_outputs(cfg: Config, batch: int, device="cuda", with_h: bool = False,
                  with_logits: bool = True):
    import torch
    f32 = torch.float32
    return StepOutputs(
        torch.empty(batch, cfg.qkv_out, dtype=f32, device=device),
        torch.empty(batch, cfg.hidden, dtype=f32, device=device),
        torch.empty(batch, cfg.n_experts, dtype=f32, device=device) if with_logits else None,
        torch.empty(batch, cfg.top_k, dtype=torch.int32, device=device),
        torch.empty(batch, cfg.top_k, dtype=f32, device=device),
        torch.empty(batch, cfg.hidden, dtype=f32, device=device),
        torch.empty(batch, cfg.hidden, dtype=f32, device=device) if with_h else None)


# -- no-alloc entry point: begin
def noalloc_max_scratch() -> int:
    """Bytes of the static scratch area decode_layer_step_noalloc uses per device."""
    return lib().decode_layer_noalloc_max_scratch()


def step_noalloc(cfg: Config, weights: Weights, io: IO, stream=None):
    """decode_layer_step_noalloc: one step with no handle and no device
    allocation, on the current device (scratch in the library's static area)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = lib().decode_layer_step_noalloc(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(io),
                                         ctypes.c_void_p(stream.cuda_stream))
    if rc != DL_OK:
        raise DecodeLayerError(rc, last_error())
# -- no-alloc entry point: end


@dataclass
class StepOutputs:
    qkv: object
    resid_out: object
    router_logits: object
    topk_idx: object
    topk_w: object
    moe_out: object
    h_out: object = None


class DecodeLayer:
    """One layer shard's weights bound to a library handle.

    `weights` maps w_qkv, w_o, norm_gain, w_router, w1, w3, w2, s1, s3, s2 to
    GPU tensors (bf16 except w_router fp32; s1/s3/s2 absent iff shared_ffn 0).
    The tensors are referenced, not copied, and must stay unchanged.
    With debug=True every step synchronises its stream and raises if the
    device status word reports an expired hand-off wait.
    """

    def __init__(self, cfg: Config, weights: dict, device: int = 0, debug: bool = False):
        self.cfg = cfg
        self.debug = debug
        self._keep = dict(weights)
        w = make_weights(cfg, weights)
        self.weights_c = w
        h = ctypes.c_void_p()
        rc = lib().decode_layer_init(ctypes.byref(cfg), ctypes.byref(w), device, ctypes.byref(h))
        if rc != DL_OK:
            raise DecodeLayerError(rc, last_error())
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().decode_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    LAUNCH_NAMES = ("proj_out_in", "shared_gateup", "router_topk_permute", "expert_gateup",
                    "expert_down_combine", "single_launch_step",
                    "batched_proj", "batched_router", "batched_topk_permute", "batched_gateup",
                    "batched_down")

    @property
    def single_max_batch(self) -> int:
        """Largest batch the single-launch path takes with this handle (0: none)."""
        return lib().decode_layer_single_max_batch(self._h)

    def set_trace(self, buf):
        """Phase trace of the single-launch kernel into a uint64 GPU tensor of
        [grid][trace_points] (None: off)."""
        import torch
        ptr = None
        if buf is not None:
            n = lib().decode_layer_grid(self._h) * lib().decode_layer_trace_points()
            if buf.dtype != torch.int64 or buf.numel() < n or not buf.is_cuda or not buf.is_contiguous():
                raise ValueError(f"trace buffer: need a contiguous int64 GPU tensor of >= {n} values")
            ptr = buf.data_ptr()
        rc = lib().decode_layer_set_trace(self._h, ptr)
        if rc != DL_OK:
            raise DecodeLayerError(rc, last_error(self._h))

    @property
    def grid(self) -> int:
        return lib().decode_layer_grid(self._h)

    def status(self, clear: bool = False) -> int:
        """Device status word (synchronise first): bit 0 a single-launch hand-off
        wait expired since the last clear."""
        v = ctypes.c_uint32()
        rc = lib().decode_layer_status(self._h, ctypes.byref(v), int(clear))
        if rc != DL_OK:
            raise DecodeLayerError(rc, last_error(self._h))
        return int(v.value)

    def set_prefetch(self, next_layer: "DecodeLayer | None"):
        """Prefetch `next_layer`'s dense weights during this layer's steps (None: off)."""
        rc = lib().decode_layer_set_prefetch(self._h, next_layer._h if next_layer is not None else None)
        if rc != DL_OK:
            raise DecodeLayerError(rc, last_error(self._h))
        self._next = next_layer   # keeps the next handle alive while this one prefetches it

    def set_spin_limit(self, rounds: int):
        """Test support: polling rounds before a hand-off wait gives up."""
        rc = lib().decode_layer_set_spin_limit(self._h, int(rounds))
        if rc != DL_OK:
            raise DecodeLayerError(rc, last_error(self._h))

    def set_step_counter(self, last_tag: int):
        """Test support: the device step counter (tag of the last step)."""
        rc = lib().decode_layer_set_step_counter(self._h, int(last_tag))
        if rc != DL_OK:
            raise DecodeLayerError(rc, last_error(self._h))

    def set_profiling(self, enable: bool):
        rc = lib().decode_layer_set_profiling(self._h, int(enable))
        if rc != DL_OK:
            raise DecodeLayerError(rc, last_error(self._h))

    def kernel_times_ms(self) -> dict:
        """Per-launch durations (ms) of the last step run with profiling on."""
        buf = (ctypes.c_float * len(self.LAUNCH_NAMES))()
        n = lib().decode_layer_kernel_times(self._h, buf, len(buf))
        if n < 0:
            raise DecodeLayerError(n, last_error(self._h))
        return {name: float(buf[i]) for i, name in enumerate(self.LAUNCH_NAMES[:n]) if buf[i] > 0}

    def alloc_outputs(self, batch: int, device="cuda", with_h: bool = False,
                      with_logits: bool = True) -> StepOutputs:
        return alloc_outputs(self.cfg, batch, device, with_h, with_logits)

    def make_io(self, x, attn, resid_in, out: StepOutputs) -> IO:
        return make_io(self.cfg, x, attn, resid_in, out)

    def step_io(self, io: IO, stream=None):
        """Enqueue one step from a prepared IO block on `stream` (default: current)."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        rc = lib().decode_layer_step(self._h, ctypes.byref(io), ctypes.c_void_p(stream.cuda_stream))
        if rc != DL_OK:
            raise DecodeLayerError(rc, last_error(self._h))
        if self.debug:
            stream.synchronize()
            st = self.status(clear=True)
            if st:
                raise DecodeLayerError(DL_ERR_HIP, f"device status {st:#x}: a hand-off wait expired "
                                                   "(the step's dependent outputs are NaN)")

    def step(self, x, attn, resid_in, out: StepOutputs | None = None, stream=None,
             with_h: bool = False) -> StepOutputs:
        if out is None:
            out = self.alloc_outputs(x.shape[0], device=x.device, with_h=with_h)
        self.step_io(self.make_io(x, attn, resid_in, out), stream)
        return out
