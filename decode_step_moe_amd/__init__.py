"""MI355X-native decode step of a mixture-of-experts transformer layer.

The compute lives in libdecode_layer.so (hand-written HIP for gfx950, C ABI
in include/decode_layer.h); `binding` is its thin ctypes binding.
"""
from .binding import (DecodeLayer, DecodeLayerError, Config, IO, Weights, StepOutputs,
                      make_config, check_config, check_io, scratch_bytes, last_error, lib,
                      DL_OK, DL_ERR_INVALID_ARG, DL_ERR_UNSUPPORTED, DL_ERR_HIP, DL_ERR_OOM,
                      DL_PATH_AUTO, DL_PATH_MULTI, DL_PATH_SINGLE, DL_PATH_BATCHED)

__all__ = ["DecodeLayer", "DecodeLayerError", "Config", "IO", "Weights", "StepOutputs",
           "make_config", "check_config", "check_io", "scratch_bytes", "last_error", "lib",
           "DL_OK", "DL_ERR_INVALID_ARG", "DL_ERR_UNSUPPORTED", "DL_ERR_HIP", "DL_ERR_OOM",
           "DL_PATH_AUTO", "DL_PATH_MULTI", "DL_PATH_SINGLE", "DL_PATH_BATCHED"]
