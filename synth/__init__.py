"""Seeded synthetic inputs for the MoE decode layer-step.

This package draws random numbers and lays them out; it computes no step of
the layer.  Both the CPU oracle's tests and the GPU path's tests/bench take
their inputs from here, so it deliberately holds none of the layer's
arithmetic (no projection, norm, router score, top-k or expert FFN).
"""
from .gen import (SHAPES, LayerShape, RawLayer, draw, f32_to_bf16_bits,
                  bf16_bits_to_f32)
from .routing import RoutedLayer, shape_router, stored_h, STORED_H_SEEDS

__all__ = ["SHAPES", "LayerShape", "RawLayer", "draw", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "RoutedLayer", "shape_router", "stored_h",
           "STORED_H_SEEDS"]
