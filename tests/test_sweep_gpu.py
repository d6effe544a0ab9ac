"""GPU parity over seeded random shapes across the configuration envelope.

Each case draws one shape (tests/sweep_shapes.py), runs it on every path
that takes it - the automatic choice (single launch when the batch fits),
the five-launch VALU path, and the matrix-core batched path when the shape
meets its tilings - and compares every output with the fp64 oracle.  A second
set draws its shapes inside the single-launch kernel's envelope, so that the
automatic choice takes that kernel.  Shape-specific indexing mistakes (a
ragged row tile, an expert count that is not a multiple of a wave, an odd qkv
width) fail here rather than at a workload.
"""
import dataclasses

import pytest
import torch

from synth import device as sdev, gen, routing
from synth.gen import LayerShape
from tests import sweep_shapes, workload
from tests.parity import say
from tests.test_parity_gpu import AUTO, BATCHED, MULTI, PATH_NAMES, check, run_gpu

pytestmark = pytest.mark.gpu

N_SHAPES = 32
N_SINGLE_SHAPES = 16


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_moe_amd  # noqa: F401  (raises if the library was not built)


def build(s, seed: int) -> routing.RoutedLayer:
    raw = gen.draw_shape(s, seed=seed)
    h = workload.oracle_h(raw)
    try:
        return routing.shape_router(raw, h)
    except ValueError:   # skewed loads not realisable at this E: route naturally
        raw.shape = dataclasses.replace(s, name=s.name + "_natural", routing="natural")
        return routing.shape_router(raw, h)


def path_taken(obj, s, path: int) -> str:
    """The path a step of batch s.batch takes on a layer made with `path`."""
    if path == MULTI:
        return "multi"
    if path == BATCHED:
        return "batched"
    if s.batch <= obj.single_max_batch:
        return "single"
    return "batched" if sweep_shapes.batched_tiling(s.hidden, s.attn_dim) else "multi"


def run_every_path(layer, tag: str) -> set:
    """Runs the layer on every path that takes its shape; returns their names."""
    from decode_step_moe_amd import DecodeLayer
    s = layer.shape
    say(f"[{tag}: {s.name}] start")
    w = sdev.upload_weights(layer)
    paths = [AUTO, MULTI] + ([BATCHED] if sweep_shapes.batched_tiling(s.hidden, s.attn_dim) else [])
    ran = set()
    for path in paths:
        obj = DecodeLayer(sdev.config_of(layer, path=path), w)
        name = path_taken(obj, s, path)
        if name in ran:
            continue
        ran.add(name)
        say(f"[{tag}: {s.name}] path={PATH_NAMES[path]} runs {name}")
        got, _ = run_gpu(layer, layer_obj=obj, path=path)
        check(layer, got, f"{tag}_{name}")
    del w
    torch.cuda.empty_cache()
    return ran


@pytest.mark.parametrize("i", range(N_SHAPES))
def test_random_shape_parity(i):
    run_every_path(build(sweep_shapes.random_shape(i), 1000 + i), f"sweep{i}")


@pytest.mark.parametrize("shape", [
    # 64 picks of 384 experts (one token fits the single launch: B k <= 64)
    LayerShape("k64_E384_b1", 1024, 1, 512, 512, 384, 64, 128, 128, "natural"),
    LayerShape("k64_E384_b5", 1024, 5, 512, 512, 384, 64, 128, 128, "zipf"),
    LayerShape("k48_E384_b3", 1024, 3, 512, 512, 384, 48, 128, 128, "natural"),
    # every expert picked by every token: 4 matrix-core chunks per expert
    LayerShape("k64_E64_b64", 1024, 64, 512, 512, 64, 64, 128, 128, "natural"),
    LayerShape("k64_E64_b17", 1024, 17, 512, 512, 64, 64, 64, 0, "natural"),
], ids=lambda s: s.name)
def test_top_k_up_to_64(shape):
    """top_k up to its limit of min(E, 64), on every path that takes the shape."""
    ran = run_every_path(build(shape, 77), shape.name)
    assert "multi" in ran


@pytest.mark.parametrize("i", range(N_SINGLE_SHAPES))
def test_random_single_launch_shape_parity(i):
    """Shapes inside the single-launch kernel's envelope: the automatic choice
    must take it, and it must agree with the oracle like the other paths."""
    ran = run_every_path(build(sweep_shapes.random_single_shape(i), 2000 + i), f"single{i}")
    assert "single" in ran
