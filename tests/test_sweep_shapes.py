"""The random shapes of the sweep parity tests stay inside the library's
envelope and reach its edges (CPU)."""
from synth import gen
from tests import sweep_shapes as ss
from tests.test_sweep_gpu import N_SHAPES, N_SINGLE_SHAPES


def test_sweep_shapes_in_envelope_and_varied():
    shapes = [ss.random_shape(i) for i in range(N_SHAPES)]
    assert all(ss.in_envelope(s) for s in shapes)
    assert len({s.name for s in shapes}) == N_SHAPES
    assert all(min(s.n_experts, s.batch * s.top_k) * 3 * s.expert_ffn * s.hidden <= ss.DRAW_BUDGET
               for s in shapes if s.batch > 1)
    tiled = [ss.batched_tiling(s.hidden, s.attn_dim) for s in shapes]
    assert any(tiled) and not all(tiled)
    assert any(s.batch == 1 for s in shapes) and any(s.batch > 16 for s in shapes)
    assert any(s.top_k == 1 for s in shapes) and any(s.top_k > 32 for s in shapes)
    assert any(s.shared_ffn == 0 for s in shapes) and any(s.shared_ffn == 256 for s in shapes)
    assert any(s.n_experts <= 3 for s in shapes) and any(s.n_experts > 900 for s in shapes)
    assert any(s.qkv_out % 8 for s in shapes) and any(s.hidden % 64 for s in shapes)
    assert {s.routing for s in shapes} >= {"natural", "zipf", "hot", "skewed"}


def test_draw_shape_matches_draw_for_a_workload():
    a = gen.draw(0)
    b = gen.draw_shape(gen.SHAPES[0], 0)
    for f in ("x", "attn", "resid", "w_qkv", "w_o", "gain", "router_noise", "s1", "s3", "s2"):
        assert (getattr(a, f) == getattr(b, f)).all(), f


def test_single_launch_sweep_shapes_fit_that_kernel():
    shapes = [ss.random_single_shape(i) for i in range(N_SINGLE_SHAPES)]
    assert all(ss.in_envelope(s) and ss.single_envelope(s) for s in shapes)
    assert any(s.shared_ffn == 0 for s in shapes) and any(s.shared_ffn > 0 for s in shapes)
    assert any(s.batch == 1 for s in shapes) and any(s.batch >= 6 for s in shapes)
    assert any(s.qkv_out > 1024 for s in shapes) and any(s.n_experts > 384 for s in shapes)
