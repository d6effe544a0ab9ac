"""The C ABI on the host (CPU only, no GPU calls that compute).

* the built library loads and exports every function include/decode_layer.h declares;
* configuration and step-argument validation return the documented codes and
  a non-empty error text, before any HIP call;
* decode_layer_init on a machine without a GPU fails cleanly with DL_ERR_HIP.
"""
import ctypes
import os
import re

import pytest

import decode_step_moe_amd as dl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    """Every function the headers under include/ declare."""
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(decode_(?:layer|attention)_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert "decode_layer_init" in names and "decode_layer_step" in names and "decode_attention_step" in names
    lib = ctypes.CDLL(dl.binding.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def good():
    return dl.make_config(7168, 512, 512, 384, 8, 128, 128, 64)


@pytest.mark.parametrize("field,value,code", [
    ("hidden", 7170, dl.DL_ERR_UNSUPPORTED), ("hidden", 0, dl.DL_ERR_UNSUPPORTED),
    ("attn_dim", 12, dl.DL_ERR_UNSUPPORTED), ("qkv_out", 0, dl.DL_ERR_UNSUPPORTED),
    ("n_experts", 2000, dl.DL_ERR_UNSUPPORTED), ("top_k", 0, dl.DL_ERR_UNSUPPORTED),
    ("top_k", 65, dl.DL_ERR_UNSUPPORTED), ("expert_ffn", 100, dl.DL_ERR_UNSUPPORTED),
    ("expert_ffn", 512, dl.DL_ERR_UNSUPPORTED), ("shared_ffn", 96, dl.DL_ERR_UNSUPPORTED),
    ("max_batch", 65, dl.DL_ERR_UNSUPPORTED), ("max_batch", 0, dl.DL_ERR_UNSUPPORTED),
    ("rms_eps", 0.0, dl.DL_ERR_UNSUPPORTED), ("rms_eps", float("inf"), dl.DL_ERR_UNSUPPORTED),
    ("score_fn", 1, dl.DL_ERR_UNSUPPORTED), ("renormalize", 0, dl.DL_ERR_UNSUPPORTED),
    ("path", 4, dl.DL_ERR_UNSUPPORTED), ("path", -1, dl.DL_ERR_UNSUPPORTED),
])
def test_config_validation(field, value, code):
    c = good()
    assert dl.check_config(c) == dl.DL_OK
    setattr(c, field, value)
    assert dl.check_config(c) == code
    assert field.split("_")[0] in dl.last_error() or len(dl.last_error()) > 10
    assert dl.scratch_bytes(c) == 0


def test_top_k_above_experts_is_unsupported():
    c = dl.make_config(512, 768, 768, 8, 9, 256, 256, 1)
    assert dl.check_config(c) == dl.DL_ERR_UNSUPPORTED


def test_shared_expert_optional_and_scratch_size():
    c = dl.make_config(512, 768, 768, 8, 2, 256, 0, 1)
    assert dl.check_config(c) == dl.DL_OK
    assert dl.scratch_bytes(good()) > 0


def _a256(n):
    return (n + 255) // 256 * 256


# The hand-off region at the front of every scratch area: tagged words of the
# single-launch path (norm partials [256][8], logits [8192], routed and shared
# activations [8192], [4096]), the step counter, the status word, the wrap
# barrier count, three arrival counters, and the batched path's gate/up group
# and down row-group counters, all sized for the whole envelope.
MAX_GU_GROUPS = (64 * 64 + 7) // 8 * (256 // 32) + (64 + 15) // 16 * (256 // 32)
HANDOFF = (_a256(8 * 256 * 8) + 2 * _a256(8 * 8192) + _a256(8 * 4096) + 3 * 256 + _a256(12)
           + _a256(4 * MAX_GU_GROUPS) + _a256(4 * (16384 // 64)))


def _step_data(B, H, E, K, F, Fs):
    nblk_o = -(-H // 16)
    return (_a256(4 * B * H) + _a256(4 * nblk_o * B) + _a256(4 * B) + _a256(4 * B * E) + 2 * _a256(4 * B * K)
            + 3 * _a256(4 * E) + 256 + _a256(4 * B * K * F) + _a256(4 * B * max(Fs, 1)))


def test_handoff_region_is_configuration_independent():
    """Every scratch area starts with the same hand-off region (so calls with
    different configurations that share one area, as the static area of
    decode_layer_step_noalloc is shared, never read each other's tagged
    words or counters), followed by the step data of the configuration."""
    cases = [(7168, 512, 512, 384, 8, 128, 128, 64), (7168, 1024, 1024, 384, 8, 256, 256, 64),
             (512, 768, 768, 8, 2, 256, 0, 1), (16384, 512, 512, 1024, 32, 32, 64, 3)]
    for (H, Dq, Do, E, K, F, Fs, B) in cases:
        c = dl.make_config(H, Dq, Do, E, K, F, Fs, B, path=dl.DL_PATH_MULTI)
        assert dl.scratch_bytes(c, 256) == HANDOFF + _step_data(B, H, E, K, F, Fs), (H, E, K, F, B)
    # the single-launch path adds nothing beyond the hand-off region
    small = dl.make_config(7168, 512, 512, 384, 8, 128, 128, 8)
    small_multi = dl.make_config(7168, 512, 512, 384, 8, 128, 128, 8, path=dl.DL_PATH_MULTI)
    assert dl.scratch_bytes(small, 256) == dl.scratch_bytes(small_multi, 256)


def test_batched_scratch_follows_the_path():
    """The batched path's arrays (qkv and router partial sums, h in fp32 and
    as bf16 hi + lo planes, gate/up and down partial tiles, the down
    projection's run bounds) exist exactly when some step can take that path."""
    c = good()                       # TP16 shard shapes, max_batch 64
    B, H, Dq, E = 64, 7168, 512, 384
    F = Fs = 128
    groups_r = (B * 8 + 7) // 8 * (F // 64)   # gate/up groups: B*k/8 16-token chunks x 64-row groups
    groups_s = (B + 15) // 16 * (Fs // 64)    # shared expert: 16-token chunks x 64-row groups
    chunks = (H // 32 + 13) // 14             # K chunks of 14 steps of 32: one partial slot each
    batched = (_a256(8 * 4 * B * Dq) + _a256(4 * (H // 256) * B * E) + _a256(4 * B * H)
               + _a256(2 * 2 * B * H) + _a256(4 * 4 * E) + _a256(8)
               + _a256((groups_r + groups_s) * chunks * 2048 * 4)
               + _a256((H // 64) * (-(-512 // (H // 64)) + 2) * 64 * 64 * 4)
               + _a256((512 + 3) * 4))            # down-projection run bounds
    auto = dl.scratch_bytes(c, 256)
    c.path = dl.DL_PATH_MULTI
    multi = dl.scratch_bytes(c, 256)
    c.path = dl.DL_PATH_BATCHED
    forced = dl.scratch_bytes(c, 256)
    assert forced == dl.scratch_bytes(c, 0)
    assert auto == forced == multi + batched
    # a batch the single-launch path covers entirely: no batched arrays under AUTO
    small = dl.make_config(7168, 512, 512, 384, 8, 128, 128, 8)
    assert dl.scratch_bytes(small, 256) == HANDOFF + _step_data(8, 7168, 384, 8, 128, 128)
    # without a single-launch plan (no CU count) AUTO takes the batched path for every batch
    assert dl.scratch_bytes(small, 0) > dl.scratch_bytes(small, 256)
    # shapes the batched tiling cannot take: AUTO never allocates its arrays
    odd_h = dl.make_config(7168 + 256, 512, 512, 384, 8, 128, 128, 64)
    odd_h_multi = dl.make_config(7168 + 256, 512, 512, 384, 8, 128, 128, 64, path=dl.DL_PATH_MULTI)
    assert dl.scratch_bytes(odd_h, 0) == dl.scratch_bytes(odd_h_multi, 0)
    odd_do = dl.make_config(7168, 512, 520, 384, 8, 128, 128, 64)
    odd_do_multi = dl.make_config(7168, 512, 520, 384, 8, 128, 128, 64, path=dl.DL_PATH_MULTI)
    assert dl.scratch_bytes(odd_do, 0) == dl.scratch_bytes(odd_do_multi, 0)


def _io(batch=1, **kw):
    ptrs = dict(x=0x1000, attn=0x2000, resid_in=0x3000, qkv=0x4000, resid_out=0x100000,
                router_logits=None, topk_idx=0x5000, topk_w=0x6000, moe_out=0x200000, h_out=None)
    ptrs.update(kw)
    return dl.IO(batch, *[ptrs[n] for n in ("x", "attn", "resid_in", "qkv", "resid_out",
                                             "router_logits", "topk_idx", "topk_w", "moe_out",
                                             "h_out")])


def test_io_validation():
    c = good()
    assert dl.check_io(c, _io()) == dl.DL_OK
    assert dl.check_io(c, _io(batch=0, x=None)) == dl.DL_OK          # no-op
    assert dl.check_io(c, _io(batch=-1)) == dl.DL_ERR_INVALID_ARG
    assert dl.check_io(c, _io(batch=65)) == dl.DL_ERR_UNSUPPORTED
    assert dl.check_io(c, _io(x=None)) == dl.DL_ERR_INVALID_ARG
    assert "io.x" in dl.last_error()
    assert dl.check_io(c, _io(moe_out=0x200004)) == dl.DL_ERR_INVALID_ARG   # misaligned
    assert dl.check_io(c, _io(router_logits=0x7008)) == dl.DL_ERR_INVALID_ARG
    assert dl.check_io(c, _io(resid_out=0x3000)) == dl.DL_OK                # exact alias allowed
    assert dl.check_io(c, _io(resid_out=0x3010)) == dl.DL_ERR_INVALID_ARG   # partial overlap


def test_init_rejects_bad_arguments_before_touching_the_gpu():
    lib = dl.lib()
    out = ctypes.c_void_p(123)
    w = dl.Weights(*([0x1000] * 10))
    bad = good()
    bad.top_k = 0
    rc = lib.decode_layer_init(ctypes.byref(bad), ctypes.byref(w), 0, ctypes.byref(out))
    assert rc == dl.DL_ERR_UNSUPPORTED and not out.value
    w_null = dl.Weights(*([0x1000] * 3 + [None] + [0x1000] * 6))
    rc = lib.decode_layer_init(ctypes.byref(good()), ctypes.byref(w_null), 0, ctypes.byref(out))
    assert rc == dl.DL_ERR_INVALID_ARG and "w_router" in dl.last_error()
    w_mis = dl.Weights(*([0x1000] * 4 + [0x1002] + [0x1000] * 5))
    rc = lib.decode_layer_init(ctypes.byref(good()), ctypes.byref(w_mis), 0, ctypes.byref(out))
    assert rc == dl.DL_ERR_INVALID_ARG and "aligned" in dl.last_error()


def test_step_and_destroy_null_handle():
    lib = dl.lib()
    assert lib.decode_layer_step(None, ctypes.byref(_io()), None) == dl.DL_ERR_INVALID_ARG
    assert lib.decode_layer_destroy(None) == dl.DL_OK
    assert lib.decode_layer_set_profiling(None, 1) == dl.DL_ERR_INVALID_ARG
    assert lib.decode_layer_set_spin_limit(None, 0) == dl.DL_ERR_INVALID_ARG
    assert lib.decode_layer_set_step_counter(None, 5) == dl.DL_ERR_INVALID_ARG


def test_library_exports_only_the_abi():
    """Built with hidden visibility: the dynamic symbol table holds the C ABI
    of include/decode_layer.h and nothing else of the library's own."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", dl.binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    text_syms = sorted({ln.split()[-1] for ln in out.splitlines() if ln.split()[1:2] == ["T"]})
    assert text_syms == header_functions(), set(text_syms) ^ set(header_functions())


def test_init_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = dl.lib()
    out = ctypes.c_void_p()
    w = dl.Weights(*([0x1000] * 10))
    rc = lib.decode_layer_init(ctypes.byref(good()), ctypes.byref(w), 0, ctypes.byref(out))
    assert rc == dl.DL_ERR_HIP and not out.value
    assert len(dl.last_error()) > 0


# ---------------------------------------------------------------- attention core
def _attn_cfg(**kw):
    from decode_step_moe_amd import attention as at
    c = dict(n_q_heads=4, n_kv_heads=1, max_tokens=8, max_requests=64, cache_len=4096, softmax_scale=128 ** -0.5)
    c.update(kw)
    return at.make_attn_config(**c)


def test_attention_workspace_and_validation():
    from decode_step_moe_amd import attention as at
    c = _attn_cfg()
    chunks = -(-4096 // 256)
    slots = 64 * 1 * chunks * (32 * 128 + 64) * 4
    # 4 query heads x 8 tokens = 32 rows per KV head: two row splits of 16, each with its counter
    assert at.workspace_bytes(c) == _a256(slots) + _a256(64 * 2 * 4)
    # at most 64 partial slots per request and KV head, whatever the cache length
    big = _attn_cfg(cache_len=1 << 20, max_requests=2)
    assert at.workspace_bytes(big) == _a256(2 * 64 * (32 * 128 + 64) * 4) + _a256(2 * 4)
    assert at.workspace_bytes(_attn_cfg(max_splits=3)) == at.workspace_bytes(c)
    for field, value in (("head_dim", 64), ("max_tokens", 9), ("max_tokens", 0), ("n_kv_heads", 3),
                         ("n_q_heads", 40), ("cache_len", 0), ("softmax_scale", 0.0), ("max_requests", 2000),
                         ("max_splits", -1)):
        bad = _attn_cfg(**{field: value}) if field != "head_dim" else at.make_attn_config(4, 1, 8, 64, 4096, 0.1, 64)
        assert at.workspace_bytes(bad) == 0, field
    # (Hq / Hkv) * T must fit 32 query rows per KV head
    assert at.workspace_bytes(_attn_cfg(n_q_heads=8, max_tokens=8)) == 0
    assert at.workspace_bytes(_attn_cfg(n_q_heads=8, n_kv_heads=2, max_tokens=8)) > 0

    def io(**kw):
        p = dict(past_len=0x1000, q=0x2000, k_new=0x3000, v_new=0x4000, k_cache=0x5000, v_cache=0x6000,
                 k_scale=0x7000, v_scale=0x8000, out=0x9000, workspace=0x10000)
        n = dict(n_requests=2, n_tokens=8, max_past=100)
        p.update({k: v for k, v in kw.items() if k in p})
        n.update({k: v for k, v in kw.items() if k in n})
        return at.AttnIO(n["n_requests"], n["n_tokens"], n["max_past"],
                         *[p[k] for k in ("past_len", "q", "k_new", "v_new", "k_cache", "v_cache", "k_scale",
                                          "v_scale", "out", "workspace")])
    assert at.check(c, io()) == dl.DL_OK
    assert at.check(c, io(n_requests=0, q=None)) == dl.DL_OK
    assert at.check(c, io(n_requests=65)) == dl.DL_ERR_UNSUPPORTED
    assert at.check(c, io(n_tokens=9)) == dl.DL_ERR_UNSUPPORTED
    assert at.check(c, io(max_past=4089)) == dl.DL_ERR_UNSUPPORTED      # max_past + T > cache_len
    assert at.check(c, io(q=None)) == dl.DL_ERR_INVALID_ARG
    assert at.check(c, io(out=0x9004)) == dl.DL_ERR_INVALID_ARG
    assert at.check(c, io(workspace=0x10010)) == dl.DL_ERR_INVALID_ARG  # 256-byte alignment
    assert "workspace" in dl.last_error()


def test_kernels_use_no_scratch_memory(tmp_path):
    """Every kernel of the built library keeps its state in registers and LDS:
    a kernel with a private segment (a stack, or an array spilled to scratch
    memory) runs every phase far slower, so the device code objects of the
    objects the build compiled are read back and each kernel's fixed private
    segment size must be 0."""
    import glob
    import subprocess
    llvm = "/opt/rocm/lib/llvm/bin"
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.o")))
    tools = [os.path.join(llvm, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not objs or not all(os.path.exists(t) for t in tools):
        pytest.skip("no build objects or no LLVM tools")
    seen = {}
    for o in objs:
        base = os.path.splitext(os.path.basename(o))[0]
        fb, co = tmp_path / f"{base}.fatbin", tmp_path / f"{base}.co"
        r = subprocess.run([tools[0], f"--dump-section=.hip_fatbin={fb}", o, str(tmp_path / f"{base}.host.o")],
                           capture_output=True, text=True)
        if r.returncode != 0 and "not found" in r.stderr:
            continue   # host code only
        assert r.returncode == 0, r.stderr
        subprocess.run([tools[1], "--unbundle", "--type=o", f"--input={fb}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                       check=True, capture_output=True)
        notes = subprocess.run([tools[2], "--notes", str(co)], check=True, capture_output=True, text=True).stdout
        names = re.findall(r"^\s+\.name:\s+(\S+)$", notes, re.M)
        sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)
        assert len(names) == len(sizes), base
        seen.update({n: int(sz) for n, sz in zip(names, sizes)})
    assert any("fused_step_kernel" in n for n in seen) and any("gateup_b" in n for n in seen)
    assert {n: sz for n, sz in seen.items() if sz} == {}
