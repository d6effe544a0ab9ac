"""CPU oracle for the decode attention core with an FP8 KV cache and
speculative-verify masking: plain, slow, float64 for the arithmetic.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path imports,
calls or links this file.  It may be used only by tests/, by the smoke check
in __graft_entry__.py and by bench.py's CPU-baseline leg.  It shares no code
with the HIP kernels.

What it computes, and where that is stated:

  * The pages run decode with an FP8 KV cache and verify 3 to 7 draft tokens
    of the DSpark speculative decoder in one step (bigchange.ai "Kimi K3 vLLM
    GPU inference benchmark", section "Where the time was going").  Neither
    page gives the attention's heads, head size, cache layout or masking;
    the readings below are the plainest ones that fit the layer-step the
    library is measured on (its out-projection consumes 512 attention
    outputs per TP16 shard: 4 query heads of 128).
  * Grouped-query attention: query head h reads KV head h // (Hq / Hkv).
  * The KV cache holds OCP FP8 E4M3 codes (4 exponent bits with bias 7, 3
    mantissa bits, no infinities, 0x7F/0xFF NaN, largest finite 448) and one
    fp32 dequantisation scale per KV head: value = decode(code) * scale.
  * A step of T query tokens per request (1 verified token plus T - 1
    drafts): the new tokens' keys and values are quantised and written to
    positions past_len .. past_len + T - 1 of the request's cache, then query
    token j attends to positions 0 .. past_len + j (causal among the new
    tokens), reading the new tokens back from the cache as the FP8 values
    later steps will see.
  * Quantisation: q = x / scale in float32 (IEEE, round to nearest), then the
    nearest E4M3 value, ties to the even code, magnitudes beyond 448 clamped
    to 448, the sign kept (so -0.0 and small negatives give 0x80).  That
    integer decision is taken in float32, the precision the kernel decides in.
  * Scores s = softmax_scale * (q . k), p = softmax over the visible keys,
    out = sum_s p_s v_s, all in float64.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64, from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** (1 - 7), (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, val)


_POS_CODES = np.arange(0x7F, dtype=np.uint8)        # the 127 non-negative finite codes
_POS_VALS = e4m3_decode(_POS_CODES)


def e4m3_encode(x32) -> np.ndarray:
    """float32 values -> nearest E4M3 codes (ties to the even code, clamped to
    +-448, sign kept, NaN -> 0x7F), by comparing with every finite code."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    even_code = (_POS_CODES % 2 == 0)[None, :]
    for c0 in range(0, flat.size, 4096):
        v = flat[c0:c0 + 4096]
        a = np.minimum(np.abs(np.nan_to_num(v)), E4M3_MAX)
        d = np.abs(_POS_VALS[None, :] - a[:, None])
        tie = d == d.min(axis=1, keepdims=True)       # one code, or two neighbours (one of them even)
        even = tie & even_code
        code = np.where(even.any(axis=1), even.argmax(axis=1), tie.argmax(axis=1)).astype(np.uint8)
        code |= np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
        out[c0:c0 + 4096] = np.where(np.isnan(v), np.uint8(0x7F), code)
    return out.reshape(x.shape)


def quantize(x_bits_bf16, scale) -> np.ndarray:
    """bf16 values (uint16 bits) divided by a float32 scale in float32, then encoded."""
    b = np.asarray(x_bits_bf16, dtype=np.uint16)
    x = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    q = (x / np.float32(scale)).astype(np.float32)
    return e4m3_encode(q)


def append_kv(k_cache, v_cache, k_new, v_new, past_len, k_scale, v_scale):
    """Returns copies of the caches ([R][Hkv][C][D] uint8) with the step's
    tokens (k_new, v_new: bf16 bits [R][T][Hkv][D]) written at positions
    past_len[r] .. past_len[r] + T - 1."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    R, T, Hkv, _ = k_new.shape
    for r in range(R):
        for j in range(T):
            pos = int(past_len[r]) + j
            for g in range(Hkv):
                kc[r, g, pos] = quantize(k_new[r, j, g], k_scale[g])
                vc[r, g, pos] = quantize(v_new[r, j, g], v_scale[g])
    return kc, vc


def attend(q_bits, k_cache, v_cache, past_len, k_scale, v_scale, softmax_scale) -> np.ndarray:
    """out [R][T][Hq][D] (float64) of query tokens q (bf16 bits [R][T][Hq][D])
    over caches that already hold the step's tokens."""
    q = (np.asarray(q_bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    R, T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    grp = Hq // Hkv
    out = np.zeros((R, T, Hq, D))
    for r in range(R):
        for j in range(T):
            n = int(past_len[r]) + j + 1          # visible keys: positions 0 .. past_len + j
            for h in range(Hq):
                g = h // grp
                K = e4m3_decode(k_cache[r, g, :n]) * float(k_scale[g])
                V = e4m3_decode(v_cache[r, g, :n]) * float(v_scale[g])
                s = float(softmax_scale) * (K @ q[r, j, h])
                p = np.exp(s - s.max())
                p /= p.sum()
                out[r, j, h] = p @ V
    return out


def decode_attention(q_bits, k_new, v_new, k_cache, v_cache, past_len, k_scale, v_scale, softmax_scale):
    """One step: append the new tokens, then attend.  Returns (out, k_cache, v_cache)."""
    kc, vc = append_kv(k_cache, v_cache, k_new, v_new, past_len, k_scale, v_scale)
    return attend(q_bits, kc, vc, past_len, k_scale, v_scale, softmax_scale), kc, vc
