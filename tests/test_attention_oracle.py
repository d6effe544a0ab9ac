"""Pins for the decode-attention oracle (oracle/attention_ref.py), CPU only.

Each pin ties the oracle to something other than itself:
  * the E4M3 format's defining values (zero, the smallest subnormal and
    normal, one, the largest finite value, NaN), counted and ordered;
  * quantisation round trips, clamping, ties to the even code and signed
    zero, checked on explicit values;
  * attention closed forms: one visible key gives its value, equal keys give
    the mean of the values, two keys give sigmoid weights, scales that cancel
    leave the output unchanged;
  * the causal mask among the step's tokens (a later draft cannot change an
    earlier token's output) and grouped heads sharing their KV head;
  * brute force with pure-Python loops and the math module on a tiny step;
  * a mutation test that plants plausible mistakes and checks a pin catches each.
"""
import math

import numpy as np
import pytest

from oracle import attention_ref as A
from synth import attn_gen, gen


def test_e4m3_defining_values():
    v = A.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1, v[0x80]) == -1
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9      # subnormals
    assert v[0x08] == 2.0 ** -6                                  # smallest normal
    assert v[0x38] == 1.0 and v[0xB8] == -1.0 and v[0x39] == 1.125
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(~np.isnan(v)) == 254
    assert np.all(np.diff(v[:0x7F]) > 0)                         # codes ordered like their values


def test_e4m3_quantisation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = A.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(A.e4m3_encode(vals), codes)            # every finite code round-trips
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (1.0624, 0x38), (1.0626, 0x39),   # ties to the even code
             (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),                       # ties among subnormals
             (448.5, 0x7E), (1000.0, 0x7E), (-1000.0, 0xFE), (464.0, 0x7E),     # clamped
             (-0.0, 0x80), (-1e-9, 0x80), (0.0, 0x00), (float("nan"), 0x7F)]
    got = A.e4m3_encode(np.array([x for x, _ in cases], dtype=np.float32))
    assert got.tolist() == [c for _, c in cases]
    # the division by the scale happens in float32 before the decision
    bits = gen.f32_to_bf16_bits(np.array([1.0], np.float32))
    assert A.quantize(bits, np.float32(1 / 64))[0] == A.e4m3_encode(np.float32(1.0) / np.float32(1 / 64))


def _step(R=2, T=3, Hq=4, Hkv=2, C=24, lo=0, hi=12, seed=7, D=16):
    return attn_gen.draw(R, T, Hq, Hkv, C, lo, hi, seed=seed, D=D)


def test_append_writes_only_the_new_positions():
    s = _step()
    kc, vc = A.append_kv(s.k_cache, s.v_cache, s.k_new, s.v_new, s.past_len, s.k_scale, s.v_scale)
    R, T = s.q.shape[:2]
    for r in range(R):
        p0 = int(s.past_len[r])
        new = np.zeros(kc.shape[2], bool)
        new[p0:p0 + T] = True
        assert np.array_equal(kc[r][:, ~new], s.k_cache[r][:, ~new])
        assert np.array_equal(vc[r][:, ~new], s.v_cache[r][:, ~new])
        for j in range(T):
            for g in range(kc.shape[1]):
                x = gen.bf16_bits_to_f32(s.k_new[r, j, g]) / s.k_scale[g]
                assert np.array_equal(kc[r, g, p0 + j], A.e4m3_encode(x.astype(np.float32)))


def test_one_visible_key_gives_its_value():
    s = _step(R=1, T=1, lo=0, hi=0)
    out, kc, vc = A.decode_attention(s.q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.past_len,
                                     s.k_scale, s.v_scale, s.softmax_scale)
    for h in range(s.q.shape[2]):
        g = h // (s.q.shape[2] // kc.shape[1])
        assert np.array_equal(out[0, 0, h], A.e4m3_decode(vc[0, g, 0]) * float(s.v_scale[g]))


def test_equal_keys_average_the_values_and_two_keys_give_sigmoid_weights():
    s = _step(R=1, T=1, lo=5, hi=5)
    kc, vc = s.k_cache.copy(), s.v_cache.copy()
    kc[0, :, :6] = kc[0, :, :1]             # six equal keys (the step's own at position 5 too)
    out = A.attend(s.q, kc, vc, s.past_len, s.k_scale, s.v_scale, s.softmax_scale)
    for h in range(4):
        g = h // 2
        V = A.e4m3_decode(vc[0, g, :6]) * float(s.v_scale[g])
        assert np.allclose(out[0, 0, h], V.mean(axis=0), rtol=1e-13, atol=1e-15)
    s2 = _step(R=1, T=1, lo=1, hi=1)
    out = A.attend(s2.q, s2.k_cache, s2.v_cache, s2.past_len, s2.k_scale, s2.v_scale, s2.softmax_scale)
    q = gen.bf16_bits_to_f32(s2.q[0, 0]).astype(np.float64)
    for h in range(4):
        g = h // 2
        K = A.e4m3_decode(s2.k_cache[0, g, :2]) * float(s2.k_scale[g])
        V = A.e4m3_decode(s2.v_cache[0, g, :2]) * float(s2.v_scale[g])
        d = s2.softmax_scale * (K[1] - K[0]) @ q[h]
        w1 = 1.0 / (1.0 + math.exp(-d))
        assert np.allclose(out[0, 0, h], (1 - w1) * V[0] + w1 * V[1], rtol=1e-12, atol=1e-14)


def test_scales_that_cancel_leave_the_output_unchanged():
    s = _step()
    base = A.attend(s.q, s.k_cache, s.v_cache, s.past_len, s.k_scale, s.v_scale, s.softmax_scale)
    out = A.attend(s.q, s.k_cache, s.v_cache, s.past_len, s.k_scale * np.float32(2), s.v_scale,
                   s.softmax_scale * 0.5)
    assert np.allclose(out, base, rtol=1e-12, atol=1e-15)


def test_drafts_are_causal_and_groups_share_their_kv_head():
    s = _step(T=4)
    out, _, _ = A.decode_attention(s.q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.past_len,
                                   s.k_scale, s.v_scale, s.softmax_scale)
    k2, v2 = s.k_new.copy(), s.v_new.copy()
    k2[:, 2:] ^= np.uint16(0x1234)          # change drafts 2 and 3
    v2[:, 2:] ^= np.uint16(0x0F0F)
    out2, _, _ = A.decode_attention(s.q, k2, v2, s.k_cache, s.v_cache, s.past_len,
                                    s.k_scale, s.v_scale, s.softmax_scale)
    assert np.array_equal(out[:, :2], out2[:, :2])
    assert not np.allclose(out[:, 2:], out2[:, 2:])
    q = s.q.copy()
    q[:, :, 1] = q[:, :, 0]                  # heads 0 and 1 share KV head 0
    q[:, :, 3] = q[:, :, 0]                  # head 3 reads KV head 1
    o, _, _ = A.decode_attention(q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.past_len,
                                 s.k_scale, s.v_scale, s.softmax_scale)
    assert np.array_equal(o[:, :, 0], o[:, :, 1])
    assert not np.allclose(o[:, :, 0], o[:, :, 3])


def brute(s):
    """Pure-Python loops and the math module; codes decoded by their own formula."""
    def dec(c):
        c = int(c)
        e, m = (c >> 3) & 15, c & 7
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        return -v if c & 0x80 else v

    def enc(x):
        best = None
        for c in range(127):
            v = dec(c)
            d = abs(v - min(abs(x), 448.0))
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        return best[1] | (0x80 if math.copysign(1.0, x) < 0 else 0)

    R, T, Hq, Hkv, D, C = s.shape
    kc = [[[list(s.k_cache[r, g, p]) for p in range(C)] for g in range(Hkv)] for r in range(R)]
    vc = [[[list(s.v_cache[r, g, p]) for p in range(C)] for g in range(Hkv)] for r in range(R)]
    for r in range(R):
        for j in range(T):
            for g in range(Hkv):
                for d in range(D):
                    xk = float(np.float32(gen.bf16_bits_to_f32(s.k_new[r, j, g, d]) / s.k_scale[g]))
                    xv = float(np.float32(gen.bf16_bits_to_f32(s.v_new[r, j, g, d]) / s.v_scale[g]))
                    kc[r][g][s.past_len[r] + j][d] = enc(xk)
                    vc[r][g][s.past_len[r] + j][d] = enc(xv)
    out = np.zeros((R, T, Hq, D))
    for r in range(R):
        for j in range(T):
            n = s.past_len[r] + j + 1
            for h in range(Hq):
                g = h // (Hq // Hkv)
                q = [float(gen.bf16_bits_to_f32(x)) for x in s.q[r, j, h]]
                sc = [s.softmax_scale * sum(q[d] * dec(kc[r][g][p][d]) * float(s.k_scale[g]) for d in range(D))
                      for p in range(n)]
                mx = max(sc)
                ex = [math.exp(x - mx) for x in sc]
                tot = sum(ex)
                for d in range(D):
                    out[r, j, h, d] = sum(ex[p] / tot * dec(vc[r][g][p][d]) * float(s.v_scale[g]) for p in range(n))
    return out, np.array(kc, np.uint8), np.array(vc, np.uint8)


def test_matches_brute_force():
    s = _step(R=2, T=3, Hq=4, Hkv=2, C=12, lo=2, hi=6, D=8)
    out, kc, vc = A.decode_attention(s.q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.past_len,
                                     s.k_scale, s.v_scale, s.softmax_scale)
    bo, bk, bv = brute(s)
    assert np.array_equal(kc, bk) and np.array_equal(vc, bv)
    assert np.allclose(out, bo, rtol=1e-12, atol=1e-14)


MUTATIONS = {
    "mask off by one": lambda q, kc, vc, pl, ks, vs, ss: _orig_attend(q, kc, vc, pl + 1, ks, vs, ss),
    "scale dropped": lambda q, kc, vc, pl, ks, vs, ss: _orig_attend(q, kc, vc, pl, ks, vs, 1.0),
    "k_scale dropped": lambda q, kc, vc, pl, ks, vs, ss: _orig_attend(q, kc, vc, pl, np.ones_like(ks), vs, ss),
    "v_scale swapped": lambda q, kc, vc, pl, ks, vs, ss: _orig_attend(q, kc, vc, pl, ks, ks, ss),
    "kv head of h as h % Hkv": lambda q, kc, vc, pl, ks, vs, ss: _orig_attend(
        q[:, :, [0, 2, 1, 3]], kc, vc, pl, ks, vs, ss)[:, :, [0, 2, 1, 3]],
}
_orig_attend = A.attend


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(monkeypatch, name):
    monkeypatch.setattr(A, "attend", MUTATIONS[name])
    caught = 0
    for pin in (test_one_visible_key_gives_its_value, test_equal_keys_average_the_values_and_two_keys_give_sigmoid_weights,
                test_scales_that_cancel_leave_the_output_unchanged, test_drafts_are_causal_and_groups_share_their_kv_head,
                test_matches_brute_force):
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught > 0, name


def test_quantisation_mutation_is_caught(monkeypatch):
    orig = A.e4m3_encode
    monkeypatch.setattr(A, "e4m3_encode", lambda x: orig(np.asarray(x, np.float32) * np.float32(1.0001)))
    with pytest.raises(AssertionError):
        test_e4m3_quantisation()
