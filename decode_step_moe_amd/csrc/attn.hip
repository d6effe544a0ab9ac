// Decode attention core: grouped-query attention over an FP8 (OCP E4M3) KV
// cache for 1 to 8 query tokens per request, the step's own tokens appended
// first (C ABI in include/decode_attention.h).
//
// The pages decode with an FP8 KV cache and verify up to 7 speculative
// drafts per step (bigchange.ai "Kimi K3 vLLM GPU inference benchmark",
// section "Where the time was going").  Decode attention reads every cached
// key and value once per step, so it is bound by HBM bandwidth at long
// contexts and by latency at short ones; the cache is read one byte per value
// and decoded on the fly.
//
// Two launches on the caller's stream:
//  1 attn_append  quantises the step's keys and values (x / scale in fp32,
//                 nearest E4M3 code, ties to even, clamped to +-448) into
//                 positions past_len .. past_len + T - 1 of each request.
//  2 attn_chunk   one workgroup per (chunk of 256 positions, request, KV
//                 head): S = Q K^T on the matrix cores (v_mfma_f32_16x16x32_bf16;
//                 queries are bf16 already and every E4M3 value is exact in
//                 bf16), the causal mask (query token j sees positions up to
//                 past_len + j), the chunk's row maxima and sums, then
//                 P V on the matrix cores with P as bf16 hi + lo and V from LDS.
//                 The chunk's (max, sum, P V) go to its slot; the last
//                 workgroup of the (request, KV head) to arrive combines the
//                 slots in chunk order and writes the outputs.
// Rows: the T tokens x Hq/Hkv heads of one KV head (at most 32), in 16-row
// matrix-core tiles.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "../../include/decode_attention.h"
#include "common.h"
#include "layer_host.h"

namespace dl {
namespace {

constexpr int kAD = 128;                               // head size
constexpr int kAChunk = 256;                           // cache positions per workgroup
constexpr int kAMaxRows = 32;                          // query rows per KV head
constexpr int kASlot = kAMaxRows * kAD + 2 * kAMaxRows; // floats per chunk slot: P V, max, sum

typedef __bf16 bf16x8a __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2a __attribute__((ext_vector_type(2)));
typedef float f32x4a __attribute__((ext_vector_type(4)));
typedef float f32x2a __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const int32_t *past_len;
  const uint16_t *q, *k_new, *v_new;
  uint8_t *k_cache, *v_cache;
  const float *k_scale, *v_scale;
  float *out;
  float *slots;        // [max_requests * Hkv][n_chunk_max][kASlot]
  unsigned *counters;  // [max_requests * Hkv]
  int R, T, Hq, Hkv, C, max_past, grp, M, n_chunk_max;
  float softmax_scale;
};

__device__ __forceinline__ f32x4a mfma16(const uint4 &a, const uint4 &b, f32x4a c) {
  v4u ua = {a.x, a.y, a.z, a.w}, ub = {b.x, b.y, b.z, b.w};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8a, ua), __builtin_bit_cast(bf16x8a, ub),
                                                 c, 0, 0, 0);
}

// x (fp32) -> E4M3 code: nearest value, ties to the even code, magnitudes of
// 448 and above clamped to 448, the sign kept, NaN -> 0x7F.
__device__ __forceinline__ unsigned e4m3_encode(float x) {
  const unsigned u = __float_as_uint(x);
  const unsigned sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) {                            // below the smallest normal 2^-6: steps of 2^-9
    return sign | (unsigned)rintf(a * 512.f);     // exact scaling, round half to even; 8 is 2^-6
  }
  int e = (int)((u >> 23) & 0xFFu) - 127;         // -6 .. 8
  const unsigned mant = u & 0x7FFFFFu;
  unsigned m3 = mant >> 20;
  const unsigned rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  if (m3 == 8u) {
    m3 = 0u;
    ++e;
  }
  return sign | ((unsigned)(e + 7) << 3) | m3;
}

// E4M3 code -> bf16 bits of the same value (exact), NaN codes -> a bf16 NaN.
__device__ __forceinline__ uint16_t e4m3_to_bf16(unsigned c) {
  const unsigned s = (c & 0x80u) << 8, e = (c >> 3) & 15u, m = c & 7u;
  if (e == 15u && m == 7u) return (uint16_t)(s | 0x7FC0u);
  if (e != 0u) return (uint16_t)(s | ((e + 120u) << 7) | (m << 4));
  if (m == 0u) return (uint16_t)s;
  // subnormal m * 2^-9: shift the leading bit of m into the implicit one
  const unsigned lz = m >= 4u ? 0u : m >= 2u ? 1u : 2u;  // leading zeros of m in 3 bits
  const unsigned ex = 120u - lz;                        // 2^-7 for m >= 4
  const unsigned mm = ((m << (lz + 1u)) & 7u) << 4;
  return (uint16_t)(s | (ex << 7) | mm);
}

__device__ __forceinline__ unsigned pack2_bf16(float a, float b) {  // round to nearest even
  f32x2a f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2a));
}
// x = hi + lo: hi truncated to bf16 (x - hi exact in fp32), lo = bf16(x - hi).
__device__ __forceinline__ void split_hi_lo(const float (&x)[8], uint4 &hi, uint4 &lo) {
  unsigned h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned ua = __float_as_uint(x[2 * j]) & 0xffff0000u;
    const unsigned ub = __float_as_uint(x[2 * j + 1]) & 0xffff0000u;
    h[j] = (ua >> 16) | ub;
    l[j] = pack2_bf16(x[2 * j] - __uint_as_float(ua), x[2 * j + 1] - __uint_as_float(ub));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppMirror>(v));
  return v;
}

__device__ __forceinline__ bool request_bad(const AttnArgs &a, int L) {
  return L < 0 || L > a.max_past || L + a.T > a.C;
}

// ---- launch 1 ---------------------------------------------------------------
// Thread: 8 consecutive elements of one (request, token, KV head) row.
__global__ void __launch_bounds__(256) attn_append(AttnArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int row = t >> 4, part = t & 15;           // row = (r T + j) Hkv + g
  if (row >= a.R * a.T * a.Hkv) return;
  const int g = row % a.Hkv, rj = row / a.Hkv, j = rj % a.T, r = rj / a.T;
  const int L = a.past_len[r];
  if (request_bad(a, L)) return;
  const size_t src = (size_t)row * kAD + part * 8;
  float kf[8], vf[8];
  unpack8(ld16(a.k_new + src), kf);
  unpack8(ld16(a.v_new + src), vf);
  const float ks = a.k_scale[g], vs = a.v_scale[g];
  unsigned kw[2] = {0u, 0u}, vw[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    kw[i >> 2] |= e4m3_encode(kf[i] / ks) << (8 * (i & 3));
    vw[i >> 2] |= e4m3_encode(vf[i] / vs) << (8 * (i & 3));
  }
  const size_t dst = ((size_t)(r * a.Hkv + g) * a.C + L + j) * kAD + part * 8;
  *reinterpret_cast<uint2 *>(a.k_cache + dst) = make_uint2(kw[0], kw[1]);
  *reinterpret_cast<uint2 *>(a.v_cache + dst) = make_uint2(vw[0], vw[1]);
}

// ---- launch 2 ---------------------------------------------------------------
__global__ void __launch_bounds__(256, 2) attn_chunk(AttnArgs a) {
  __shared__ uint16_t lut[256];
  __shared__ __align__(16) uint8_t vsh[kAChunk * kAD];      // V rows of the chunk (E4M3)
  __shared__ __align__(16) float psh[kAMaxRows][kAChunk];   // P of the chunk
  __shared__ float redm[4][kAMaxRows], redl[4][kAMaxRows];
  __shared__ float rowm[kAMaxRows], rowl[kAMaxRows];
  __shared__ int s_last;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g4 = lane >> 4;
  const int c = blockIdx.x, rg = blockIdx.y, r = rg / a.Hkv, g = rg % a.Hkv;
  const int L = a.past_len[r];
  const int M = a.M, grp = a.grp;
  if (request_bad(a, L)) {
    // an impossible length: this request's outputs are NaN, nothing else runs
    if (c == 0)
      for (int q = tid; q < M * kAD; q += 256) {
        const int row = q / kAD, d = q % kAD, j = row / grp, h = g * grp + row % grp;
        a.out[((size_t)(r * a.T + j) * a.Hq + h) * kAD + d] = __builtin_nanf("");
      }
    return;
  }
  const int len = L + a.T;                              // positions after the append
  const int nch = (len + kAChunk - 1) / kAChunk;
  if (c >= nch) return;                                 // past this request's end: not counted
  const int p0 = c * kAChunk;
  const size_t cbase = (size_t)rg * a.C * kAD;
  // every load up front (addresses clamped to the request's last position):
  // this thread's 8 words of the chunk's V rows, its wave's K fragments, its
  // query fragments
  uint4 vst[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int w = tid + 256 * k, p = min(p0 + (w >> 3), len - 1);
    vst[k] = ld16(a.v_cache + cbase + (size_t)p * kAD + 16 * (w & 7));
  }
  uint2 kr[4][4];  // [key tile][K step]: key p0 + 64 wv + 16 kt + n, elements 32 s + 8 g4 ..
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int p = min(p0 + 64 * wv + 16 * kt + n, len - 1);
    const uint8_t *kp = a.k_cache + cbase + (size_t)p * kAD + 8 * g4;
#pragma unroll
    for (int s = 0; s < 4; ++s) kr[kt][s] = *reinterpret_cast<const uint2 *>(kp + 32 * s);
  }
  uint4 qa[2][4];  // [row tile][K step]: row rt 16 + n
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = min(rt * 16 + n, M - 1), j = row / grp, h = g * grp + row % grp;
    const uint16_t *qp = a.q + ((size_t)(r * a.T + j) * a.Hq + h) * kAD + 8 * g4;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[rt][s] = ld16(qp + 32 * s);
  }
  lut[tid] = e4m3_to_bf16((unsigned)tid);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int w = tid + 256 * k;
    reinterpret_cast<uint4 *>(vsh)[w] = p0 + (w >> 3) < len ? vst[k] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  const int nrt = (M + 15) >> 4;
  // ---- S = Q K^T for this wave's 64 positions
  f32x4a acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[rt][kt] = f32x4a{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint2 b = kr[kt][s];
      const uint4 kb = make_uint4(lut[b.x & 255u] | ((unsigned)lut[(b.x >> 8) & 255u] << 16),
                                  lut[(b.x >> 16) & 255u] | ((unsigned)lut[b.x >> 24] << 16),
                                  lut[b.y & 255u] | ((unsigned)lut[(b.y >> 8) & 255u] << 16),
                                  lut[(b.y >> 16) & 255u] | ((unsigned)lut[b.y >> 24] << 16));
      acc[0][kt] = mfma16(qa[0][s], kb, acc[0][kt]);
      if (nrt > 1) acc[1][kt] = mfma16(qa[1][s], kb, acc[1][kt]);
    }
  // ---- scale, mask, the chunk's row maxima
  const float sc = a.softmax_scale * a.k_scale[g];
  const float kNegInf = -__builtin_inff();
  float mx[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * 16 + 4 * g4 + i, lim = L + row / grp;  // last visible position
      float m = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int p = p0 + 64 * wv + 16 * kt + n;
        const float v = row < M && p <= lim ? acc[rt][kt][i] * sc : kNegInf;
        acc[rt][kt][i] = v;
        m = fmaxf(m, v);
      }
      mx[rt][i] = row16_max(m);
    }
  if (n == 0)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) redm[wv][rt * 16 + 4 * g4 + i] = mx[rt][i];
  __syncthreads();
  if (tid < kAMaxRows) rowm[tid] = fmaxf(fmaxf(redm[0][tid], redm[1][tid]), fmaxf(redm[2][tid], redm[3][tid]));
  __syncthreads();
  // ---- P = exp(S - max) (0 where masked), the chunk's row sums
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * 16 + 4 * g4 + i;
      const float m = rowm[row];
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const float v = acc[rt][kt][i];
        const float p = v == kNegInf ? 0.f : expf(v - m);
        psh[row][64 * wv + 16 * kt + n] = p;
        sum += p;
      }
      sum = row16_sum(sum);
      if (n == 0) redl[wv][row] = sum;
    }
  __syncthreads();
  if (tid < kAMaxRows) rowl[tid] = ((redl[0][tid] + redl[1][tid]) + redl[2][tid]) + redl[3][tid];
  // ---- O = P V: wave wv takes columns 32 wv .. 32 wv + 31 over the chunk
  f32x4a o[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) o[rt][dt] = f32x4a{0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < kAChunk / 32; ++ks) {
    uint4 vb[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const uint8_t *vp = vsh + (32 * ks + 8 * g4) * kAD + 32 * wv + 16 * dt + n;
      unsigned h[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) h[jj] = lut[vp[jj * kAD]];
      vb[dt] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      if (rt >= nrt) break;
      const float *pp = &psh[rt * 16 + n][32 * ks + 8 * g4];
      const float4 x0 = *reinterpret_cast<const float4 *>(pp), x1 = *reinterpret_cast<const float4 *>(pp + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint4 hi, lo;
      split_hi_lo(x, hi, lo);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        o[rt][dt] = mfma16(hi, vb[dt], o[rt][dt]);
        o[rt][dt] = mfma16(lo, vb[dt], o[rt][dt]);
      }
    }
  }
  // ---- this chunk's slot: P V (row, column), max, sum; written through
  float *slot = a.slots + ((size_t)rg * a.n_chunk_max + c) * kASlot;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + 4 * g4 + i, d = 32 * wv + 16 * dt + n;
        if (row < M) __hip_atomic_store(slot + row * kAD + d, o[rt][dt][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  __syncthreads();
  if (tid < M) {
    __hip_atomic_store(slot + kAMaxRows * kAD + tid, rowm[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slot + kAMaxRows * kAD + kAMaxRows + tid, rowl[tid], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  wt_stores_complete();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.counters + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)nch - 1u;
    if (s_last) __hip_atomic_store(a.counters + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  // ---- the last chunk of (request, KV head): combine the slots in chunk order
  const float *slots = a.slots + (size_t)rg * a.n_chunk_max * kASlot;
  for (int q = tid; q < M * (kAD / 16); q += 256) {
    const int row = q / (kAD / 16), d0 = 16 * (q % (kAD / 16));
    float m = kNegInf, l = 0.f, acc16[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc16[e] = 0.f;
    for (int cc = 0; cc < nch; ++cc) {
      const float *sl = slots + (size_t)cc * kASlot;
      const float mc = __hip_atomic_load(sl + kAMaxRows * kAD + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (mc == kNegInf) continue;   // no visible position of this row in that chunk
      const float lc = __hip_atomic_load(sl + kAMaxRows * kAD + kAMaxRows + row, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      if (mc > m) {
        const float f = m == kNegInf ? 0.f : expf(m - mc);
        l *= f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc16[e] *= f;
        m = mc;
      }
      const float f = expf(mc - m);
      l += lc * f;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        acc16[e] += f * __hip_atomic_load(sl + row * kAD + d0 + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int j = row / grp, h = g * grp + row % grp;
    float *op = a.out + ((size_t)(r * a.T + j) * a.Hq + h) * kAD + d0;
    const float inv = a.v_scale[g] / l;  // V entered as its E4M3 values: scale once here
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<float4 *>(op + e) = make_float4(acc16[e] * inv, acc16[e + 1] * inv, acc16[e + 2] * inv,
                                                        acc16[e + 3] * inv);
  }
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cfg(const decode_attention_config *c) {
  using host::fail;
  if (!c) return fail(nullptr, DL_ERR_INVALID_ARG, "attention config is NULL");
  if (c->head_dim != kAD) return fail(nullptr, DL_ERR_UNSUPPORTED, "head_dim=%d: only 128 is supported", c->head_dim);
  if (c->n_kv_heads < 1 || c->n_kv_heads > 64 || c->n_q_heads < 1 || c->n_q_heads > 256 ||
      c->n_q_heads % c->n_kv_heads)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "heads: need 1 <= n_kv_heads <= 64 dividing n_q_heads <= 256 (%d, %d)",
                c->n_q_heads, c->n_kv_heads);
  if (c->max_tokens < 1 || c->max_tokens > 8)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "max_tokens=%d: need 1..8", c->max_tokens);
  if (c->n_q_heads / c->n_kv_heads * c->max_tokens > kAMaxRows)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "(n_q_heads / n_kv_heads) * max_tokens must be <= %d", kAMaxRows);
  if (c->max_requests < 1 || c->max_requests > 1024 || (long)c->max_requests * c->n_kv_heads > 65535)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "max_requests=%d: need 1..1024 and max_requests * n_kv_heads <= 65535",
                c->max_requests);
  if (c->cache_len < 1 || c->cache_len > (1 << 20))
    return fail(nullptr, DL_ERR_UNSUPPORTED, "cache_len=%d: need 1..2^20", c->cache_len);
  if (!(c->softmax_scale > 0.f) || !std::isfinite(c->softmax_scale))
    return fail(nullptr, DL_ERR_UNSUPPORTED, "softmax_scale must be positive and finite");
  return DL_OK;
}

int check_io(const decode_attention_config *c, const decode_attention_io *io) {
  using host::fail;
  int rc = check_cfg(c);
  if (rc != DL_OK) return rc;
  if (!io) return fail(nullptr, DL_ERR_INVALID_ARG, "attention io is NULL");
  if (io->n_requests < 0) return fail(nullptr, DL_ERR_INVALID_ARG, "n_requests=%d is negative", io->n_requests);
  if (io->n_requests > c->max_requests)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "n_requests=%d exceeds max_requests=%d", io->n_requests, c->max_requests);
  if (io->n_requests == 0) return DL_OK;
  if (io->n_tokens < 1 || io->n_tokens > c->max_tokens)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "n_tokens=%d: need 1..max_tokens=%d", io->n_tokens, c->max_tokens);
  if (io->max_past < 0 || (long)io->max_past + io->n_tokens > c->cache_len)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "max_past=%d: need 0 <= max_past and max_past + n_tokens <= cache_len=%d",
                io->max_past, c->cache_len);
  const void *req[] = {io->past_len, io->q, io->k_new, io->v_new, io->k_cache, io->v_cache,
                       io->k_scale, io->v_scale, io->out, io->workspace};
  const char *names[] = {"past_len", "q", "k_new", "v_new", "k_cache", "v_cache", "k_scale", "v_scale", "out",
                         "workspace"};
  for (int i = 0; i < 10; ++i) {
    if (!req[i]) return fail(nullptr, DL_ERR_INVALID_ARG, "attention io.%s is NULL", names[i]);
    if (!aligned16(req[i])) return fail(nullptr, DL_ERR_INVALID_ARG, "attention io.%s is not 16-byte aligned", names[i]);
  }
  if (reinterpret_cast<uintptr_t>(io->workspace) & 255u)
    return fail(nullptr, DL_ERR_INVALID_ARG, "attention io.workspace is not 256-byte aligned");
  return DL_OK;
}

size_t slot_bytes(const decode_attention_config *c) {
  return (size_t)c->max_requests * c->n_kv_heads * ((c->cache_len + kAChunk - 1) / kAChunk) * kASlot * 4;
}

}  // namespace
}  // namespace dl

using namespace dl;

extern "C" {

size_t decode_attention_workspace_bytes(const decode_attention_config *cfg) {
  if (check_cfg(cfg) != DL_OK) return 0;
  return align256(slot_bytes(cfg)) + align256((size_t)cfg->max_requests * cfg->n_kv_heads * 4);
}

int decode_attention_check(const decode_attention_config *cfg, const decode_attention_io *io) {
  return check_io(cfg, io);
}

int decode_attention_step(const decode_attention_config *cfg, const decode_attention_io *io, void *hip_stream) {
  int rc = check_io(cfg, io);
  if (rc != DL_OK) return rc;
  if (io->n_requests == 0) return DL_OK;
  const hipStream_t st = (hipStream_t)hip_stream;
  AttnArgs a{};
  a.past_len = io->past_len;
  a.q = (const uint16_t *)io->q;
  a.k_new = (const uint16_t *)io->k_new;
  a.v_new = (const uint16_t *)io->v_new;
  a.k_cache = io->k_cache;
  a.v_cache = io->v_cache;
  a.k_scale = io->k_scale;
  a.v_scale = io->v_scale;
  a.out = io->out;
  a.slots = (float *)io->workspace;
  a.counters = (unsigned *)((char *)io->workspace + align256(slot_bytes(cfg)));
  a.R = io->n_requests;
  a.T = io->n_tokens;
  a.Hq = cfg->n_q_heads;
  a.Hkv = cfg->n_kv_heads;
  a.C = cfg->cache_len;
  a.max_past = io->max_past;
  a.grp = cfg->n_q_heads / cfg->n_kv_heads;
  a.M = a.grp * a.T;
  a.n_chunk_max = (cfg->cache_len + kAChunk - 1) / kAChunk;
  a.softmax_scale = cfg->softmax_scale;
  const int rows = a.R * a.T * a.Hkv;
  hipLaunchKernelGGL(attn_append, dim3((rows * 16 + 255) / 256), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return host::fail(nullptr, DL_ERR_HIP, "attention append launch failed: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(attn_chunk, dim3((io->max_past + a.T + kAChunk - 1) / kAChunk, a.R * a.Hkv), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return host::fail(nullptr, DL_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return DL_OK;
}

}  // extern "C"
