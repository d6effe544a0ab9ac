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
// One launch on the caller's stream, one workgroup of 4 waves per (split,
// request, KV head); a split takes tps consecutive tiles of 256 positions,
// 64 per wave.  Rows are the T tokens x Hq/Hkv query heads of the KV head
// (at most 32, in 16-row matrix-core tiles).  Per tile, each wave on its own:
//  - loads its 64 keys' K and V codes (the step's own positions are
//    quantised from k_new / v_new instead, x / scale in fp32 to the nearest
//    E4M3 code, and written to the cache by the lane holding them);
//  - S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16; the codes
//    are decoded to bf16 by the hardware conversion, exactly, and queries
//    are bf16 already), the causal mask (token j sees positions up to
//    past_len + j), an online softmax of its own;
//  - O^T += V^T P^T on the matrix cores, P as bf16 hi + lo straight from the
//    S^T registers, V^T from the wave's own LDS slice (byte-transposed in
//    registers on the way in), so no barrier is needed inside the tile loop.
// The waves merge through LDS; a request's single workgroup writes its
// outputs, otherwise each workgroup's partial (max, sum, O) goes to its slot
// and the last workgroup of the (request, KV head) to arrive combines the
// slots in slot order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/decode_attention.h"
#include "common.h"
#include "layer_host.h"

namespace dl {
namespace {

constexpr int kAD = 128;                 // head size
constexpr int kATile = 256;              // cache positions per workgroup tile (64 per wave)
constexpr int kAMaxRows = 32;            // query rows per KV head (in row splits of 16 per workgroup)
constexpr int kAMaxSplit = 64;           // workgroups per (request, KV head, row split)
constexpr int kASlot = 16 * kAD + 2 * 16; // floats per partial: O [row][d], max, sum of 16 rows
constexpr int kAVRow = 72;               // LDS bytes per head-dim row of a wave's V^T slice (64 keys + pad)
constexpr int kAVWave = kAD * kAVRow;    // LDS bytes of one wave's V^T slice
constexpr int kAPoRow = 20;              // floats per head-dim row of a wave's merge area (16 rows + pad)
constexpr int kALds = (4 * kAVWave > (128 + 4 * kAD * kAPoRow) * 4) ? 4 * kAVWave : (128 + 4 * kAD * kAPoRow) * 4;
static_assert(2 * kAMaxSplit * 16 * 4 <= kALds, "combine weights");
constexpr unsigned kCoherent = 16;       // buffer cache policy: coherent at agent scope
constexpr int kASpecRequests = 4;        // at most this many requests: the first tile is loaded speculatively

typedef __bf16 bf16x8a __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2a __attribute__((ext_vector_type(2)));
typedef float f32x4a __attribute__((ext_vector_type(4)));
typedef float f32x2a __attribute__((ext_vector_type(2)));
typedef unsigned v4ua __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const int32_t *past_len;
  const uint16_t *q, *k_new, *v_new;
  uint8_t *k_cache, *v_cache;
  const float *k_scale, *v_scale;
  float *out;
  uint16_t *out_bf16;  // optional: out rounded to bf16, same element order
  float *slots;        // [max_requests * Hkv][n_split][kASlot]
  unsigned *counters;  // [max_requests * Hkv * row splits]
  int R, T, Hq, Hkv, C, max_past, grp, M, RS, tps, n_split;
  float softmax_scale;
  int spec;            // nonzero: the first tile is requested before the past length arrives
};

__device__ __forceinline__ f32x4a mfma16(const uint4 &a, const uint4 &b, f32x4a c) {
  v4ua ua = {a.x, a.y, a.z, a.w}, ub = {b.x, b.y, b.z, b.w};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8a, ua), __builtin_bit_cast(bf16x8a, ub),
                                                 c, 0, 0, 0);
}

// x (fp32) -> E4M3 code: nearest value, ties to the even code, magnitudes of
// 448 and above clamped to 448, the sign kept, NaN -> 0x7F.  Branch-free: at
// and above 2^-6 the fp32 pattern is rounded to 3 mantissa bits (to nearest,
// ties to even, a carry moving into the exponent) and the exponent rebiased
// from 127 to 7; below 2^-6 the codes are the multiples of 2^-9, a * 512
// rounded to the nearest integer, ties to even (exact scaling).
__device__ __forceinline__ unsigned e4m3_encode(float x) {
  const unsigned u = __float_as_uint(x), ua = u & 0x7FFFFFFFu;
  const float a = fabsf(x);
  const unsigned rn = ((ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20) - (120u << 3);
  const unsigned rs = (unsigned)rintf(a * 512.f);
  unsigned c = a < 0.015625f ? rs : rn;
  c = a >= 448.f ? 0x7Eu : c;
  c |= (u >> 24) & 0x80u;
  return a != a ? 0x7Fu : c;
}

// 8 bf16 values / scale (fp32 division) -> 8 E4M3 codes
__device__ __forceinline__ uint2 quant8(const uint16_t *src, float scale) {
  float f[8];
  unpack8(ld16(src), f);
  unsigned w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i >> 2] |= e4m3_encode(f[i] / scale) << (8 * (i & 3));
  return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ unsigned word(const uint4 &v, int c) {   // c: a compile-time constant after unrolling
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// 4 x 4 byte transpose: byte k of o[j] = byte j of a_k
__device__ __forceinline__ void transpose4(unsigned a0, unsigned a1, unsigned a2, unsigned a3, unsigned (&o)[4]) {
  // selector bytes 0..3 pick bytes of the second operand, 4..7 of the first
  const unsigned t01l = __builtin_amdgcn_perm(a1, a0, 0x05010400u), t01h = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
  const unsigned t23l = __builtin_amdgcn_perm(a3, a2, 0x05010400u), t23h = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
}

// 8 E4M3 codes -> 8 bf16 (exact: the hardware decodes OCP E4M3, scale 1)
template <bool HI>
__device__ __forceinline__ unsigned cvt2(unsigned w) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ uint4 fp8x8_bf16(unsigned a, unsigned b) {
  return make_uint4(cvt2<false>(a), cvt2<true>(a), cvt2<false>(b), cvt2<true>(b));
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

__device__ __forceinline__ float max4g(float v) {  // max over the 4 lanes n, n + 16, n + 32, n + 48
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float sum4g(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

__device__ __forceinline__ bool request_bad(const AttnArgs &a, int L) {
  return L < 0 || L > a.max_past || L + a.T > a.C;
}

// Key order inside a wave's 64-key slice of a tile.  The P V product takes
// 32 keys per matrix-core step q; lane group g4 supplies 8 of them, element
// jj.  With this order the scores a lane holds after S^T = K Q^T (keys
// 16 kt + 4 g4 + i of its query row) are exactly the P^T operand it supplies.
__device__ __forceinline__ int slice_key(int q, int g4, int jj) { return 32 * q + 16 * (jj >> 2) + 4 * g4 + (jj & 3); }

// PF: the next tile's loads are issued during this tile's softmax and P V
// (used when a workgroup takes more than one tile).
// One workgroup: tiles [tb, te) of one (request, KV head) and 16 of its query
// rows (row split rs), 4 waves each taking 64 keys of every tile with a
// softmax of their own; the waves merge at the end; the workgroup's partial
// goes to the output directly when it is the request's only one, else to its
// slot, and the last workgroup of the (request, KV head, row split) to arrive
// combines the slots.
// fp32 to bf16, rounded to nearest even (a NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const unsigned u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Four consecutive outputs at element index i (a multiple of 4), and their
// bf16 copy when asked for.
__device__ __forceinline__ void put_out4(const AttnArgs &a, size_t i, float4 v) {
  *reinterpret_cast<float4 *>(a.out + i) = v;
  if (a.out_bf16) {
    const unsigned lo = bf16_rne(v.x) | ((unsigned)bf16_rne(v.y) << 16);
    const unsigned hi = bf16_rne(v.z) | ((unsigned)bf16_rne(v.w) << 16);
    *reinterpret_cast<uint2 *>(a.out_bf16 + i) = make_uint2(lo, hi);
  }
}

template <bool PF>
__global__ void __launch_bounds__(256, 2) attn_step(AttnArgs a) {
  __shared__ __align__(16) uint8_t lds[kALds];         // V^T slices; later the wave merge and combine weights
  __shared__ __align__(16) uint8_t newc[2 * 8 * kAD];  // this step's K and V codes [K | V][token][d]
  __shared__ int s_last;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g4 = lane >> 4;
  const int s = blockIdx.x, rgs = blockIdx.y, rg = rgs / a.RS, rs = rgs % a.RS, r = rg / a.Hkv, g = rg % a.Hkv;
  const int L = a.past_len[r];
  const int M = a.M, grp = a.grp, T = a.T, row0 = 16 * rs;
  constexpr float kNegInf = -__builtin_inff();
  const size_t cbase = (size_t)rg * a.C * kAD;
  const int tb = s * a.tps;

  // ---- loads of one tile: this wave's 64 V rows (lane m = lane / 8 takes
  // the 8 keys of P V chunk m, 16 head-dim bytes 16 (lane % 8) ..) and its
  // K fragments (key 16 kt + n, head-dim bytes 64 h + 16 g4 ..), positions
  // clamped to pmax; none when the wave's keys all lie at or past pend.
  const int vm = lane >> 3, vdg = lane & 7;
  // plain locals: a lambda must not take the address of the kernel arguments
  const uint8_t *const kcache = a.k_cache, *const vcache = a.v_cache;
  uint4 vst[8], kr[4][2];
  auto load_tile = [&](int t, int pmax, int pend) __attribute__((always_inline)) {
    const int p0 = t * kATile + 64 * wv;
    if (p0 >= pend) return;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int p = min(p0 + slice_key(vm >> 2, vm & 3, k), pmax);
      vst[k] = ld16(vcache + cbase + (size_t)p * kAD + 16 * vdg);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const uint8_t *kp = kcache + cbase + (size_t)min(p0 + 16 * kt + n, pmax) * kAD + 16 * g4;
      kr[kt][0] = ld16(kp);
      kr[kt][1] = ld16(kp + 64);
    }
  };
  // With few requests the first tile is requested before the past length
  // arrives, its positions clamped to the cache's capacity (the step's own
  // positions and those past the end are replaced or masked below, as in
  // every tile); a split that then finds itself past its request's end has
  // read one tile for nothing.
  if (a.spec) load_tile(tb, a.C - 1, a.C);
  // query fragments: row row0 + n, head-dim elements in the K fragments' order
  uint4 qa[4];
  {
    const int row = min(row0 + n, M - 1), j = row / grp, h = g * grp + row % grp;
    const uint16_t *qp = a.q + ((size_t)(r * T + j) * a.Hq + h) * kAD + 16 * g4;
#pragma unroll
    for (int st = 0; st < 4; ++st) qa[st] = ld16(qp + 64 * (st >> 1) + 8 * (st & 1));
  }
  const float ksc = a.k_scale[g], vsc = a.v_scale[g];
  if (request_bad(a, L)) {
    // an impossible length: this request's outputs are NaN, nothing else runs
    if (s == 0)
      for (int q = tid; q < 16 * kAD; q += 256) {
        const int row = row0 + q / kAD, d = q % kAD, j = row / grp, h = g * grp + row % grp;
        if (row < M) {
          const size_t i = ((size_t)(r * T + j) * a.Hq + h) * kAD + d;
          a.out[i] = __builtin_nanf("");
          if (a.out_bf16) a.out_bf16[i] = 0x7fc0u;
        }
      }
    __builtin_amdgcn_s_waitcnt(0x0f70);                  // vmcnt(0): no load left in flight
    return;
  }
  const int len = L + T;                                 // positions after this step's tokens
  const int ntile = (len + kATile - 1) / kATile;
  if (tb >= ntile) {                                     // past this request's end: not counted
    __builtin_amdgcn_s_waitcnt(0x0f70);
    return;
  }
  const int te = min(tb + a.tps, ntile), nact = (ntile + a.tps - 1) / a.tps;
  const int lr = max(L - 1, 0);                          // cache reads stay below the step's own positions
  const size_t new_row0 = (size_t)r * T * a.Hkv + g;    // row (r, j, g) of k_new / v_new is new_row0 + j Hkv
  if (!a.spec) load_tile(tb, lr, len);
  // a wave's running state for row row0 + n: its maximum (the same in the 4
  // lane groups), its sum over the lane's own keys, O^T columns d = 16 dt + 4 g4 + i
  float am = kNegInf, al = 0.f;
  f32x4a ao[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) ao[dt] = f32x4a{0.f, 0.f, 0.f, 0.f};
  // ---- this step's own positions that fall in this workgroup's tiles: the
  // T new keys and values quantised once (x / scale in fp32, nearest E4M3
  // code) into LDS, where the tile loop takes them from, and written to the
  // cache by row split 0 of the workgroup, their only owner
  const int own0 = max(L, tb * kATile), own1 = min(len, te * kATile);
  if (own0 < own1) {                                     // workgroup-uniform
    for (int e = tid; e < 2 * T * 16; e += 256) {       // (K or V, token j, 8 head-dim elements)
      const int kind = e / (T * 16), j = (e >> 4) % T, part = e & 15;
      const uint16_t *src = (kind ? a.v_new : a.k_new) + (new_row0 + (size_t)j * a.Hkv) * kAD + 8 * part;
      const uint2 c = quant8(src, kind ? vsc : ksc);
      *reinterpret_cast<uint2 *>(newc + (kind * 8 + j) * kAD + 8 * part) = c;
      const int p = L + j;
      if (rs == 0 && p >= own0 && p < own1)
        *reinterpret_cast<uint2 *>((kind ? a.v_cache : a.k_cache) + cbase + (size_t)p * kAD + 8 * part) = c;
    }
    __syncthreads();
  }
  uint8_t *vsh = lds + wv * kAVWave;
  const float sc = a.softmax_scale * ksc * 1.44269504088896340736f;   // scores in log2 units
  const int lim = row0 + n < M ? L + (row0 + n) / grp : -1;           // this lane's row's last visible position

  for (int t = tb; t < te; ++t) {
    const int p0 = t * kATile + 64 * wv;
    const bool live = p0 < len;                          // wave-uniform
    f32x4a sa[4];
    if (live) {
      if (p0 + 64 > L) {                                 // wave-uniform: the slice holds new or past-the-end keys
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int p = p0 + slice_key(vm >> 2, vm & 3, k);
          // past the end: zero (their P is 0, but 0 * NaN is not); new: from LDS
          if (p >= len) vst[k] = make_uint4(0u, 0u, 0u, 0u);
          else if (p >= L) vst[k] = *reinterpret_cast<const uint4 *>(newc + (8 + p - L) * kAD + 16 * vdg);
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int p = p0 + 16 * kt + n;
          if (p >= L && p < len) {
            kr[kt][0] = *reinterpret_cast<const uint4 *>(newc + (p - L) * kAD + 16 * g4);
            kr[kt][1] = *reinterpret_cast<const uint4 *>(newc + (p - L) * kAD + 64 + 16 * g4);
          }
        }
      }
      // V^T into this wave's slice: head-dim row d holds the 64 keys in slice
      // order, chunk m (8 bytes) = the keys this lane loaded (the LDS queue of
      // a wave is in order, so the previous tile's reads are done)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        unsigned lo[4], hi[4];
        transpose4(word(vst[0], c), word(vst[1], c), word(vst[2], c), word(vst[3], c), lo);
        transpose4(word(vst[4], c), word(vst[5], c), word(vst[6], c), word(vst[7], c), hi);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2 *>(vsh + (16 * vdg + 4 * c + j) * kAVRow + 8 * vm) = make_uint2(lo[j], hi[j]);
      }
      // S^T = K Q^T: keys 16 kt + 4 g4 + i of query row row0 + n
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sa[kt] = f32x4a{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const uint4 &w = kr[kt][st >> 1];
          const uint4 kb = (st & 1) ? fp8x8_bf16(w.z, w.w) : fp8x8_bf16(w.x, w.y);
          sa[kt] = mfma16(kb, qa[st], sa[kt]);
        }
    }
    if (PF && t + 1 < te) load_tile(t + 1, lr, len);     // overlaps the softmax and P V below
    if (live) {
      uint4 ph[2], pl[2];
      float mt = kNegInf;
      if (p0 + 64 > L) {                                 // wave-uniform: only a tile holding a row's end masks
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = p0 + 16 * kt + 4 * g4 + i <= lim ? sa[kt][i] * sc : kNegInf;
            sa[kt][i] = v;
            mt = fmaxf(mt, v);
          }
      } else {
        const float rowv = lim >= 0 ? 1.f : 0.f;         // rows past M: every key masked
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = rowv != 0.f ? sa[kt][i] * sc : kNegInf;
            sa[kt][i] = v;
            mt = fmaxf(mt, v);
          }
      }
      mt = max4g(mt);
      const float mn = fmaxf(am, mt);
      const float ms = mn == kNegInf ? 0.f : mn;         // nothing visible yet: every p below is 0
      const float alpha = __builtin_amdgcn_exp2f(am - ms);   // 0 from -inf, 1 if unchanged
      am = mn;
      al *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) ao[dt] *= alpha;
      float x[2][8];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(sa[kt][i] - ms);   // masked: exp2(-inf) = 0
          al += p;
          x[kt >> 1][4 * (kt & 1) + i] = p;
        }
      split_hi_lo(x[0], ph[0], pl[0]);
      split_hi_lo(x[1], ph[1], pl[1]);
      // O^T += V^T P^T: head-dim rows 16 dt + n, chunk 4 q + g4 of the slice
      __builtin_amdgcn_s_waitcnt(0xc07f);                // lgkmcnt(0): this wave's V^T writes are done
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const uint2 c = *reinterpret_cast<const uint2 *>(vsh + (16 * dt + n) * kAVRow + 8 * (4 * q + g4));
          const uint4 va = fp8x8_bf16(c.x, c.y);
          ao[dt] = mfma16(va, ph[q], ao[dt]);
          ao[dt] = mfma16(va, pl[q], ao[dt]);
        }
    }
  }
  al = sum4g(al);

  // ---- merge the 4 waves: maxima and sums first; then each wave's O^T
  // scaled to the common maximum into its own area ([d][row], rows padded so
  // that neither the writes nor the reads below meet a bank conflict), added
  // in wave order by every thread
  float *st_m = reinterpret_cast<float *>(lds), *st_l = st_m + 64, *po = st_m + 128;
  __syncthreads();                                       // every wave is done with its V^T slice
  if (g4 == 0) {
    st_m[wv * 16 + n] = am;
    st_l[wv * 16 + n] = al;
  }
  __syncthreads();
  {
    float mr = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) mr = fmaxf(mr, st_m[w * 16 + n]);
    const float fw = __builtin_amdgcn_exp2f(am - (mr == kNegInf ? 0.f : mr));   // this wave's factor, 0 at -inf
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[(wv * kAD + 16 * dt + 4 * g4 + i) * kAPoRow + n] = ao[dt][i] * fw;
  }
  __syncthreads();
  // thread: row lrow = tid % 16 of the split, head-dim words d4 = tid / 16 + 16 k
  const int lrow = tid & 15, grow = row0 + lrow;
  float mr = kNegInf, lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) mr = fmaxf(mr, st_m[w * 16 + lrow]);
#pragma unroll
  for (int w = 0; w < 4; ++w) lsum += st_l[w * 16 + lrow] * __builtin_amdgcn_exp2f(st_m[w * 16 + lrow] - (mr == kNegInf ? 0.f : mr));
  f32x4a o2[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int d0 = 4 * ((tid >> 4) + 16 * k);
    o2[k] = f32x4a{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) o2[k][i] += po[(w * kAD + d0 + i) * kAPoRow + lrow];
  }
  const int gj = grow / grp, gh = g * grp + grow % grp;
  if (nact == 1) {
    // the request's only workgroup: outputs directly
    if (grow < M) {
      const float f = vsc / lsum;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        put_out4(a, ((size_t)(r * T + gj) * a.Hq + gh) * kAD + 4 * ((tid >> 4) + 16 * k),
                 make_float4(o2[k][0] * f, o2[k][1] * f, o2[k][2] * f, o2[k][3] * f));
    }
    return;
  }
  // this workgroup's partial to its slot, written through to the device coherence point
  {
    const __amdgpu_buffer_rsrc_t rs1 = __builtin_amdgcn_make_buffer_rsrc(
        a.slots + ((size_t)rgs * a.n_split + s) * kASlot, 0, kASlot * 4, 0x00020000);
    if (grow < M) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4ua, o2[k]), rs1,
                                               (lrow * kAD + 4 * ((tid >> 4) + 16 * k)) * 4, 0, kCoherent);
      if (tid < 16) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mr), rs1, (16 * kAD + lrow) * 4, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lsum), rs1, (16 * kAD + 16 + lrow) * 4, 0, kCoherent);
      }
    }
  }
  wt_stores_complete();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.counters + rgs, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)nact - 1u;
    if (s_last) __hip_atomic_store(a.counters + rgs, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the last workgroup of (request, KV head, row split): combine the nact
  // partials in slot order: per-row weights exp2(m_c - max) * v_scale / total
  // from every slot's max and sum, then outputs = sum_c weight_c * O_c.
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      a.slots + (size_t)rgs * a.n_split * kASlot, 0, a.n_split * kASlot * 4, 0x00020000);
  float *wm = reinterpret_cast<float *>(lds);
  // one round trip: as (row ar, lane aj) = (tid / 16, tid % 16) every thread
  // requests the maxima and sums of slots aj, aj + 16, ..., then its outputs'
  // words of the first 16 slots (clamped slots, used only when real; a thread
  // of a row past the step's rows gets an offset past the buffer's end, which
  // loads zero without a memory access); the weights are reduced over the 16
  // lanes of a row while the output words are in flight
  f32x4a v[2][16];
  const int obase = grow < M ? (lrow * kAD + 4 * (tid >> 4)) * 4 : 0x40000000;   // bytes; past the end for no row
  auto load_o = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < 16; ++cc)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = min(c0 + cc, nact - 1);
        v[k][cc] = __builtin_bit_cast(f32x4a, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rsb, obase + (c * kASlot + 64 * k) * 4, 0, kCoherent));
      }
  };
  {
    constexpr int kPer = kAMaxSplit / 16;
    const int ar = tid >> 4, aj = tid & 15;
    float mc[kPer], lc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int base = min(aj + 16 * i, nact - 1) * kASlot + 16 * kAD + ar;
      mc[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsb, base * 4, 0, kCoherent));
      lc[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsb, (base + 16) * 4, 0, kCoherent));
    }
    // the output words after them: the weights need only the maxima and sums
    __builtin_amdgcn_sched_barrier(0);
    load_o(0);
    __builtin_amdgcn_sched_barrier(0);
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (aj + 16 * i < nact) mx = fmaxf(mx, mc[i]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float f[kPer], tot = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      f[i] = aj + 16 * i < nact ? __builtin_amdgcn_exp2f(mc[i] - mx) : 0.f;   // 0 for a slot at -inf
      tot += f[i] * lc[i];
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) tot += __shfl_xor(tot, o);
    const float scl = vsc / tot;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (aj + 16 * i < nact) wm[(aj + 16 * i) * 16 + ar] = f[i] * scl;
  }
  __syncthreads();
  if (grow < M) {
    f32x4a o[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (int c0 = 0; c0 < nact; c0 += 16) {
      if (c0 > 0) load_o(c0);
#pragma unroll
      for (int cc = 0; cc < 16; ++cc)
        if (c0 + cc < nact)
#pragma unroll
          for (int k = 0; k < 2; ++k) o[k] += wm[(c0 + cc) * 16 + lrow] * v[k][cc];
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      put_out4(a, ((size_t)(r * T + gj) * a.Hq + gh) * kAD + 4 * ((tid >> 4) + 16 * k),
               make_float4(o[k][0], o[k][1], o[k][2], o[k][3]));
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
  if (c->max_requests < 1 || c->max_requests > 1024 ||
      (long)c->max_requests * c->n_kv_heads * ((c->n_q_heads / c->n_kv_heads * c->max_tokens + 15) / 16) > 65535)
    return fail(nullptr, DL_ERR_UNSUPPORTED,
                "max_requests=%d: need 1..1024 and max_requests * n_kv_heads * row splits <= 65535", c->max_requests);
  if (c->cache_len < 1 || c->cache_len > (1 << 20))
    return fail(nullptr, DL_ERR_UNSUPPORTED, "cache_len=%d: need 1..2^20", c->cache_len);
  if (!(c->softmax_scale > 0.f) || !std::isfinite(c->softmax_scale))
    return fail(nullptr, DL_ERR_UNSUPPORTED, "softmax_scale must be positive and finite");
  if (c->max_splits < 0) return fail(nullptr, DL_ERR_INVALID_ARG, "max_splits=%d is negative", c->max_splits);
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
  if (io->out_bf16 && (reinterpret_cast<uintptr_t>(io->out_bf16) & 7u))
    return fail(nullptr, DL_ERR_INVALID_ARG, "attention io.out_bf16 is not 8-byte aligned");
  return DL_OK;
}

int n_split_of(const decode_attention_config *c) {   // partial slots per (request, KV head)
  return std::min(kAMaxSplit, (c->cache_len + kATile - 1) / kATile);
}

int rs_of(const decode_attention_config *c) {   // row splits of 16 query rows at max_tokens
  return (c->n_q_heads / c->n_kv_heads * c->max_tokens + 15) / 16;
}

size_t slot_bytes(const decode_attention_config *c) {
  return (size_t)c->max_requests * c->n_kv_heads * rs_of(c) * n_split_of(c) * kASlot * 4;
}

int cus_of_current_device() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    n = std::max(1, host::cu_count(dev));
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace
}  // namespace dl

using namespace dl;

extern "C" {

size_t decode_attention_workspace_bytes(const decode_attention_config *cfg) {
  if (check_cfg(cfg) != DL_OK) return 0;
  return align256(slot_bytes(cfg)) + align256((size_t)cfg->max_requests * cfg->n_kv_heads * rs_of(cfg) * 4);
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
  a.out_bf16 = (uint16_t *)io->out_bf16;
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
  a.RS = (a.M + 15) / 16;
  a.n_split = n_split_of(cfg);
  a.softmax_scale = cfg->softmax_scale;
  // splits per (request, KV head, row split): about two workgroups per CU in
  // all, and at least two tiles of 256 positions per workgroup where the
  // context has them (every split pays the partial hand-off and adds a slot to
  // the combine, which one CU reads), at most n_split, each taking tps
  // consecutive tiles
  const int rg = a.R * a.Hkv * a.RS;
  const int tiles = (io->max_past + a.T + kATile - 1) / kATile;
  const int want = std::max(1, (2 * cus_of_current_device() + rg - 1) / rg);
  int split = std::min(std::min(std::min(tiles, a.n_split), want), std::max(1, (tiles + 1) / 2));
  if (cfg->max_splits > 0) split = std::min(split, cfg->max_splits);
  a.tps = (tiles + split - 1) / split;
  split = (tiles + a.tps - 1) / a.tps;
  // few requests: the step is latency-bound and splits past a short
  // request's end are few, so the first tile is worth requesting early
  a.spec = a.R <= kASpecRequests;
  const dim3 grid(split, rg);
  void (*kern)(AttnArgs) = a.tps > 1 ? attn_step<true> : attn_step<false>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return host::fail(nullptr, DL_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return DL_OK;
}

}  // extern "C"
