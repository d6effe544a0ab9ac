// Device helpers shared by the decode-layer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dl {

constexpr int kWave = 64;
constexpr int kBlock = 256;           // 4 waves per workgroup everywhere
constexpr int kWavesPerBlock = kBlock / kWave;

// ---- bf16 <-> fp32 (bf16 kept as raw 16-bit patterns) ---------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4 &w, float (&f)[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// ---- 16-byte global loads --------------------------------------------------
// Weights are streamed once per step: load them non-temporally so that they
// do not evict the small activation vectors every wave re-reads from L2.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
  v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld_stream16f(const void *p) {
  v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ float4 ld16f(const void *p) { return *reinterpret_cast<const float4 *>(p); }
// Four floats at float index i of buffer r, read at device scope (past the
// CU's and the XCD's caches): a value another XCD wrote through is seen even
// where this XCD still holds an earlier copy of the line.
__device__ __forceinline__ float4 ld16f_dev(__amdgpu_buffer_rsrc_t r, int i) {
  const v4f v = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, i * 4, 0, 16));
  return make_float4(v.x, v.y, v.z, v.w);
}

// ---- wave reductions -------------------------------------------------------
// DPP lane permutes inside rows of 16 lanes, then readlane across the 4 rows:
// VALU and scalar work only (no LDS-routed shuffle on the dependent chain).
// Every lane of a row adds the same two operands at each step (only their
// order differs, and fp addition is commutative), so all lanes agree bit for
// bit and the result does not depend on the lane.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each half-row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each row

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  v += dpp_mov<kDppMirror>(v);
  return v;
}

// Sum over the wave, returned (uniform) in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return (r0 + r1) + (r2 + r3);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64),
// returned in every lane of the group.
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 2) v += dpp_mov<kDppXor1>(v);
  if (width >= 4) v += dpp_mov<kDppXor2>(v);
  if (width >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if (width >= 16) v += dpp_mov<kDppMirror>(v);
  if (width >= 32) v += __shfl_xor(v, 16, kWave);
  if (width >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// ---- activation loaders: 8 consecutive values of token t as fp32 ----------
// Activations are small (one row per token) and re-read by many waves, so
// they use ordinary cached loads.
struct ActBf16 {          // bf16 [tokens][ld]
  const uint16_t *base;
  int ld;
  __device__ __forceinline__ void load8(int t, int k, float (&a)[8]) const {
    unpack8(ld16(base + (size_t)t * ld + k), a);
  }
};

struct ActF32 {           // fp32 [tokens][ld]
  const float *base;
  int ld;
  __device__ __forceinline__ void load8(int t, int k, float (&a)[8]) const {
    const float *p = base + (size_t)t * ld + k;
    float4 u = ld16f(p), v = ld16f(p + 4);
    a[0] = u.x; a[1] = u.y; a[2] = u.z; a[3] = u.w;
    a[4] = v.x; a[5] = v.y; a[6] = v.z; a[7] = v.w;
  }
};

// fp32 activations gathered through a token list (routed experts).
template <int NT>
struct ActF32Gather {
  const float *base;
  int ld;
  int tok[NT];
  __device__ __forceinline__ void load8(int t, int k, float (&a)[8]) const {
    const float *p = base + (size_t)tok[t] * ld + k;
    float4 u = ld16f(p), v = ld16f(p + 4);
    a[0] = u.x; a[1] = u.y; a[2] = u.z; a[3] = u.w;
    a[4] = v.x; a[5] = v.y; a[6] = v.z; a[7] = v.w;
  }
};

// ---- the skinny-GEMM inner loop ------------------------------------------
// acc[r][t] += sum over this lane's K positions of W_r[k] * act_t[k], for NR
// bf16 weight rows and NT tokens.  The lane visits k = k0, k0+kstride, ...
// (< K), 8 elements (16 bytes of weights) per visit; K, k0 and kstride are
// multiples of 8.  U visits are unrolled so that U*NR independent 16-byte
// weight loads are in flight before the first one is consumed.
template <int NR, int NT, int U, class Act>
__device__ __forceinline__ void stream_rows_bf16(const uint16_t *const (&w)[NR], const Act &act,
                                                 int k0, int kstride, int K, float (&acc)[NR][NT]) {
  int k = k0;
  for (; k + (U - 1) * kstride < K; k += U * kstride) {
    uint4 wv[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < NR; ++r) wv[u][r] = ld_stream16(w[r] + k + u * kstride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a[NT][8];
#pragma unroll
      for (int t = 0; t < NT; ++t) act.load8(t, k + u * kstride, a[t]);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float wf[8];
        unpack8(wv[u][r], wf);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][t] = fmaf(wf[e], a[t][e], acc[r][t]);
      }
    }
  }
  for (; k < K; k += kstride) {
    uint4 wv[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) wv[r] = ld_stream16(w[r] + k);
    float a[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t) act.load8(t, k, a[t]);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float wf[8];
      unpack8(wv[r], wf);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][t] = fmaf(wf[e], a[t][e], acc[r][t]);
    }
  }
}

__device__ __forceinline__ uint4 zero_unless(bool keep, const uint4 &v) {
  const unsigned m = keep ? 0xffffffffu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Loads are issued in batches and kept apart from the arithmetic that
// consumes them by a scheduling barrier: left to itself the compiler
// interleaves each load with its first use, which leaves one load in flight
// per wave.  A wave's loads complete in issue order, so a batch's first use
// waits only for the batch's first loads.
#define DL_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// ---- row GEMV building blocks -------------------------------------------------
// Activation sources for wave_rows_dot: raw() requests 8 consecutive values
// of token t at element k (no use yet), unpack() turns them into fp32.
struct ActBf16Rows {  // bf16 [tokens][ld], token index clamped to tmax
  const uint16_t *base;
  int ld, tmax;
  typedef uint4 Raw;
  __device__ __forceinline__ Raw raw(int t, int k) const {
    const int tt = t < tmax ? t : tmax;
    return ld16(base + (size_t)tt * ld + k);
  }
  __device__ __forceinline__ void unpack(const Raw &r, float (&v)[8]) const { unpack8(r, v); }
};

template <int NT>
struct HgGather {  // fp32 rows of a token list
  const float *base;
  int ld;
  int tok[NT];
  struct Raw { float4 a, b; };
  __device__ __forceinline__ Raw raw(int t, int k) const {
    const float *p = base + (size_t)tok[t] * ld + k;
    return Raw{ld16f(p), ld16f(p + 4)};
  }
  __device__ __forceinline__ void unpack(const Raw &r, float (&v)[8]) const {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
};

// One wave: dot products of NR bf16 weight rows (16-byte chunks [cbeg, cend)
// of each, i.e. elements [8 cbeg, 8 cend)) with NT activation rows.  Lane l
// takes chunks cbeg + l, cbeg + l + 64, ...; the weight and activation loads
// of CPB chunks are issued together (addresses clamped to the last chunk,
// weights of chunks beyond it zeroed afterwards), so a batch is one memory
// round trip.  The sums come back in every lane.
template <int NR, int NT, int CPB, class Act>
__device__ __forceinline__ void wave_rows_dot(const uint16_t *const (&w)[NR], int cbeg, int cend,
                                              const Act &act, float (&out)[NR][NT]) {
  const int lane = threadIdx.x & 63;
  float acc[NR][NT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
  for (int c0 = cbeg; c0 < cend; c0 += CPB * kWave) {
    uint4 wv[CPB][NR];
    typename Act::Raw ar[CPB][NT];
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int c = min(c0 + lane + kWave * u, cend - 1);
#pragma unroll
      for (int r = 0; r < NR; ++r) wv[u][r] = ld_stream16(w[r] + (size_t)c * 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) ar[u][t] = act.raw(t, c * 8);
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const bool on = c0 + lane + kWave * u < cend;
      float a[NT][8];
#pragma unroll
      for (int t = 0; t < NT; ++t) act.unpack(ar[u][t], a[t]);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float wf[8];
        unpack8(zero_unless(on, wv[u][r]), wf);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][t] = fmaf(wf[e], a[t][e], acc[r][t]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) out[r][t] = wave_sum(acc[r][t]);
}

// ---- wave top-k ---------------------------------------------------------------
// A float mapped to an unsigned word that orders like the float (-0 ranks as
// +0, the two compare equal); the result is at least 1, so that 0 can mark an
// absent or taken candidate.
__device__ __forceinline__ unsigned rank_bits(float v) {
  unsigned u = __float_as_uint(v == 0.f ? 0.f : v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return u > 1u ? u : 1u;
}
__device__ __forceinline__ float unrank_bits(unsigned u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned dpp_umax(unsigned v) {
  // Rows outside ROWS read 0, the identity of the maximum, so they keep v.
  // With 0 as the moved value's default the compiler folds the move into
  // the maximum (one v_max_u32 with a DPP source per step).
  const unsigned o = (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, ROWS == 0xf);
  return o > v ? o : v;
}
// Largest word over the wave; result uniform.
__device__ __forceinline__ unsigned wave_umax(unsigned v) {
  v = dpp_umax<kDppXor1, 0xf>(v);
  v = dpp_umax<kDppXor2, 0xf>(v);
  v = dpp_umax<kDppHalfMirror, 0xf>(v);
  v = dpp_umax<kDppMirror, 0xf>(v);  // rows of 16 uniform
  v = dpp_umax<0x142, 0xa>(v);       // row_bcast:15 -> rows 1, 3
  v = dpp_umax<0x143, 0xc>(v);       // row_bcast:31 -> rows 2, 3
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k over one wave.  Lane l offers the candidates e = l + 64 c (c < NC,
// e < E) with values lv[c]; lane j < K receives the j-th pick in the order
// "larger value first, then smaller index".  The picks are K distinct
// indices below E whatever the values (a NaN ranks above +inf).  Needs K <= E.
// Each round takes the wave maximum of the 32-bit value keys; the lowest
// index holding that key is found through a ballot (a second maximum, over
// inverted indices, only when several lanes hold it).
template <int NC>
__device__ __forceinline__ void wave_topk(const float (&lv)[NC], int E, int K, int &my_idx, float &my_v) {
  const int lane = threadIdx.x & 63;
  unsigned key[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) key[c] = lane + 64 * c < E ? rank_bits(lv[c]) : 0u;
  int mine_idx = 0;
  unsigned mine_key = 1u;
  for (int j = 0; j < K; ++j) {
    unsigned m = key[0];
#pragma unroll
    for (int c = 1; c < NC; ++c) m = key[c] > m ? key[c] : m;
    const unsigned g = wave_umax(m);
    // this lane's lowest index holding g, as 0xffffffff - index (0: none)
    unsigned inv = 0u;
#pragma unroll
    for (int c = NC - 1; c >= 0; --c) inv = key[c] == g ? 0xffffffffu - (unsigned)(lane + 64 * c) : inv;
    const unsigned long long holders = __ballot(inv != 0u);
    unsigned best;
    if (__popcll(holders) == 1)
      best = (unsigned)__builtin_amdgcn_readlane((int)inv, __ffsll((long long)holders) - 1);
    else
      best = wave_umax(inv);
    const int id = (int)(0xffffffffu - best);
#pragma unroll
    for (int c = 0; c < NC; ++c) key[c] = id == lane + 64 * c ? 0u : key[c];
    if (lane == j) {
      mine_idx = id;
      mine_key = g;
    }
  }
  my_idx = mine_idx;
  my_v = unrank_bits(mine_key);
}

// Top-k over one wave whose candidates are numbered in lane order: lane l
// holds key[c] for candidate base + 64 c + l (keys from rank_bits, 0 for an
// absent or taken candidate).  Lane j < K receives the key and the number of
// the j-th pick, "larger key first, then smaller number".  Each round takes
// the wave maximum g of the lanes' largest keys; the smallest number holding
// g is the lowest lane of the first block c whose ballot of key[c] == g is
// not empty, so equal keys need no second reduction.  Once every present key
// is taken a round picks a key of 0 (never returned when K does not exceed
// the number of present candidates).
template <int NC>
__device__ __forceinline__ void wave_topk_blocks(unsigned (&key)[NC], int base, int K, unsigned &pick_key,
                                                 int &pick_idx) {
  const int lane = threadIdx.x & 63;
  pick_key = 0u;
  pick_idx = 0;
  for (int j = 0; j < K; ++j) {
    unsigned m = key[0];
#pragma unroll
    for (int c = 1; c < NC; ++c) m = key[c] > m ? key[c] : m;
    const unsigned g = wave_umax(m);
    unsigned long long hold = 0;
    int cs = 0;
#pragma unroll
    for (int c = NC - 1; c >= 0; --c) {
      const unsigned long long b = __ballot(key[c] == g);
      if (b) {
        hold = b;
        cs = c;
      }
    }
    const int p = __ffsll((long long)hold) - 1;
    if (lane == j) {
      pick_key = g;
      pick_idx = base + 64 * cs + p;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (c == cs && lane == p) key[c] = 0u;
  }
}

// Merge of candidate lists over one wave: lane l holds key and number of
// candidate l, where among equal keys a lower lane always has the smaller
// number (for instance, the concatenated pick lists of wave_topk_blocks over
// consecutive ranges).  Lane j < K receives the j-th pick in the same order.
__device__ __forceinline__ void wave_topk_merge(unsigned key, int idx, int K, unsigned &pick_key, int &pick_idx) {
  const int lane = threadIdx.x & 63;
  pick_key = 0u;
  pick_idx = 0;
  for (int j = 0; j < K; ++j) {
    const unsigned g = wave_umax(key);
    const int p = __ffsll((long long)__ballot(key == g)) - 1;
    const int id = __builtin_amdgcn_readlane(idx, p);
    if (lane == j) {
      pick_key = g;
      pick_idx = id;
    }
    if (lane == p) key = 0u;
  }
}

__device__ __forceinline__ float silu_mul(float u, float v) { return u / (1.0f + expf(-u)) * v; }

// Renormalised sigmoid weights of the k picks of one token, over one wave:
// lane j < K holds the logit l_j of pick j (lane 0 the largest).  Returns, in
// lane j < K, w_j = s_j / sum_i s_i with s = sigmoid(l), evaluated as
// exp(ls_j - ls_0) / sum_i exp(ls_i - ls_0) with ls = log sigmoid(l)
// = min(l, 0) - log1p(exp(-|l|)): the same value, but finite for logits whose
// sigmoid underflows fp32 (below about -87), where s_j / sum s would be 0/0.
// Every term of the sum lies in (0, 1] and the first is 1.
__device__ __forceinline__ float pick_weights(float l, int K) {
  const int lane = threadIdx.x & 63;
  const float ls = fminf(l, 0.f) - log1pf(expf(-fabsf(l)));
  const float ls0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(ls)));
  const float r = lane < K ? expf(ls - ls0) : 0.f;
  return r / wave_sum(r);
}

// ---- cross-workgroup hand-off ------------------------------------------------
// Waits until every memory operation this wave has issued has completed; for
// stores written through to the device's coherence point (agent-scope atomic
// stores, or buffer stores with the write-through bit), completion means the
// value is visible to every other workgroup of the device.  The signal fences
// keep the compiler from moving memory operations across the wait.
__device__ __forceinline__ void wt_stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Every workgroup of a phase publishes its partial results, then counts
// itself in `counter`; the workgroup that arrives last sees every other
// workgroup's results.  Release (before the count) and acquire (after it)
// are at agent scope, which on a multi-XCD part also writes back / invalidates
// the per-XCD L2 as needed.  Nothing produced by another workgroup is read
// before the acquire; only static weights may be loaded earlier.
// Returns true in every thread of the last workgroup.  The last workgroup
// re-arms the counter for the next step.
__device__ __forceinline__ bool arrive_last(unsigned *counter, unsigned nblocks, int *lds_flag) {
  __threadfence();          // release this thread's stores at agent scope
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = (prev == nblocks - 1) ? 1 : 0;
  }
  __syncthreads();
  bool last = *lds_flag != 0;
  if (last) {
    __threadfence();        // acquire for every thread of the last workgroup
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return last;
}

// The same hand-off without cache-wide fences: the caller has written the
// values it hands over with agent-scope atomic stores (written through to
// the device's coherence point), and the last workgroup reads them back with
// agent-scope atomic loads.  Each thread's stores have completed before the
// workgroup is counted.  An agent-scope fence would instead write back and
// invalidate the whole L2 of the XCD, once per workgroup.
__device__ __forceinline__ bool arrive_last_wt(unsigned *counter, unsigned nblocks, int *lds_flag) {
  wt_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = prev == nblocks - 1;
    if (*lds_flag) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *lds_flag != 0;
}

}  // namespace dl
