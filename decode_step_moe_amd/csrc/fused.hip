// The whole layer-step as ONE persistent launch, for small batches.
//
// A decode step at one to a few tokens moves 75-360 MB of weights through a
// chain of dependent reductions (RMSNorm needs all of r1, top-k needs every
// router logit, the down projection needs every SwiGLU activation of an
// expert).  As separate kernels each dependency costs a launch boundary and a
// ramp of the HBM pipe.  The pages' decode backend attacks the same problem by
// fusing the per-layer kernels and overlapping the shared expert and a weight
// prefetch with the dependent work (wireai.ir "vLLM's speed jump on NVIDIA
// Blackwell servers; record 842 tokens/s for Kimi K3", sections "Compressing
// the decode loop by kernel fusion" and "Four key changes behind the jump",
// bullets 1-4).  Here the grid is one workgroup per CU, all resident at once,
// and the dependencies are hand-offs between phases of the same kernel.
//
// Workgroup w owns the H-slice S_w = [w*slice, (w+1)*slice) of the hidden
// dimension, router rows e = w and w + G, and shared-expert ffn row f = w.
// Phases:
//
//  A  out-projection rows i in S_w:  r1 = r + attn Wo^T     -> resid_out
//     hg = g * r1 (global and LDS); per-token partial sum of r1^2 over S_w
//     -> published.  Then the workgroup's router rows and shared-expert
//     gate/up rows (static weights) are requested into registers.
//  B  1/rms(t) from the G partial sums (every workgroup, identical order);
//     h = hg / rms is read back from global memory and
//     l[t, e] = h[t] . Wr[e]                          -> published
//     a_s[t, f] = silu(S1[f] . h[t]) * (S3[f] . h[t])  -> published
//  C  every workgroup reads all logits and takes the same top-k decision
//     (descending logit, ties to the lower expert id; s = sigmoid(l),
//     w = s / sum s over the k picks), builds the same per-expert token lists
//     in LDS, then computes its share of the routed gate/up rows:
//     a[p, f] = silu(W1[e, f] . h[t_p]) * (W3[e, f] . h[t_p])
//     for every (expert e, token t_p) pair p -> published.
//  D  y[t, i] for i in S_w:  sum_f S2[i, f] a_s[t, f]
//                           + sum over the k picks of t, in pick order, of
//                             w_p sum_f W2[e_p, i, f] a[p, f].
//     Each y element is produced by one thread in a fixed order.  The first
//     down-projection weights are requested before waiting for a.
//     Last, the attention input projection rows qkv[t, j] = x[t] . Wqkv[j] of
//     this workgroup's share of j (independent of everything else; placed at
//     the end so that its traffic never queues in front of a hand-off).
//
// Hand-offs.  Values produced by one workgroup for another (partial sums,
// logits, SwiGLU activations) are written as 64-bit pairs (value, tag) with
// device-scope relaxed atomic stores, and read by polling with device-scope
// relaxed atomic loads until the tag equals this step's tag: a consumer waits
// exactly for the data it needs, with one memory round trip and no counter
// that every workgroup would have to serialise on.  The tag is the handle's
// step counter + 1, kept in device memory and advanced by workgroup 0 at the
// end of each step, so it is also right under HIP-graph replay.  hg and the
// outputs are ordinary stores; hg is released (agent-scope fence) before the
// phase-A hand-off values and acquired after them.  Only static weights are
// read before a wait (the ordering rule of wireai.ir, "Oversight and
// validation for AI-generated kernels").  Every wait is bounded: on expiry the
// kernel records an error in the handle's status word and runs to completion.
//
// Wave-wide reductions on the serial parts (top-k, lists) use DPP lane
// permutes and readlane rather than LDS-routed shuffles.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dl {

namespace {

constexpr int kFT = kFusedThreads;          // 512 threads, 8 waves
constexpr int kFWaves = kFT / kWave;
constexpr int kRtrJ = kFusedMaxH / 4 / kFT; // float4 chunks per thread per router row (4)
constexpr int kShJ = kFusedMaxH / 8 / kFT;  // 16-byte bf16 chunks per thread per shared row (2)

// ---- tagged hand-off values -------------------------------------------------
__device__ __forceinline__ void put_tagged(uint64_t *p, float v, unsigned tag) {
  uint64_t x = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Completes a poll started with ld_tagged(p) -> x: re-reads until the tag
// matches or the spin budget is spent (then *bad is set).
__device__ __forceinline__ float finish_tagged(const uint64_t *p, uint64_t x, unsigned tag, int limit,
                                               int *bad) {
  int n = 0;
  while ((unsigned)(x >> 32) != tag) {
    if (++n > limit) {
      *bad = 1;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    x = ld_tagged(p);
  }
  return __uint_as_float((unsigned)x);
}

// ---- DPP wave arg-max ---------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ void amax(float &v, int &i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}
// Largest value over the wave, ties to the lower index; result uniform.
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
  amax(v, i, dpp_f<0xB1>(v), dpp_i<0xB1>(i));    // quad_perm [1,0,3,2]
  amax(v, i, dpp_f<0x4E>(v), dpp_i<0x4E>(i));    // quad_perm [2,3,0,1]
  amax(v, i, dpp_f<0x141>(v), dpp_i<0x141>(i));  // row_half_mirror
  amax(v, i, dpp_f<0x140>(v), dpp_i<0x140>(i));  // row_mirror: rows of 16 uniform
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  int bi = __builtin_amdgcn_readlane(i, 15);
#pragma unroll
  for (int r = 1; r < 4; ++r)
    amax(bv, bi, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r + 15)),
         __builtin_amdgcn_readlane(i, 16 * r + 15));
  v = bv;
  i = bi;
}

// ---- activations ------------------------------------------------------------
struct ActBf16Rows {  // bf16 [tokens][ld], token index clamped to tmax
  const uint16_t *base;
  int ld, tmax;
  __device__ __forceinline__ void load8(int t, int k, float (&v)[8]) const {
    int tt = t < tmax ? t : tmax;
    unpack8(ld16(base + (size_t)tt * ld + k), v);
  }
};

template <int NT>
struct HgGather {  // fp32 hg rows of a token list
  const float *base;
  int ld;
  int tok[NT];
  __device__ __forceinline__ void load8(int t, int k, float (&v)[8]) const {
    const float *p = base + (size_t)tok[t] * ld + k;
    float4 u = ld16f(p), w = ld16f(p + 4);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    v[4] = w.x; v[5] = w.y; v[6] = w.z; v[7] = w.w;
  }
};

// One wave: dot products of NR bf16 weight rows (16-byte chunks [cbeg, cend)
// of each, i.e. elements [8 cbeg, 8 cend)) with NT activation rows.  Lane l
// takes chunks cbeg + l, cbeg + l + 64, ...; up to CPB chunks of every row are
// loaded before any is consumed.  The sums come back in every lane.
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
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int c = c0 + lane + kWave * u;
#pragma unroll
      for (int r = 0; r < NR; ++r) wv[u][r] = c < cend ? ld_stream16(w[r] + (size_t)c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int c = c0 + lane + kWave * u;
      if (c < cend) {
        float a[NT][8];
#pragma unroll
        for (int t = 0; t < NT; ++t) act.load8(t, c * 8, a[t]);
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
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) out[r][t] = wave_sum(acc[r][t]);
}

__device__ __forceinline__ float silu_mul(float u, float v) { return u / (1.0f + expf(-u)) * v; }

__device__ __forceinline__ float dot4(const float4 &a, const float4 &b, float s) {
  s = fmaf(a.x, b.x, s);
  s = fmaf(a.y, b.y, s);
  s = fmaf(a.z, b.z, s);
  return fmaf(a.w, b.w, s);
}

// Phase trace (measurement only): thread 0 stamps the device wall clock.
__device__ __forceinline__ void stamp(const FusedArgs &a, int point) {
  if (a.trace && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * kTracePoints + point] = wall_clock64();
}

struct Lds {
  float hg[kFusedMaxB][kFusedMaxSlice];
  float sq[kFusedMaxB][kFusedMaxSlice];
  float red[kFWaves * 4 * kFusedMaxB];
  float inv_rms[kFusedMaxB];
  // logits for top-k, later the routed SwiGLU activations [pair][F]
  float big[kFusedBig];
  float act_s[kFusedActS];
  // top-k and lists
  int sel[kFusedMaxPairs];
  float selw[kFusedMaxPairs];
  int pos[kFusedMaxPairs];
  int act_exp[kFusedMaxPairs];
  int act_cnt[kFusedMaxPairs];
  int act_off[kFusedMaxPairs];
  int pair_tok[kFusedMaxPairs];
  int pair_exp[kFusedMaxPairs];
  float pair_w[kFusedMaxPairs];
  int n_active;
  // gate/up partials: [wave][token]
  float uv[kFWaves][kFusedMaxB];
  // phase D contributions: [item = shared token t | B + pair p][row in slice]
  float contrib[(kFusedMaxB + kFusedMaxPairs) * kFusedMaxSlice];
  int bad;
};

// ---- phase A: out-projection rows of the slice ------------------------------
template <int NT>
__device__ void oproj_rows(const FusedArgs &a, Lds &L, int i0, int ni) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int B = a.B;
  const ActBf16Rows act{a.attn, a.Do, B - 1};
  const int nch = a.Do >> 3;
  // up to kFusedMaxSlice / 8 = 4 rows per wave, all issued together; the
  // residual and gain of lane t's (row, token t) are requested up front too
  const uint16_t *rows[4];
  int il[4];
  float res[4], gn[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    il[r] = wv + kFWaves * r;
    const int i = i0 + min(il[r], ni - 1);
    rows[r] = a.w_o + (size_t)i * a.Do;
    const bool mine = lane < B && il[r] < ni;
    res[r] = mine ? a.resid_in[(size_t)lane * a.H + i] : 0.f;
    gn[r] = mine ? bf16_lo(a.gain[i]) : 0.f;
  }
  float o[4][NT];
  wave_rows_dot<4, NT, 2>(rows, 0, nch, act, o);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float mine = 0.f;  // lane t keeps token t's sum
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (lane == t) mine = o[r][t];
    if (lane < B && il[r] < ni) {
      const int i = i0 + il[r];
      const size_t ix = (size_t)lane * a.H + i;
      const float r1 = res[r] + mine;
      a.resid_out[ix] = r1;
      const float hgv = gn[r] * r1;
      a.hg[ix] = hgv;
      L.hg[lane][il[r]] = hgv;
      L.sq[lane][il[r]] = r1 * r1;
    }
  }
}

// 16-byte weight chunks per lane in flight per row, by token count
template <int NT>
constexpr int cpb_for() { return NT <= 2 ? 16 : NT <= 4 ? 8 : 4; }

template <int NT>
__device__ void qkv_rows(const FusedArgs &a, int j0, int nj) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const ActBf16Rows act{a.x, a.H, a.B - 1};
  const int nch = a.H >> 3;
  for (int jl = wv; jl < nj; jl += kFWaves) {
    const uint16_t *row[1] = {a.w_qkv + (size_t)(j0 + jl) * a.H};
    float s[1][NT];
    wave_rows_dot<1, NT, cpb_for<NT>()>(row, 0, nch, act, s);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (lane == t && t < a.B) a.qkv[(size_t)t * a.Dq + j0 + jl] = s[0][t];
  }
}

// ---- phase C: routed gate/up, one (expert, ffn row) pair per two waves ------
template <int NT>
__device__ void routed_gateup_row(const FusedArgs &a, Lds &L, int slot, int f) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = L.act_exp[slot], cnt = L.act_cnt[slot], off = L.act_off[slot];
  HgGather<NT> act;
  act.base = a.hg;
  act.ld = a.H;
#pragma unroll
  for (int t = 0; t < NT; ++t) act.tok[t] = L.pair_tok[off + (t < cnt ? t : cnt - 1)];
  const uint16_t *row[1] = {((wv & 1) ? a.w3 : a.w1) + ((size_t)e * a.F + f) * a.H};
  float s[1][NT];
  wave_rows_dot<1, NT, cpb_for<NT>()>(row, 0, a.H >> 3, act, s);
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (lane == t) L.uv[wv][t] = s[0][t];
}

// ---- phase D: one (item, row) unit per group of LPG lanes --------------------
// Items 0..B-1 are the shared expert's tokens (weights S2, activations
// act_s), items B..B+P-1 the routed pairs (weights W2 of the pair's expert,
// activations act, scaled by the pair's weight); F = 8 * LPG for both.
// Without a shared expert the items start at B.
template <int LPG>
struct Down {
  static constexpr int NG = kFT / LPG;  // lane groups
  static constexpr int R = 8;           // units per group whose weights are in flight together
  const FusedArgs &a;
  Lds &L;
  int i0, ni, item0, n_units;
  __device__ void issue(int round, uint4 (&wv)[R]) const {
    const int g = threadIdx.x / LPG, lg = threadIdx.x % LPG;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int u = g + NG * (round * R + r);
      wv[r] = make_uint4(0, 0, 0, 0);
      if (u < n_units) {
        const int item = item0 + u / ni, il = u % ni;
        const uint16_t *row = item < a.B ? a.s2 + (size_t)(i0 + il) * a.F
                                         : a.w2 + ((size_t)L.pair_exp[item - a.B] * a.H + i0 + il) * a.F;
        wv[r] = ld_stream16(row + lg * 8);
      }
    }
  }
  __device__ void consume(int round, const uint4 (&wv)[R]) const {
    const int g = threadIdx.x / LPG, lg = threadIdx.x % LPG;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int u = g + NG * (round * R + r);
      if (u < n_units) {
        const int item = item0 + u / ni, il = u % ni;
        const float *ap = item < a.B ? L.act_s + item * a.F + lg * 8 : L.big + (item - a.B) * a.F + lg * 8;
        float wf[8];
        unpack8(wv[r], wf);
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) s = fmaf(wf[q], ap[q], s);
        s = group_sum(s, LPG);
        if (lg == 0) L.contrib[item * kFusedMaxSlice + il] = item < a.B ? s : s * L.pair_w[item - a.B];
      }
    }
  }
  __device__ int rounds() const { return (n_units + NG * R - 1) / (NG * R); }
};

template <class Fn>
__device__ __forceinline__ void by_tokens(int n, Fn fn) {
  if (n <= 1) fn(std::integral_constant<int, 1>{});
  else if (n <= 2) fn(std::integral_constant<int, 2>{});
  else if (n <= 4) fn(std::integral_constant<int, 4>{});
  else fn(std::integral_constant<int, 8>{});
}

template <class Fn>
__device__ __forceinline__ void by_lpg(int F, Fn fn) {
  switch (F) {
    case 32: fn(std::integral_constant<int, 4>{}); break;
    case 64: fn(std::integral_constant<int, 8>{}); break;
    case 128: fn(std::integral_constant<int, 16>{}); break;
    default: fn(std::integral_constant<int, 32>{}); break;
  }
}

}  // namespace

__global__ void __launch_bounds__(kFT, 1) fused_step_kernel(FusedArgs a) {
  __shared__ Lds L;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int w = blockIdx.x, G = gridDim.x;
  const int B = a.B, E = a.E, K = a.K, H = a.H;
  const unsigned epoch = *a.epoch;
  if (epoch == 0xffffffffu) {  // tag space exhausted: refuse (status 2)
    if (w == 0 && tid == 0) atomicOr(a.status, 2u);
    return;
  }
  const unsigned tag = epoch + 1;
  if (tid == 0) L.bad = 0;
  const int i0 = w * a.slice;
  const int ni = max(0, min(a.slice, H - i0));
  stamp(a, 0);

  // ================= phase A =================
  if (ni > 0) by_tokens(B, [&](auto nt) { oproj_rows<decltype(nt)::value>(a, L, i0, ni); });
  __syncthreads();
  stamp(a, 1);
  // release hg (ordinary stores) before the hand-off values that announce it
  if (tid == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid < B) {
    float s = 0.f;
    for (int il = 0; il < ni; ++il) s += L.sq[tid][il];
    put_tagged(a.pss + (size_t)w * B + tid, s, tag);
  }
  // static weights for phase B, requested now: router rows e0 = w, e1 = w + G
  // (fp32, float4 chunk c = tid + kFT*j of H/4) and shared gate/up row f = w
  // (bf16, 16-byte chunk c = tid + kFT*j of H/8)
  const int e0 = w, e1 = w + G;
  const bool has_e0 = e0 < E, has_e1 = e1 < E, has_f = w < a.Fs;
  float4 rt[2][kRtrJ];
  uint4 sh[2][kShJ];
#pragma unroll
  for (int j = 0; j < kRtrJ; ++j) {
    const int c = tid + kFT * j;
    const bool in = c < (H >> 2);
    rt[0][j] = has_e0 && in ? ld_stream16f(a.w_router + (size_t)e0 * H + 4 * c) : make_float4(0, 0, 0, 0);
    rt[1][j] = has_e1 && in ? ld_stream16f(a.w_router + (size_t)e1 * H + 4 * c) : make_float4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kShJ; ++j) {
    const int c = tid + kFT * j;
    const bool in = has_f && c < (H >> 3);
    sh[0][j] = in ? ld_stream16(a.s1 + (size_t)w * H + 8 * c) : make_uint4(0, 0, 0, 0);
    sh[1][j] = in ? ld_stream16(a.s3 + (size_t)w * H + 8 * c) : make_uint4(0, 0, 0, 0);
  }
  stamp(a, 2);

  // ================= phase B =================
  {
    // poll all G partial sums of every token at once, then reduce per token
    uint64_t x[kFusedMaxB];
#pragma unroll
    for (int t = 0; t < kFusedMaxB; ++t)
      if (tid < G && t < B) x[t] = ld_tagged(a.pss + (size_t)tid * B + t);
#pragma unroll
    for (int t = 0; t < kFusedMaxB; ++t) {
      if (t < B) {
        float v = tid < G ? finish_tagged(a.pss + (size_t)tid * B + t, x[t], tag, a.spin_limit, &L.bad) : 0.f;
        v = wave_sum(v);
        if (lane == 0) L.red[wv * kFusedMaxB + t] = v;
      }
    }
    __syncthreads();
    if (tid < B) {
      float s = 0.f;
      for (int q = 0; q < kFWaves; ++q) s += L.red[q * kFusedMaxB + tid];
      L.inv_rms[tid] = 1.0f / sqrtf(s / (float)H + a.eps);
    }
    __syncthreads();
  }
  // every workgroup's hg is now announced: acquire before reading it
  if (tid == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  stamp(a, 4);
  if (a.h_out && ni > 0)
    for (int q = tid; q < B * ni; q += kFT) {
      const int t = q / ni, il = q % ni;
      a.h_out[(size_t)t * H + i0 + il] = L.hg[t][il] * L.inv_rms[t];
    }
  if (has_e0 || has_f) {  // uniform over the workgroup
    // per token: this thread's partial dots [router row 0, row 1, S1, S3],
    // wave-reduced, then the 8 wave totals summed in order
    for (int t = 0; t < B; ++t) {
      const float *hrow = a.hg + (size_t)t * H;
      float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
      for (int j = 0; j < kRtrJ; ++j) {
        const int c = tid + kFT * j;
        if (c < (H >> 2)) {
          const float4 hv = ld16f(hrow + 4 * c);
          p0 = dot4(rt[0][j], hv, p0);
          p1 = dot4(rt[1][j], hv, p1);
        }
      }
#pragma unroll
      for (int j = 0; j < kShJ; ++j) {
        const int c = tid + kFT * j;
        if (has_f && c < (H >> 3)) {
          const float4 h0 = ld16f(hrow + 8 * c), h1 = ld16f(hrow + 8 * c + 4);
          const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
          float w1f[8], w3f[8];
          unpack8(sh[0][j], w1f);
          unpack8(sh[1][j], w3f);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            p2 = fmaf(w1f[q], hv[q], p2);
            p3 = fmaf(w3f[q], hv[q], p3);
          }
        }
      }
      p0 = wave_sum(p0);
      p1 = wave_sum(p1);
      p2 = wave_sum(p2);
      p3 = wave_sum(p3);
      if (lane == 0) {
        float *r = L.red + (wv * kFusedMaxB + t) * 4;
        r[0] = p0; r[1] = p1; r[2] = p2; r[3] = p3;
      }
    }
    __syncthreads();
    if (tid < B) {
      float q4[4] = {0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < kFWaves; ++q)
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) q4[k2] += L.red[(q * kFusedMaxB + tid) * 4 + k2];
      const float inv = L.inv_rms[tid];
      if (has_e0) {
        const float l = q4[0] * inv;
        put_tagged(a.logit + (size_t)tid * E + e0, l, tag);
        if (a.logits_out) a.logits_out[(size_t)tid * E + e0] = l;
      }
      if (has_e1) {
        const float l = q4[1] * inv;
        put_tagged(a.logit + (size_t)tid * E + e1, l, tag);
        if (a.logits_out) a.logits_out[(size_t)tid * E + e1] = l;
      }
      if (has_f) put_tagged(a.act_s + (size_t)tid * a.Fs + w, silu_mul(q4[2] * inv, q4[3] * inv), tag);
    }
  }
  stamp(a, 5);

  // ================= phase C =================
  {
    const int n = B * E;
    constexpr int PER = kFusedBig / kFT;
    uint64_t x[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int q = tid + r * kFT;
      if (q < n) x[r] = ld_tagged(a.logit + q);
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int q = tid + r * kFT;
      if (q < n) L.big[q] = finish_tagged(a.logit + q, x[r], tag, a.spin_limit, &L.bad);
    }
  }
  __syncthreads();
  stamp(a, 7);
  // top-k per token, one wave per token: lane l holds experts l, l+64, ...
  for (int t = wv; t < B; t += kFWaves) {
    constexpr int NC = kFusedMaxE / 64;
    float lv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = lane + 64 * c;
      lv[c] = e < E ? L.big[t * E + e] : -INFINITY;
    }
    int my_idx = 0;
    float my_s = 0.f, ssum = 0.f;
    for (int j = 0; j < K; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (lv[c] > bv) { bv = lv[c]; bi = lane + 64 * c; }   // c ascending: ties keep the lower id
      wave_argmax(bv, bi);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (bi == lane + 64 * c) lv[c] = -INFINITY;
      const float s = 1.0f / (1.0f + expf(-bv));
      ssum += s;
      if (lane == j) { my_idx = bi; my_s = s; }
    }
    if (lane < K) {
      const float wgt = my_s / ssum;
      L.sel[t * K + lane] = my_idx;
      L.selw[t * K + lane] = wgt;
      if (w == 0) {
        a.topk_idx[(size_t)t * K + lane] = my_idx;
        a.topk_w[(size_t)t * K + lane] = wgt;
      }
    }
  }
  __syncthreads();
  stamp(a, 13);
  // per-expert lists, one wave: lane p = pick (t, r) = t*K + r.  Pairs are
  // ordered by (expert, token); active experts ascending.
  if (wv == 0) {
    const int P = B * K;
    const int e_p = lane < P ? L.sel[lane] : 0x7fff;
    const int key = lane < P ? e_p * 64 + lane / K : 0x7fffffff;
    int rank = 0, before = 0, same = 0;
    for (int q = 0; q < P; ++q) {
      const int kq = __builtin_amdgcn_readlane(key, q);
      const int eq = kq >> 6;
      rank += kq < key;
      before += (eq == e_p) && kq < key;
      same += eq == e_p;
    }
    const bool first = lane < P && before == 0;
    const unsigned long long fm = __ballot(first);
    int slot = 0;
    for (int q = 0; q < P; ++q)
      if ((fm >> q) & 1ull) slot += __builtin_amdgcn_readlane(e_p, q) < e_p;
    if (lane < P) {
      L.pair_tok[rank] = lane / K;
      L.pair_exp[rank] = e_p;
      L.pair_w[rank] = L.selw[lane];
      L.pos[lane] = rank;
      if (first) {
        L.act_exp[slot] = e_p;
        L.act_cnt[slot] = same;
        L.act_off[slot] = rank;
      }
    }
    if (lane == 0) L.n_active = __popcll(fm);
  }
  __syncthreads();
  stamp(a, 8);
  // routed gate/up: row pairs (active slot, ffn row) in contiguous blocks per workgroup
  {
    const int n_act = L.n_active;
    const int total = n_act * a.F;
    const int per = (total + G - 1) / G;
    const int rp0 = w * per, nrp = max(0, min(per, total - rp0));
    for (int m = 0; m < nrp; m += kFWaves / 2) {
      const int mm = m + (wv >> 1);
      if (mm < nrp) {
        const int slot = (rp0 + mm) / a.F, f = (rp0 + mm) % a.F;
        by_tokens(L.act_cnt[slot], [&](auto nt) { routed_gateup_row<decltype(nt)::value>(a, L, slot, f); });
      }
      __syncthreads();
      // combine: thread (pair-in-round pp, token j)
      const int pp = tid >> 3, j = tid & 7;
      if (pp < kFWaves / 2 && m + pp < nrp) {
        const int s2 = (rp0 + m + pp) / a.F, f2 = (rp0 + m + pp) % a.F;
        const int c2 = L.act_cnt[s2], o2 = L.act_off[s2];
        if (j < c2) {
          const int t = L.pair_tok[o2 + j];
          const float u = L.uv[2 * pp][j] * L.inv_rms[t], v = L.uv[2 * pp + 1][j] * L.inv_rms[t];
          put_tagged(a.act + (size_t)(o2 + j) * a.F + f2, silu_mul(u, v), tag);
        }
      }
      __syncthreads();
    }
  }
  stamp(a, 9);

  // ================= phase D =================
  {
    const int P = B * K;
    const int item0 = a.Fs > 0 ? 0 : B;
    by_lpg(a.F, [&](auto lpg) {
      constexpr int LPG = decltype(lpg)::value;
      const Down<LPG> d{a, L, i0, ni, item0, ni > 0 ? (B + P - item0) * ni : 0};
      uint4 wq[Down<LPG>::R];
      d.issue(0, wq);  // static weights: requested before the wait
      // gather every SwiGLU activation into LDS (routed [P][F], shared [B][Fs])
      {
        constexpr int PER = kFusedBig / kFT;
        const int n = P * a.F;
        uint64_t x[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) {
          const int q = tid + r * kFT;
          if (q < n) x[r] = ld_tagged(a.act + q);
        }
        const int ns = B * a.Fs;
        constexpr int PERS = kFusedActS / kFT;
        uint64_t xs[PERS];
#pragma unroll
        for (int r = 0; r < PERS; ++r) {
          const int q = tid + r * kFT;
          if (q < ns) xs[r] = ld_tagged(a.act_s + q);
        }
#pragma unroll
        for (int r = 0; r < PER; ++r) {
          const int q = tid + r * kFT;
          if (q < n) L.big[q] = finish_tagged(a.act + q, x[r], tag, a.spin_limit, &L.bad);
        }
#pragma unroll
        for (int r = 0; r < PERS; ++r) {
          const int q = tid + r * kFT;
          if (q < ns) L.act_s[q] = finish_tagged(a.act_s + q, xs[r], tag, a.spin_limit, &L.bad);
        }
      }
      __syncthreads();
      stamp(a, 10);
      const int nr = d.rounds();
      for (int r = 0; r < nr; ++r) {
        if (r > 0) d.issue(r, wq);
        d.consume(r, wq);
      }
    });
    __syncthreads();
    for (int q = tid; q < B * ni; q += kFT) {
      const int t = q / ni, il = q % ni;
      float y = a.Fs > 0 ? L.contrib[t * kFusedMaxSlice + il] : 0.f;
      for (int r = 0; r < K; ++r) y += L.contrib[(B + L.pos[t * K + r]) * kFusedMaxSlice + il];
      a.moe_out[(size_t)t * H + i0 + il] = y;
    }
  }
  stamp(a, 11);
  // attention input projection (independent of everything else)
  {
    const int rq = (a.Dq + G - 1) / G;
    const int j0 = w * rq, nj = max(0, min(rq, a.Dq - j0));
    if (nj > 0) by_tokens(B, [&](auto nt) { qkv_rows<decltype(nt)::value>(a, j0, nj); });
  }
  __syncthreads();
  stamp(a, 3);
  if (tid == 0) {
    if (L.bad) atomicOr(a.status, 1u);
    if (w == 0) *a.epoch = tag;   // every workgroup has read this step's epoch (all pss seen)
  }
}

hipError_t launch_fused(const FusedArgs &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(fused_step_kernel, dim3(grid), dim3(kFT), 0, s, a);
  return hipGetLastError();
}

int fused_blocks_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_step_kernel, kFusedThreads, 0) != hipSuccess) return 0;
  return n;
}

}  // namespace dl
