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
// Work of workgroup w (G workgroups):
//   * the H-slice S_w = [w*slice, (w+1)*slice) of the out-projection, the
//     norm statistics and the down projection;
//   * "units" u = w and w + G of the E + Fs row units: unit u < E is router
//     row u (fp32), unit u >= E is the shared expert's gate/up row pair
//     f = u - E (bf16); both are H*4 bytes, so the load is balanced;
//   * its share of the routed gate/up rows and of the qkv rows.
//
// Phases:
//  A  r1 = r + attn Wo^T on S_w -> resid_out; hg = g * r1 (global and LDS);
//     per-token partial sum of r1^2 over S_w -> published.
//     The unit rows (static weights) are requested into LDS.
//  B  1/rms(t) from the G partial sums (every workgroup, identical order);
//     with h = hg / rms read back from global memory:
//     l[t, e] = h[t] . Wr[e] -> published;
//     a_s[t, f] = silu(S1[f] . h[t]) * (S3[f] . h[t]) -> published.
//  C  (while the control waves gather the logits, the stream waves compute
//     this workgroup's rows of the attention input projection qkv = x Wqkv^T,
//     which depends on nothing else and so fills that hand-off's idle HBM
//     time — the role the pages give a side stream, bullets 1 and 3)
//     every workgroup reads all logits and takes the same top-k decision
//     (descending logit, ties to the lower expert id; s = sigmoid(l),
//     w = s / sum s over the k picks), builds the same per-expert token lists
//     in LDS (with one token, the top-k wave ranks its k distinct experts
//     directly), then computes its share of the routed gate/up rows:
//     a[p, f] = silu(W1[e, f] . h[t_p]) * (W3[e, f] . h[t_p])
//     for every (expert e, token t_p) pair p -> published.
//  D  y[t, i] for i in S_w:  sum_f S2[i, f] a_s[t, f]
//                           + sum over the k picks of t, in pick order, of
//                             w_p sum_f W2[e_p, i, f] a[p, f].
//     The first down-projection rows of the slice are staged in LDS while the
//     activations are in flight.  Each (item, row) dot product is formed in
//     a fixed order (by one thread when every unit is staged, else by a lane
//     group), and each y element is the sum of its items in pick order.
//
// Wave roles.  A wave's loads complete in issue order, so a poll issued after
// a bulk weight request waits for that request.  Waves 0-3 (control) poll and
// never have bulk requests outstanding when they do; waves 4-7 (stream)
// request the static weights of later phases (unit rows, qkv rows, the first
// down-projection rows) ahead of time.  All eight stream the routed rows.
//
// Hand-offs.  Values produced by one workgroup for another (partial sums,
// logits, SwiGLU activations) are written as 64-bit pairs (value, tag) with
// device-scope relaxed atomic stores, and read by polling with device-scope
// relaxed atomic loads until the tag equals this step's tag: a consumer waits
// exactly for the data it needs, with one memory round trip and no counter
// that every workgroup would have to serialise on.  The tag is the handle's
// step counter + 1, kept in device memory and advanced by workgroup 0 at the
// end of each step, so it is also right under HIP-graph replay.  hg is
// written with device-scope stores that have completed before the phase-A
// hand-off values are published; after that hand-off a step of several tokens
// acquires (agent-scope fence) and reads hg through the caches, and a step of
// one token reads it at device scope.  Only static weights are
// read before a wait (the ordering rule of wireai.ir, "Oversight and
// validation for AI-generated kernels").  Every wait is bounded: on expiry the
// kernel records an error in the handle's status word and runs to completion.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dl {

namespace {

constexpr int kFT = kFusedThreads;          // 512 threads, 8 waves
constexpr int kFWaves = kFT / kWave;
constexpr int kCtl = 256;                   // control threads (waves 0-3); stream threads are kCtl..kFT-1
constexpr int kStr = kFT - kCtl;
constexpr int kUnitU4 = kFusedMaxH / 4;     // 16-byte words of one unit row (H*4 bytes)
constexpr int kUnitJ = kUnitU4 / kStr;      // words per stream thread per unit (8)
constexpr int kChunkJ = kFusedMaxH / 8 / kFT;  // 8-element chunks per thread in phase B (2)
static_assert(kFusedW2Words % kStr == 0, "staging split");

// ---- tagged hand-off values -------------------------------------------------
__device__ __forceinline__ void put_tagged(uint64_t *p, float v, unsigned tag) {
  uint64_t x = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits for N tagged values whose first reads x[i] (of p[i]) are already in
// flight: every round re-reads all values whose tag is not yet this step's,
// together, so a thread waiting on N late values pays one round trip per
// round, not one per value.  On expiry of the spin budget *bad is set.
template <int N>
__device__ __forceinline__ void finish_tagged_n(const uint64_t *const (&p)[N], uint64_t (&x)[N], const bool (&use)[N],
                                                unsigned tag, int limit, int *bad) {
  for (int n = 0;; ++n) {
    bool done = true;
#pragma unroll
    for (int i = 0; i < N; ++i) done &= !use[i] || (unsigned)(x[i] >> 32) == tag;
    if (done) return;
    if (n >= limit) {
      *bad = 1;
      return;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (use[i] && (unsigned)(x[i] >> 32) != tag) x[i] = ld_tagged(p[i]);
  }
}
// Polls n tagged values src[i], i = first, first + stride, ... into dst[i],
// eight requests in flight per thread.
__device__ __forceinline__ void gather_tagged(const uint64_t *src, float *dst, int first, int stride, int n,
                                              unsigned tag, int limit, int *bad) {
  for (int i0 = first; i0 < n; i0 += 8 * stride) {
    const uint64_t *p[8];
    uint64_t x[8];
    bool use[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = i0 + r * stride;
      use[r] = i < n;
      p[r] = src + (use[r] ? i : first);
      x[r] = ld_tagged(p[r]);
    }
    finish_tagged_n<8>(p, x, use, tag, limit, bad);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = i0 + r * stride;
      if (i < n) dst[i] = __uint_as_float((unsigned)x[r]);
    }
  }
}

__device__ __forceinline__ void as8(const uint4 &a, const uint4 &b, float (&f)[8]) {
  f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
  f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
}

// Phase trace (measurement only): thread 0 stamps the device wall clock.
__device__ __forceinline__ void stamp(const FusedArgs &a, int point) {
  if (a.trace && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * kTracePoints + point] = wall_clock64();
}

struct Lds {
  float hg[kFusedMaxB][kFusedMaxSlice];
  float red[kFWaves * kFusedMaxB * 4];
  float inv_rms[kFusedMaxB];
  union {
    uint4 unit[2][kUnitU4];   // phase A/B: this workgroup's unit rows
    float logits[kFusedBig];  // phase C: every logit
    struct {                  // phase D
      float act[kFusedBig];
      float act_s[kFusedActS];
      float contrib[(kFusedMaxB + kFusedMaxPairs) * kFusedMaxSlice];
    } d;
  } u;
  uint4 w2[kFusedW2Words];    // phase D: the first down-projection rows of the slice
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
  // split top-k of one token: each wave's picks, and the waves that have
  // written theirs
  unsigned tk_key[kWave];
  int tk_idx[kWave];
  int tk_arrive;
  // gate/up sums of a round: [item][K half][W1 | W3][token]
  float uv[4][2][2][kFusedMaxB];
  // list building: per-wave partial counts of keys below / of the same expert
  int part_lt[kFWaves][kWave];
  int part_same[kFWaves][kWave];
  float sqw[kFWaves][kFusedMaxB];  // per-wave partial sums of r1^2
  float qkvp[kStr / kWave][kFusedQkvRows][kFusedMaxB];  // input-projection partial sums per stream wave
  int arrive;
  int bad;
};

// ---- phase A: out-projection rows of the slice -------------------------------
// Wave v owns rows il = v + 8r (r < 4) of the slice.  Lane t < B keeps token
// t: r1 -> resid_out, hg -> global (device-scope stores, written through) and
// LDS, and returns its partial sum of r1^2 over the wave's rows.
template <int NT>
__device__ float oproj_rows(const FusedArgs &a, Lds &L, int i0, int ni) {
  constexpr int NR = kFusedMaxSlice / kFWaves;  // 4
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int B = a.B;
  const ActBf16Rows act{a.attn, a.Do, B - 1};
  const int nch = a.Do >> 3;
  const uint16_t *rows[NR];
  int il[NR];
  float res[NR];
  uint16_t gn[NR];
  // every load unconditional (token and row clamped), so that none of them
  // is waited for before the weight loads are issued
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    il[r] = wv + kFWaves * r;
    const int i = i0 + min(il[r], ni - 1);
    rows[r] = a.w_o + (size_t)i * a.Do;
    res[r] = a.resid_in[(size_t)min(lane, B - 1) * a.H + i];
    gn[r] = a.gain[i];
  }
  float o[NR][NT];
  wave_rows_dot<NR, NT, (NT >= 8 ? 1 : 2)>(rows, 0, nch, act, o);
  float sq = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float mine = 0.f;  // lane t keeps token t's sum
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (lane == t) mine = o[r][t];
    if (lane < B && il[r] < ni) {
      const int i = i0 + il[r];
      const size_t ix = (size_t)lane * a.H + i;
      const float r1 = res[r] + mine;
      a.resid_out[ix] = r1;
      const float hgv = bf16_lo(gn[r]) * r1;
      __hip_atomic_store(a.hg + ix, hgv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      L.hg[lane][il[r]] = hgv;
      sq += r1 * r1;
    }
  }
  return sq;
}

// ---- phase C: gate/up rows --------------------------------------------------
// A gate/up item's tokens: a routed expert's LDS token list, or all B tokens
// of the shared expert.
struct GuRow {
  const int *toks = nullptr;  // LDS token list, or nullptr for tokens 0..cnt-1
  int cnt = 0;
  __device__ __forceinline__ int tok(int t) const {
    const int tt = t < cnt ? t : cnt - 1;
    return toks ? toks[tt] : tt;
  }
};

// 16-byte chunks per lane per load batch: 2 weight words and NT activation
// octets each, about 100 VGPRs in flight.
template <int NT>
constexpr int gu_cpb() { return NT <= 1 ? 7 : NT <= 2 ? 4 : NT <= 4 ? 2 : 1; }

// One wave: the W1 and W3 rows of one item over 16-byte chunks [cbeg, cend)
// (8 elements each), dotted with the hg rows of the item's tokens.  Every
// load of a batch - weights and activations - is issued before any is used,
// so a batch costs one memory round trip.  Sums come back in every lane.
template <int NT>
__device__ void gateup_pair(const GuRow &r, const uint16_t *row1, const uint16_t *row3, const float *hg, int H,
                            int cbeg, int cend, float (&su)[NT], float (&sv)[NT]) {
  constexpr int CPB = gu_cpb<NT>();
  const int lane = threadIdx.x & 63;
  const float *hrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) hrow[t] = hg + (size_t)r.tok(t) * H;
  float au[NT], av[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) au[t] = av[t] = 0.f;
  for (int c0 = cbeg; c0 < cend; c0 += CPB * kWave) {
    uint4 w1[CPB], w3[CPB];
    float4 x[CPB][NT][2];
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int cc = min(c0 + lane + kWave * u, cend - 1);
      w1[u] = ld_stream16(row1 + (size_t)cc * 8);
      w3[u] = ld_stream16(row3 + (size_t)cc * 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        x[u][t][0] = ld16f(hrow[t] + (size_t)cc * 8);
        x[u][t][1] = ld16f(hrow[t] + (size_t)cc * 8 + 4);
      }
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const bool on = c0 + lane + kWave * u < cend;
      float f1[8], f3[8];
      unpack8(zero_unless(on, w1[u]), f1);
      unpack8(zero_unless(on, w3[u]), f3);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float hv[8] = {x[u][t][0].x, x[u][t][0].y, x[u][t][0].z, x[u][t][0].w,
                             x[u][t][1].x, x[u][t][1].y, x[u][t][1].z, x[u][t][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          au[t] = fmaf(f1[e], hv[e], au[t]);
          av[t] = fmaf(f3[e], hv[e], av[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    su[t] = wave_sum(au[t]);
    sv[t] = wave_sum(av[t]);
  }
}

// The same with the item's hg rows staged in LDS (hl: [cnt][H] fp32, row t
// of token t of the item): only the weights travel from memory, 7 chunks of
// each row per load batch.
template <int NT>
__device__ void gateup_pair_lds(const uint16_t *row1, const uint16_t *row3, const float *hl, int cnt, int H,
                                int cbeg, int cend, float (&su)[NT], float (&sv)[NT]) {
  constexpr int CPB = 7;
  const int lane = threadIdx.x & 63;
  float au[NT], av[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) au[t] = av[t] = 0.f;
  for (int c0 = cbeg; c0 < cend; c0 += CPB * kWave) {
    uint4 w1[CPB], w3[CPB];
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int cc = min(c0 + lane + kWave * u, cend - 1);
      w1[u] = ld_stream16(row1 + (size_t)cc * 8);
      w3[u] = ld_stream16(row3 + (size_t)cc * 8);
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int cc = min(c0 + lane + kWave * u, cend - 1);
      const bool on = c0 + lane + kWave * u < cend;
      float f1[8], f3[8];
      unpack8(zero_unless(on, w1[u]), f1);
      unpack8(zero_unless(on, w3[u]), f3);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float *hp = hl + (size_t)min(t, cnt - 1) * H + (size_t)cc * 8;
        const float4 x0 = *reinterpret_cast<const float4 *>(hp), x1 = *reinterpret_cast<const float4 *>(hp + 4);
        const float hv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          au[t] = fmaf(f1[e], hv[e], au[t]);
          av[t] = fmaf(f3[e], hv[e], av[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    su[t] = wave_sum(au[t]);
    sv[t] = wave_sum(av[t]);
  }
}

// ---- phase D: one (item, row) unit per group of LPG lanes --------------------
// Items 0..B-1 are the shared expert's tokens (weights S2, activations
// act_s), items B..B+P-1 the routed pairs (weights W2 of the pair's expert,
// activations act, scaled by the pair's weight); F = 8 * LPG for both.
// Without a shared expert the items start at B.  Unit u = (item0 + u / ni,
// row u % ni).  The weights of units [0, U0) are staged in LDS by the stream
// threads while the activations are awaited; the rest are streamed.
// A lane group walks its units with a fixed stride, so the (item, row) of
// each is advanced by an add and one compare instead of a division by the
// slice height.
struct UnitWalk {
  int item, il, dq, dr, ni;
  // position of unit u and the increment of a stride of s units
  __device__ UnitWalk(int u, int s, int item0, int ni_) : ni(ni_) {
    item = item0 + u / ni;
    il = u % ni;
    dq = s / ni;
    dr = s % ni;
  }
  __device__ void next() {
    item += dq;
    il += dr;
    if (il >= ni) {
      il -= ni;
      ++item;
    }
  }
};

template <int LPG>
struct Down {
  static constexpr int NG = kFT / LPG;  // lane groups
  static constexpr int R = 16;  // units per lane group per load batch
  const FusedArgs &a;
  Lds &L;
  int i0, ni, item0, n_units;
  __device__ int u0_end() const { return min(n_units, kFusedW2Words / LPG); }
  __device__ const uint16_t *row(int item, int il) const {
    return item < a.B ? a.s2 + (size_t)(i0 + il) * a.F
                      : a.w2 + ((size_t)L.pair_exp[item - a.B] * a.H + i0 + il) * a.F;
  }
  __device__ const uint16_t *row_of(int u) const { return row(item0 + u / ni, u % ni); }
  // stream threads: word k of the staged range is unit k / LPG, lane k % LPG
  // (words past the range load the last word, so every load of the batch
  // issues unconditionally and the batch is one memory round trip)
  __device__ void stage() const {
    const int ue = u0_end(), n = ue * LPG;
    if (n == 0) return;
    constexpr int J = kFusedW2Words / kStr;  // 16
    constexpr int S = kStr / LPG;            // units between a thread's words
    static_assert(kStr % LPG == 0, "staging stride");
    const int st = threadIdx.x - kCtl, lg = st % LPG;
    const uint16_t *last = row_of(ue - 1) + (LPG - 1) * 8;
    UnitWalk wk(st / LPG, S, item0, ni);
    uint4 v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int u = st / LPG + S * j;
      v[j] = ld_stream16(u < ue ? row(wk.item, wk.il) + lg * 8 : last);
      wk.next();
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = st + kStr * j;
      if (k < n) L.w2[swz(k / LPG, k % LPG)] = v[j];
    }
  }
  // LDS word of word j of staged unit u: the words of a unit are rotated by
  // an xor with u, so that threads reading word j of consecutive units hit
  // different banks, and a lane group reading one unit still covers all
  __device__ static int swz(int u, int j) { return u * LPG + (j ^ (u & (LPG - 1))); }
  __device__ void use(int item, int il, const uint4 &wv) const {
    const int lg = threadIdx.x % LPG;
    const float *ap = item < a.B ? L.u.d.act_s + item * a.F + lg * 8 : L.u.d.act + (item - a.B) * a.F + lg * 8;
    float wf[8];
    unpack8(wv, wf);
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) s = fmaf(wf[q], ap[q], s);
    s = group_sum(s, LPG);
    if (lg == 0) L.u.d.contrib[item * kFusedMaxSlice + il] = item < a.B ? s : s * L.pair_w[item - a.B];
  }
  // every unit staged: one unit per thread, its whole row summed in order,
  // with no cross-lane sums
  __device__ void compute_staged() const {
    for (int u = threadIdx.x; u < n_units; u += kFT) {
      const int item = item0 + u / ni, il = u % ni;
      const float *ap = item < a.B ? L.u.d.act_s + item * a.F : L.u.d.act + (item - a.B) * a.F;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < LPG; ++j) {
        float wf[8];
        unpack8(L.w2[swz(u, j)], wf);
        const float4 x0 = *reinterpret_cast<const float4 *>(ap + 8 * j);
        const float4 x1 = *reinterpret_cast<const float4 *>(ap + 8 * j + 4);
        s = fmaf(wf[0], x0.x, s);
        s = fmaf(wf[1], x0.y, s);
        s = fmaf(wf[2], x0.z, s);
        s = fmaf(wf[3], x0.w, s);
        s = fmaf(wf[4], x1.x, s);
        s = fmaf(wf[5], x1.y, s);
        s = fmaf(wf[6], x1.z, s);
        s = fmaf(wf[7], x1.w, s);
      }
      L.u.d.contrib[item * kFusedMaxSlice + il] = item < a.B ? s : s * L.pair_w[item - a.B];
    }
  }
  // all threads: staged units from LDS, then the rest streamed
  __device__ void compute() const {
    if (n_units == 0) return;
    const int g = threadIdx.x / LPG, lg = threadIdx.x % LPG;
    const int ue = u0_end();
    if (ue == n_units) {
      compute_staged();
      return;
    }
    {
      UnitWalk wk(g, NG, item0, ni);
      for (int ub = 0; ub < ue; ub += NG * R) {
        uint4 wv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int u = ub + g + NG * r;
          wv[r] = u < ue ? L.w2[swz(u, lg)] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int u = ub + g + NG * r;
          if (u < ue) use(wk.item, wk.il, wv[r]);
          wk.next();
        }
      }
    }
    if (ue >= n_units) return;
    const uint16_t *last = row_of(n_units - 1) + lg * 8;
    UnitWalk wk(ue + g, NG, item0, ni);
    for (int ub = ue; ub < n_units; ub += NG * R) {
      uint4 wv[R];
      UnitWalk lw = wk;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int u = ub + g + NG * r;
        wv[r] = ld_stream16(u < n_units ? row(lw.item, lw.il) + lg * 8 : last);
        lw.next();
      }
      DL_SCHED_FENCE();
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int u = ub + g + NG * r;
        if (u < n_units) use(wk.item, wk.il, wv[r]);
        wk.next();
      }
    }
  }
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

// ---- cross-layer prefetch ------------------------------------------------------
// The rows that workgroup w of the next layer reads before its first
// hand-off - the out-projection rows of its slice and its two unit rows
// (router row, or shared-expert row pair): up to five ranges - are touched
// once per 64-byte sector, so that they sit in this XCD's L2 (workgroup w of
// the next launch runs on the same XCD) and in the memory-side cache when
// that layer starts.  The values are folded into a word that is written only
// under a condition that never holds, which keeps the loads without using
// them.  Threads [t0, kFT) take the sectors, numbered across the ranges in
// turn; each issues up to kPfDepth loads before it waits, so that a few waves
// cover them all in one memory round trip.
constexpr int kPfDepth = 12;
__device__ __forceinline__ unsigned prefetch_next(const FusedArgs &a, int w, int G, int i0, int ni, int t0) {
  const int E = a.E, H = a.H;
  const int fs_b = max(0, min(a.Fs, 2 * G - E));
  const char *p[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  unsigned n[5] = {0u, 0u, 0u, 0u, 0u};  // sectors per range
  if (ni > 0) {
    p[0] = reinterpret_cast<const char *>(a.pf_w_o + (size_t)i0 * a.Do);
    n[0] = ((unsigned)ni * a.Do * 2u + 63u) >> 6;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int u = w + G * q;
    if (u < E) {
      p[1 + 2 * q] = reinterpret_cast<const char *>(a.pf_w_router + (size_t)u * H);
      n[1 + 2 * q] = ((unsigned)H * 4u + 63u) >> 6;
    } else if (u < E + fs_b) {
      p[1 + 2 * q] = reinterpret_cast<const char *>(a.pf_s1 + (size_t)(u - E) * H);
      p[2 + 2 * q] = reinterpret_cast<const char *>(a.pf_s3 + (size_t)(u - E) * H);
      n[1 + 2 * q] = n[2 + 2 * q] = ((unsigned)H * 2u + 63u) >> 6;
    }
  }
  const unsigned total = n[0] + n[1] + n[2] + n[3] + n[4];
  const int tt = (int)threadIdx.x - t0, nt = kFT - t0;
  unsigned acc = 0;
  for (unsigned s0 = 0; s0 < total; s0 += (unsigned)(kPfDepth * nt)) {
    unsigned v[kPfDepth];
#pragma unroll
    for (int j = 0; j < kPfDepth; ++j) {
      // sector s of the concatenated ranges (past the end: the last one)
      unsigned s = min(s0 + tt + (unsigned)nt * j, total - 1u);
      const char *b = p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (s < n[r]) {
          b = p[r];
          break;
        }
        s -= n[r];
      }
      v[j] = *reinterpret_cast<const unsigned *>(b + 64u * s);
    }
#pragma unroll
    for (int j = 0; j < kPfDepth; ++j) acc ^= v[j];
  }
  return acc;
}

// ---- phase C, stream waves: the attention input projection ------------------
// It depends on nothing else in the step, so it fills the logits hand-off:
// this workgroup's rows are j = w + G q (q < kFusedQkvRows), taken two at a
// time; stream wave sw covers the quarter sw of K.  The four partial sums of
// a row are added in wave order after the phase's barrier.
template <int NT>
__device__ void qkv_rows(const FusedArgs &a, Lds &L, int w, int G) {
  constexpr int CPB = NT >= 4 ? 2 : 4;
  const int sw = (threadIdx.x - kCtl) >> 6, lane = threadIdx.x & 63;
  const int nc = a.H >> 3, cb = sw * nc / 4, ce = (sw + 1) * nc / 4;
  const ActBf16Rows act{a.x, a.H, a.B - 1};
  for (int q = 0; q < kFusedQkvRows && w + G * q < a.Dq; q += 2) {
    const int j0 = w + G * q, j1 = min(j0 + G, a.Dq - 1);
    const uint16_t *row[2] = {a.w_qkv + (size_t)j0 * a.H, a.w_qkv + (size_t)j1 * a.H};
    float s[2][NT];
    wave_rows_dot<2, NT, CPB>(row, cb, ce, act, s);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (lane == t && q + r < kFusedQkvRows) L.qkvp[sw][q + r][t] = s[r][t];
  }
}

__global__ void __launch_bounds__(kFT, 1) fused_step_kernel(FusedArgs a) {
  __shared__ Lds L;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool ctl = tid < kCtl;
  const int st = tid - kCtl;  // stream-thread index (valid when !ctl)
  const int w = blockIdx.x, G = gridDim.x;
  const int B = a.B, E = a.E, K = a.K, H = a.H;
  // this step's tag: the last step's tag + 1, skipping 0 (the tag of a slot
  // never written); the step with the last tag clears every hand-off slot at
  // its end, so after the wrap no slot holds a tag of the new round
  // (a vector load: it completes under the first weight loads instead of
  // holding the start-of-kernel barrier for a memory round trip)
  const unsigned epoch = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned tag = epoch == 0xffffffffu ? 1u : epoch + 1u;
  const float kNaN = __builtin_nanf("");
  if (tid == 0) {
    L.bad = 0;
    L.arrive = 0;
    L.tk_arrive = 0;
  }
  __syncthreads();
  const int i0 = w * a.slice;
  const int ni = max(0, min(a.slice, H - i0));
  stamp(a, 0);

  // ================= phase A =================
  {
    // out-projection rows.  Each wave leaves its partial sums of r1^2 in LDS
    // once its hg values are written through; the last wave to arrive adds
    // the 8 partials in wave order and publishes them (no workgroup barrier).
    float sq = 0.f;
    if (ni > 0) by_tokens(B, [&](auto nt) { sq = oproj_rows<decltype(nt)::value>(a, L, i0, ni); });
    wt_stores_complete();  // this wave's device-scope hg stores have completed
    if (lane < B) L.sqw[wv][lane] = sq;
    int arrived = 0;
    if (lane == 0) arrived = __hip_atomic_fetch_add(&L.arrive, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    arrived = __builtin_amdgcn_readfirstlane(arrived);
    if (arrived == kFWaves - 1 && lane < B) {
      float s8 = 0.f;
#pragma unroll
      for (int v = 0; v < kFWaves; ++v) s8 += __hip_atomic_load(&L.sqw[v][lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      put_tagged(a.pss + (size_t)w * B + lane, s8, tag);
    }
  }
  stamp(a, 1);
  // Units u = w and w + G of this workgroup: u < E is router row u (fp32,
  // H * 4 bytes); E <= u < E + fs_b is the shared expert's row pair
  // f = u - E (S1 row f then S3 row f, bf16, also H * 4 bytes).  Shared rows
  // f >= fs_b join the routed gate/up items of phase C.
  const int fs_b = max(0, min(a.Fs, 2 * G - E));
  const int er[2] = {w, w + G};
  int kind[2];  // 0 none, 1 router row, 2 shared row pair
#pragma unroll
  for (int q = 0; q < 2; ++q) kind[q] = er[q] < E ? 1 : er[q] < E + fs_b ? 2 : 0;
  if (!ctl) {
    // stream threads: the unit rows (static weights) -> LDS
    uint4 v[2][kUnitJ];
    const int nw = H >> 2;  // 16-byte words per unit
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      // router: words [0, nw) of the fp32 row; shared: S1 row f in words
      // [0, nw/2) and S3 row f in words [nw/2, nw)
      const int half = nw >> 1;
      const uint4 *src0, *src1;
      if (kind[q] == 2) {
        src0 = reinterpret_cast<const uint4 *>(a.s1 + (size_t)(er[q] - E) * H);
        src1 = reinterpret_cast<const uint4 *>(a.s3 + (size_t)(er[q] - E) * H);
      } else {
        src0 = reinterpret_cast<const uint4 *>(a.w_router + (size_t)min(er[q], E - 1) * H);
        src1 = src0 + half;
      }
#pragma unroll
      for (int j = 0; j < kUnitJ; ++j) {
        const int i = st + kStr * j;
        v[q][j] = kind[q] && i < nw ? ld_stream16(i < half ? src0 + i : src1 + (i - half)) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int j = 0; j < kUnitJ; ++j) {
        const int i = st + kStr * j;
        if (kind[q] && i < nw) L.u.unit[q][i] = v[q][j];
      }
  } else {
    // control threads: the G*B partial sums pss[w][t], thread tid polling
    // words tid + kCtl*j, so each wave instruction reads 64 consecutive words
    const int N = G * B;
    const uint64_t *pp[kFusedMaxB];
    uint64_t x[kFusedMaxB];
    bool use[kFusedMaxB];
#pragma unroll
    for (int j = 0; j < kFusedMaxB; ++j) {
      const int i = tid + kCtl * j;
      use[j] = i < N;
      pp[j] = a.pss + (use[j] ? i : 0);
      x[j] = use[j] ? ld_tagged(pp[j]) : 0ull;
    }
    finish_tagged_n<kFusedMaxB>(pp, x, use, tag, a.spin_limit, &L.bad);
    stamp(a, 2);
    if ((kWave % B) == 0) {
      // B divides the wave: every word of this thread is token tid % B; sum
      // them, then over the lanes of the same token (xor strides >= B), and
      // leave one partial per wave and token
      float v = 0.f;
#pragma unroll
      for (int j = 0; j < kFusedMaxB; ++j) v += use[j] ? __uint_as_float((unsigned)x[j]) : 0.f;
      if (B == 1)
        v = wave_sum(v);
      else
        for (int m = B; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
      if (lane < B) L.red[wv * kFusedMaxB + lane] = v;
    } else {
      // otherwise the words land in LDS (the down-projection staging area,
      // free until phase D) and one wave per token adds them
      float *pssv = reinterpret_cast<float *>(L.w2);
#pragma unroll
      for (int j = 0; j < kFusedMaxB; ++j)
        if (use[j]) pssv[tid + kCtl * j] = __uint_as_float((unsigned)x[j]);
    }
  }
  __syncthreads();
  // token t's sum over the workgroups in a fixed order (the same in every
  // workgroup, so every workgroup derives the same 1/rms)
  if ((kWave % B) == 0) {
    if (tid < B) {
      float s = 0.f;
      for (int q = 0; q < kCtl / kWave; ++q) s += L.red[q * kFusedMaxB + tid];
      L.inv_rms[tid] = 1.0f / sqrtf(s / (float)H + a.eps);
    }
  } else if (wv < B) {
    const float *pssv = reinterpret_cast<const float *>(L.w2);
    float s = 0.f;
    for (int q = lane; q < G; q += kWave) s += pssv[q * B + wv];
    s = wave_sum(s);
    if (lane == 0) L.inv_rms[wv] = 1.0f / sqrtf(s / (float)H + a.eps);
  }
  // every workgroup's hg is now announced.  With several tokens, acquire
  // before reading it through the caches (drops any line of an earlier
  // step's hg from this XCD's caches).  With one token every read of hg is
  // at device scope instead (phase B here, the copy staged in LDS in phase
  // C), which spares the acquire's cache invalidation on the critical path.
  if (B > 1 && tid == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  stamp(a, 4);
  // After a wait of this workgroup has expired, every value it publishes and
  // every output it writes from then on is NaN (an index -1): the failure
  // reaches the outputs instead of leaving stale values behind.  Indices used
  // inside the kernel still come from the top-k, so they stay valid.
  const bool poison_b = L.bad != 0;

  // ================= phase B: router logits and shared-expert rows ==========
  if (a.h_out && ni > 0)
    for (int q = tid; q < B * ni; q += kFT) {
      const int t = q / ni, il = q % ni;
      a.h_out[(size_t)t * H + i0 + il] = poison_b ? kNaN : L.hg[t][il] * L.inv_rms[t];
    }
  if (kind[0] || kind[1]) by_tokens(B, [&](auto tgc) {  // uniform over the workgroup
    const int nc = H >> 3;    // 8-element chunks c = tid + kFT*j
    // tokens whose hg chunks are requested together: the whole batch (up to 8)
    constexpr int TG = decltype(tgc)::value;
    for (int t0 = 0; t0 < B; t0 += TG) {
      float4 hx[TG][kChunkJ][2];
      if constexpr (TG == 1) {  // one token: device scope, no acquire before
        const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc((void *)a.hg, 0, H * 4, 0x00020000);
#pragma unroll
        for (int j = 0; j < kChunkJ; ++j) {
          const int c = min(tid + kFT * j, nc - 1);
          hx[0][j][0] = ld16f_dev(hr, 8 * c);
          hx[0][j][1] = ld16f_dev(hr, 8 * c + 4);
        }
      } else {
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          const float *hrow = a.hg + (size_t)min(t0 + tt, B - 1) * H;
#pragma unroll
          for (int j = 0; j < kChunkJ; ++j) {
            const int c = min(tid + kFT * j, nc - 1);
            hx[tt][j][0] = ld16f(hrow + 8 * c);
            hx[tt][j][1] = ld16f(hrow + 8 * c + 4);
          }
        }
      }
      DL_SCHED_FENCE();
      if constexpr (TG == 1) {
        // the whole row is now in this workgroup's registers: keep a copy in
        // the down-projection staging area (free until phase D), where every
        // gate/up item of phase C reads it
        float4 *hl = reinterpret_cast<float4 *>(L.w2);
#pragma unroll
        for (int j = 0; j < kChunkJ; ++j) {
          const int c = tid + kFT * j;
          if (c < nc) {
            hl[2 * c] = hx[0][j][0];
            hl[2 * c + 1] = hx[0][j][1];
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < TG; ++tt) {
        const int t = t0 + tt;
        if (t >= B) break;
        float p[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // [unit][router or S1 | S3]
#pragma unroll
        for (int j = 0; j < kChunkJ; ++j) {
          const int c = tid + kFT * j;
          if (c < nc) {
            const float hv[8] = {hx[tt][j][0].x, hx[tt][j][0].y, hx[tt][j][0].z, hx[tt][j][0].w,
                                 hx[tt][j][1].x, hx[tt][j][1].y, hx[tt][j][1].z, hx[tt][j][1].w};
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              float wa[8];
              if (kind[q] == 1) {
                as8(L.u.unit[q][2 * c], L.u.unit[q][2 * c + 1], wa);
#pragma unroll
                for (int k2 = 0; k2 < 8; ++k2) p[q][0] = fmaf(wa[k2], hv[k2], p[q][0]);
              } else if (kind[q] == 2) {
                unpack8(L.u.unit[q][c], wa);
#pragma unroll
                for (int k2 = 0; k2 < 8; ++k2) p[q][0] = fmaf(wa[k2], hv[k2], p[q][0]);
                unpack8(L.u.unit[q][nc + c], wa);
#pragma unroll
                for (int k2 = 0; k2 < 8; ++k2) p[q][1] = fmaf(wa[k2], hv[k2], p[q][1]);
              }
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            if (kind[q] == 0 || (m == 1 && kind[q] != 2)) continue;
            const float v = wave_sum(p[q][m]);
            if (lane == 0) L.red[((wv * kFusedMaxB + t) * 2 + q) * 2 + m] = v;
          }
      }
    }
    __syncthreads();
    if (tid < 2 * B) {
      const int q = tid & 1, t = tid >> 1;
      float sp[2] = {0.f, 0.f};
      for (int v = 0; v < kFWaves; ++v) {
        sp[0] += L.red[((v * kFusedMaxB + t) * 2 + q) * 2 + 0];
        sp[1] += L.red[((v * kFusedMaxB + t) * 2 + q) * 2 + 1];
      }
      if (kind[q] == 1) {
        const float l = poison_b ? kNaN : sp[0] * L.inv_rms[t];
        put_tagged(a.logit + (size_t)t * E + er[q], l, tag);
        if (a.logits_out) a.logits_out[(size_t)t * E + er[q]] = l;
      } else if (kind[q] == 2) {
        const int f = er[q] - E;
        put_tagged(a.act_s + (size_t)t * a.Fs + f,
                   poison_b ? kNaN : silu_mul(sp[0] * L.inv_rms[t], sp[1] * L.inv_rms[t]), tag);
      }
    }
  });
  __syncthreads();   // the unit rows in LDS are dead from here on
  stamp(a, 5);

  // ================= phase C =================
  unsigned pf_acc = 0;
  if (ctl) {
    gather_tagged(a.logit, L.u.logits, tid, kCtl, B * E, tag, a.spin_limit, &L.bad);
  } else {
    by_tokens(B, [&](auto nt) { qkv_rows<decltype(nt)::value>(a, L, w, G); });
    // one token, in a workgroup without units (phase B did not read hg):
    // its hg row, at device scope, into the down-projection staging area
    if (B == 1 && !(kind[0] || kind[1])) {
      static_assert(sizeof(float) * kFusedMaxH <= sizeof(L.w2), "one hg row fits the staging area");
      const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc((void *)a.hg, 0, H * 4, 0x00020000);
      constexpr int PT = kFusedMaxH / 4 / kStr;  // 16-byte words per stream thread (at most)
      const int nw = H >> 2, st = tid - kCtl;
      float4 v[PT];
#pragma unroll
      for (int j = 0; j < PT; ++j) v[j] = ld16f_dev(hr, 4 * min(st + kStr * j, nw - 1));
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (st + kStr * j < nw) reinterpret_cast<float4 *>(L.w2)[st + kStr * j] = v[j];
    }
  }
  __syncthreads();
  stamp(a, 7);
  const bool poison_c = L.bad != 0;
  for (int q = tid; q < kFusedQkvRows * B; q += kFT) {
    const int r = q / B, t = q % B, j = w + G * r;
    if (j < a.Dq)
      a.qkv[(size_t)t * a.Dq + j] = ((L.qkvp[0][r][t] + L.qkvp[1][r][t]) + L.qkvp[2][r][t]) + L.qkvp[3][r][t];
  }
  // One token: its candidates are spread over nwk waves, one per lane; each
  // takes its k largest, and wave 0 merges those lists.  A round then costs a
  // wave maximum and a ballot instead of a maximum over several candidates
  // per lane and a search for the lowest index holding it.
  const int nwk = (E + kWave - 1) / kWave;
  const bool split_topk = B == 1 && nwk * K <= kWave;
  const int busy = split_topk ? nwk : B;  // waves the top-k uses
  // The waves the top-k leaves idle touch the next layer's first rows
  // meanwhile: no wave polls during the top-k, so HBM is idle.
  if (a.pf_w_o && busy < kFWaves && wv >= busy) pf_acc = prefetch_next(a, w, G, i0, ni, busy * kWave);
  // scores of the k picks of token t, renormalised (lane j holds pick j),
  // written out; with one token its lists as well.  With the split top-k
  // the weights are deferred: selw keeps the picks' logits, and a control
  // wave turns them into weights in phase D, while it waits for the
  // activations (only phase D reads them), so gate/up starts earlier.
  auto finish_token = [&](int t, int my_idx, float my_l) __attribute__((always_inline)) {
    const float wgt = split_topk ? my_l : pick_weights(my_l, K);
    if (lane < K) {
      L.sel[t * K + lane] = my_idx;
      L.selw[t * K + lane] = wgt;
      if (w == 0) {
        a.topk_idx[(size_t)t * K + lane] = poison_c ? -1 : my_idx;
        if (!split_topk) a.topk_w[(size_t)t * K + lane] = poison_c ? kNaN : wgt;
      }
    }
    if (B == 1) {
      // one token: its k picks are k distinct experts, so this wave builds
      // the lists at once - pair order is expert order, each expert one pair
      int rank = 0;
      for (int i = 0; i < K; ++i) rank += __builtin_amdgcn_readlane(my_idx, i) < my_idx;
      if (lane < K) {
        L.pair_tok[rank] = 0;
        L.pair_exp[rank] = my_idx;
        L.pair_w[rank] = wgt;
        L.pos[lane] = rank;
        L.act_exp[rank] = my_idx;
        L.act_cnt[rank] = 1;
        L.act_off[rank] = rank;
      }
      if (lane == 0) L.n_active = K;
    }
  };
  if (split_topk) {
    if (wv < nwk) {
      stamp(a, 14);
      const int e = wv * kWave + lane;
      unsigned key[1] = {e < E ? rank_bits(L.u.logits[e]) : 0u};
      unsigned pk;
      int pi;
      wave_topk_blocks<1>(key, wv * kWave, K, pk, pi);
      if (lane < K) {
        L.tk_key[wv * K + lane] = pk;
        L.tk_idx[wv * K + lane] = pi;
      }
      // wave 0 waits for the other lists only: a workgroup barrier would
      // also wait for the prefetching waves
      if (wv > 0) {
        if (lane == 0) __hip_atomic_fetch_add(&L.tk_arrive, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        while (__hip_atomic_load(&L.tk_arrive, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < nwk - 1) {
        }
        const unsigned mk = lane < nwk * K ? L.tk_key[lane] : 0u;
        const int mi = lane < nwk * K ? L.tk_idx[lane] : 0;
        wave_topk_merge(mk, mi, K, pk, pi);
        stamp(a, 15);
        finish_token(0, pi, unrank_bits(pk));
      }
    }
  } else {
    // one wave per token: lane l holds experts l, l+64, ...
    for (int t = wv; t < B; t += kFWaves) {
      int my_idx;
      float my_l;
      stamp(a, 14);
      auto pick = [&](auto ncc) {  // as many candidates per lane as E needs
        constexpr int NC = decltype(ncc)::value;
        float lv[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int e = lane + 64 * c;
          lv[c] = e < E ? L.u.logits[t * E + e] : 0.f;
        }
        wave_topk<NC>(lv, E, K, my_idx, my_l);
      };
      if (E <= 128) pick(std::integral_constant<int, 2>{});
      else if (E <= 256) pick(std::integral_constant<int, 4>{});
      else if (E <= 384) pick(std::integral_constant<int, 6>{});
      else pick(std::integral_constant<int, kFusedMaxE / 64>{});
      stamp(a, 15);
      finish_token(t, my_idx, my_l);
    }
  }
  if (B > 1) {  // several tokens: counted in parallel by all waves
    __syncthreads();
    stamp(a, 13);
    // per-expert lists.  Pick p = t*K + r has key e_p * 64 + t; pairs are
    // ordered by key (expert, then token), active experts ascending.  All
    // threads count, for pick p, the keys below its own and the picks of the
    // same expert in one eighth of the picks; wave 0 adds the eight parts,
    // places the pairs and marks each expert's first pair.
    {
      const int P = B * K;
      const int p = lane, part = wv, q0 = part * (kFusedMaxPairs / kFWaves);
      int lt = 0, same = 0;
      if (p < P) {
        const int ep = L.sel[p], kp = ep * 64 + p / K;
  #pragma unroll
        for (int i = 0; i < kFusedMaxPairs / kFWaves; ++i) {
          const int q = q0 + i;
          if (q < P) {
            const int eq = L.sel[q];
            lt += eq * 64 + q / K < kp;
            same += eq == ep;
          }
        }
      }
      L.part_lt[part][p] = lt;
      L.part_same[part][p] = same;
    }
    __syncthreads();
    if (wv == 0) {
      const int P = B * K;
      int rank = 0, same = 0;
  #pragma unroll
      for (int part = 0; part < kFWaves; ++part) {
        rank += L.part_lt[part][lane];
        same += L.part_same[part][lane];
      }
      if (lane < P) {
        const int ep = L.sel[lane];
        L.pair_tok[rank] = lane / K;
        L.pair_exp[rank] = ep;
        L.pair_w[rank] = L.selw[lane];
        L.pos[lane] = rank;
        L.part_same[0][rank] = same;   // count of the pair's expert, by sorted position
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
      __builtin_amdgcn_wave_barrier();
      const int r = lane;
      const int er = r < P ? L.pair_exp[r] : -1;
      const bool first = r < P && (r == 0 || L.pair_exp[r - 1] != er);
      const unsigned long long fm = __ballot(first);
      if (first) {
        const int slot = __popcll(fm & ((1ull << r) - 1ull));
        L.act_exp[slot] = er;
        L.act_cnt[slot] = L.part_same[0][r];
        L.act_off[slot] = r;
      }
      if (lane == 0) L.n_active = __popcll(fm);
    }
  }  // B > 1
  stamp(a, 12);
  __syncthreads();
  stamp(a, 8);
  // gate/up items: routed (active slot, ffn row) pairs, then the shared
  // expert's rows f >= fs_b that phase B did not take, in that order.  An
  // item costs 3 (in thirds of a one-token item); when the hg rows of its
  // tokens do not fit in LDS its activations come from the L2 with its
  // weights, in load batches whose depth falls with the token count, and it
  // costs 8 (3 or 4 tokens) or 10 (5 to 8), the times measured per item
  // against a one-token item; workgroup w
  // takes the items whose cost prefix lies in [w C / G, (w + 1) C / G), a
  // contiguous run of about equal cost, mostly rows of one expert.  With 8 or
  // more items in its run a workgroup stages the hg rows of each expert's
  // tokens in LDS once (when they fit) and its waves stream only weights.
  // Rounds of up to 4 items: waves 2i and 2i + 1 take both rows (W1 and W3)
  // of item i of the round over the two halves of K, so the item's
  // activation loads serve both rows.
  {
    const int n_rt = L.n_active * a.F;
    const int total = n_rt + (a.Fs - fs_b);
    const int nc = H >> 3, cmid = nc >> 1;
    const int cap = (int)(sizeof(L.u) / (4 * (size_t)H));  // tokens whose hg rows fit in LDS
    // per-slot item cost and its exclusive prefix over the slots (n_active <= 64 lanes)
    const int ns = L.n_active;
    auto item_cost = [&](int cnt) { return cnt <= cap ? 3 : cnt <= 4 ? 8 : 10; };
    const int cl = lane < ns ? item_cost(L.act_cnt[lane]) : 0;
    int incl = cl * a.F;
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += v;
    }
    const int excl = incl - cl * a.F;
    const int c_rt = __shfl(incl, kWave - 1, kWave);
    const int c_sh = item_cost(B);
    const long C = c_rt + (long)(a.Fs - fs_b) * c_sh;
    // the first item whose cost prefix is >= x
    auto first_item = [&](long x) -> int {
      if (x >= C) return total;
      if (x >= c_rt) return n_rt + (int)((x - c_rt + c_sh - 1) / c_sh);
      const int sl = __popcll(__ballot(lane < ns && excl <= x)) - 1;
      const int es = __shfl(excl, sl, kWave), cs = __shfl(cl, sl, kWave);
      return sl * a.F + (int)((x - es + cs - 1) / cs);
    };
    const int kb = first_item((long)w * C / G), ke = first_item((long)(w + 1) * C / G);
    // one token: its hg row is already in LDS (phase B or C) and every item reads it there
    const bool pre = B == 1;
    const bool stage = !pre && ke - kb >= 8;
    float *hl = pre ? reinterpret_cast<float *>(L.w2) : reinterpret_cast<float *>(&L.u);
    int staged = -2;  // token set in LDS: active slot, or -1 for the shared expert
    auto set_of = [&](int it) { return it < n_rt ? it / a.F : -1; };
    for (int k0 = kb; k0 < ke;) {
      const int sk0 = set_of(k0);
      int kend = min(ke, k0 + 4);
      if (stage)  // a staged round holds one expert's items
        for (int k = k0 + 1; k < kend; ++k)
          if (set_of(k) != sk0) {
            kend = k;
            break;
          }
      const int cnt0 = sk0 >= 0 ? L.act_cnt[sk0] : B;
      const bool lds = pre || (stage && cnt0 <= cap);  // this round's activations come from LDS
      if (lds && !pre && staged != sk0) {
        GuRow r0;
        r0.toks = sk0 >= 0 ? L.pair_tok + L.act_off[sk0] : nullptr;
        r0.cnt = cnt0;
        const int wpr = H >> 2, nw = r0.cnt * wpr;  // 16-byte words
        for (int q0 = tid; q0 < nw; q0 += 8 * kFT) {
          float4 v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int q = min(q0 + kFT * j, nw - 1), t = q / wpr, c = q % wpr;
            v[j] = ld16f(a.hg + (size_t)r0.tok(t) * H + 4 * c);
          }
          DL_SCHED_FENCE();
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int q = q0 + kFT * j;
            if (q < nw) *reinterpret_cast<float4 *>(hl + 4 * q) = v[j];
          }
        }
        __syncthreads();
        staged = sk0;
      }
      const int ki = k0 + (wv >> 1), hf = wv & 1;
      if (ki < kend) {
        const int it = ki, sk = set_of(it);
        GuRow r;
        const uint16_t *row1, *row3;
        if (sk >= 0) {
          const size_t ro = ((size_t)L.act_exp[sk] * a.F + it % a.F) * H;
          row1 = a.w1 + ro;
          row3 = a.w3 + ro;
          r.toks = L.pair_tok + L.act_off[sk];
          r.cnt = L.act_cnt[sk];
        } else {
          const size_t ro = (size_t)(fs_b + it - n_rt) * H;
          row1 = a.s1 + ro;
          row3 = a.s3 + ro;
          r.toks = nullptr;
          r.cnt = B;
        }
        by_tokens(r.cnt, [&](auto ntc) {
          constexpr int NT = decltype(ntc)::value;
          float su[NT], sv[NT];
          if (lds)
            gateup_pair_lds<NT>(row1, row3, hl, r.cnt, H, hf ? cmid : 0, hf ? nc : cmid, su, sv);
          else
            gateup_pair<NT>(r, row1, row3, a.hg, H, hf ? cmid : 0, hf ? nc : cmid, su, sv);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (lane == t) {
              L.uv[wv >> 1][hf][0][t] = su[t];
              L.uv[wv >> 1][hf][1][t] = sv[t];
            }
          }
        });
      }
      __syncthreads();
      // combine: thread (item-in-round is, token j)
      const int is = tid >> 3, j = tid & 7;
      if (is < kend - k0) {
        const int it = k0 + is, sk = set_of(it);
        const float su = L.uv[is][0][0][j] + L.uv[is][1][0][j];
        const float sv = L.uv[is][0][1][j] + L.uv[is][1][1][j];
        if (sk >= 0) {
          const int f2 = it % a.F;
          const int c2 = L.act_cnt[sk], o2 = L.act_off[sk];
          if (j < c2) {
            const int t = L.pair_tok[o2 + j];
            put_tagged(a.act + (size_t)(o2 + j) * a.F + f2,
                       poison_c ? kNaN : silu_mul(su * L.inv_rms[t], sv * L.inv_rms[t]), tag);
          }
        } else if (j < B) {
          put_tagged(a.act_s + (size_t)j * a.Fs + (fs_b + it - n_rt),
                     poison_c ? kNaN : silu_mul(su * L.inv_rms[j], sv * L.inv_rms[j]), tag);
        }
      }
      __syncthreads();
      k0 = kend;
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
      if (!ctl) {
        d.stage();   // the first down-projection rows (static weights) -> LDS
      } else {
        if (split_topk && wv == 0) {  // the one token's deferred pick weights
          const float wgt = pick_weights(lane < K ? L.selw[lane] : 0.f, K);
          if (lane < K) {
            L.pair_w[L.pos[lane]] = wgt;
            if (w == 0) a.topk_w[lane] = poison_c ? kNaN : wgt;
          }
        }
        // every SwiGLU activation -> LDS
        gather_tagged(a.act, L.u.d.act, tid, kCtl, P * a.F, tag, a.spin_limit, &L.bad);
        gather_tagged(a.act_s, L.u.d.act_s, tid, kCtl, B * a.Fs, tag, a.spin_limit, &L.bad);
      }
      __syncthreads();
      stamp(a, 10);
      d.compute();
    });
    __syncthreads();
    const bool poison_d = L.bad != 0;
    for (int q = tid; q < B * ni; q += kFT) {
      const int t = q / ni, il = q % ni;
      float y = a.Fs > 0 ? L.u.d.contrib[t * kFusedMaxSlice + il] : 0.f;
      for (int r = 0; r < K; ++r) y += L.u.d.contrib[(B + L.pos[t * K + r]) * kFusedMaxSlice + il];
      a.moe_out[(size_t)t * H + i0 + il] = poison_d ? kNaN : y;
    }
  }
  stamp(a, 11);
  __syncthreads();
  if (tag == 0xffffffffu) {
    // the last tag before the wrap: once every workgroup is past its last
    // read of this step (a grid barrier on a monotonic arrival count), each
    // clears its share of the hand-off slots back to tag 0
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(a.wrap, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned target = (prev / (unsigned)G + 1u) * (unsigned)G;
      for (int n = 0; __hip_atomic_load(a.wrap, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++n) {
        if (n >= a.spin_limit) {
          L.bad = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    for (size_t i = (size_t)w * kFT + tid; i < a.tag_words; i += (size_t)G * kFT)
      __hip_atomic_store(a.tag_base + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  stamp(a, 3);
  if (pf_acc == 0x9e3779b9u && a.B < 0) a.status[0] = pf_acc;  // never true: keeps the prefetch loads
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
