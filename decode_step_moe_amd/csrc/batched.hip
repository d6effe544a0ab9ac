// The layer-step for batches of up to 64 tokens, as five launches.
//
// At tens of tokens an expert is shared by many tokens (the hot-expert case:
// 64 tokens over 32 experts, 16 tokens each), and a row-at-a-time GEMV that
// re-reads every token's activations for every 16 bytes of weights runs out
// of vector issue long before HBM runs out of bandwidth.  Every contraction
// whose weights are shared by 16 or more tokens therefore runs on the matrix
// cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation); experts with fewer
// tokens keep the VALU GEMV.  The decode step is the same as in the
// single-launch kernel (wireai.ir "vLLM's speed jump on NVIDIA Blackwell
// servers; record 842 tokens/s for Kimi K3", section "Four key changes behind
// the jump", bullets 1-3: input projection, out-projection into the residual
// and norm, router before the shared and routed experts).
//
// Launches (all on the caller's stream; data passes through L2/HBM):
//  1 proj_b    Wo tiles of 16 rows, K = Do split over the 4 waves:
//                r1 = r + attn Wo^T -> resid_out, hg = g r1, per-workgroup
//                sums of r1^2.
//              Wqkv tiles of 16 rows, K = H split over 4 workgroups x 4 waves:
//                partial qkv sums.
//  2 router_b  fp32 router dot products d[t, e] = hg[t] . Wr[e] on MFMA
//              (v_mfma_f32_16x16x4_f32), 32 experts x 256 K per workgroup;
//              also sums the qkv partials (fixed order) -> qkv.
//  3 topk_b    one workgroup per token: 1/rms, h = hg / rms (fp32 and bf16
//              hi + lo planes), logits l = d / rms, top-k by repeated wave
//              arg-max (descending, ties to the lower expert id), weights
//              s / sum s with s = sigmoid(l).  The last workgroup to finish
//              builds the per-expert token lists (active experts ascending,
//              tokens ascending inside an expert).
//  4 gateup_b  a[p, f] = silu(W1[e, f] . h[t_p]) * (W3[e, f] . h[t_p]):
//              matrix-core units (64 rows of W1 and W3 x a 16-token chunk
//              x a K chunk) cut into one contiguous run per workgroup, two
//              workgroups per CU, K chunks combined by the last to arrive;
//              then the VALU items of experts with fewer than 16 tokens.
//  5 down_b    16 rows of y per workgroup over every active expert and the
//              shared expert, summed in a fixed order in LDS:
//              y[t, i] = S2[i] . a_s[t] + sum_p w_p W2[e_p, i] . a[p].
//
// MFMA operands.  x, attn and the weights are bf16 already.  h and the SwiGLU
// activations are fp32; each is split as x = hi + lo with hi = x truncated
// to bf16 (x - hi is exact) and lo = bf16(x - hi), and both halves are
// multiplied into the same accumulator, which keeps about 16 significant
// bits of x (relative error below 2^-16) against the weights' exact bf16.
//
// Weight loads.  A matrix-core operand fragment is 16 rows x 64 bytes per
// load instruction (the next 64 bytes of each row follow in the next K
// step), and these kernels read weights with ordinary cached loads: on this
// pattern they stream measurably faster than non-temporal loads.
//
// Every output element is produced by one thread, in an order that depends
// only on the shapes, so results are bit-identical from run to run.
#include "common.h"
#include "kernels.h"

namespace dl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Lane layout of v_mfma_f32_16x16x32_bf16 (lane l, n = l % 16, g = l / 16):
// A[n][8g + j] and B[8g + j][n] for j < 8 (8 consecutive K values, one
// 16-byte load from a K-contiguous row), D[4g + i][n] for i < 4.
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
  v4u u = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x4 mfma_bf16(const uint4 &a, const uint4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {  // round to nearest even
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}
// x = hi + lo as two packed bf16 octets (element j in bits 16j.. of the octet).
__device__ __forceinline__ void split8(const float (&x)[8], uint4 &hi, uint4 &lo) {
  unsigned h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned ua = __float_as_uint(x[2 * j]) & 0xffff0000u;
    const unsigned ub = __float_as_uint(x[2 * j + 1]) & 0xffff0000u;
    h[j] = (ua >> 16) | ub;
    l[j] = pack_bf16(x[2 * j] - __uint_as_float(ua), x[2 * j + 1] - __uint_as_float(ub));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}
__device__ __forceinline__ void load8f(const float *p, float (&x)[8]) {
  const float4 u = ld16f(p), v = ld16f(p + 4);
  x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
  x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
}

// One wave: acc[c] += A_c (16 x 32 nks) . W^T (32 nks x 16) with bf16 A rows
// at ap[c] and weight rows at wp (both already offset by this lane's row and
// its 8g K position).  U K-steps of loads per batch; the K-steps of the last
// batch beyond nks re-read step nks-1 and multiply zero weights.
template <int NC, int U>
__device__ __forceinline__ void mfma_rows(const uint16_t *wp, const uint16_t *const (&ap)[NC], int nks,
                                          f32x4 (&acc)[NC]) {
  for (int ks = 0; ks < nks; ks += U) {
    uint4 wv[U], av[U][NC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(ks + u, nks - 1) * 32;
      wv[u] = ld16(wp + k);
#pragma unroll
      for (int c = 0; c < NC; ++c) av[u][c] = ld16(ap[c] + k);
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint4 w = zero_unless(ks + u < nks, wv[u]);
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = mfma_bf16(av[u][c], w, acc[c]);
    }
  }
}

template <class Fn>
__device__ __forceinline__ void by_chunks(int nc, Fn fn) {
  switch (nc) {
    case 1: fn(std::integral_constant<int, 1>{}); break;
    case 2: fn(std::integral_constant<int, 2>{}); break;
    case 3: fn(std::integral_constant<int, 3>{}); break;
    default: fn(std::integral_constant<int, 4>{}); break;
  }
}

// ================================================================ launch 1
// red[w][token][n]: wave w's share of output (token, row r0 + n).
__global__ void __launch_bounds__(kBlock) proj_b(BatchArgs a, int n_wo) {
  __shared__ float red[kWavesPerBlock][kMaxBatch][16];
  __shared__ float sq[kMaxBatch][16];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int B = a.B;
  const bool wo = (int)blockIdx.x < n_wo;
  int r0, split = 0, nks, ld;
  const uint16_t *wp, *abase;
  if (wo) {
    r0 = blockIdx.x * 16;
    const int kw = wv * (a.Do / 4) + 8 * g;
    wp = a.w_o + (size_t)(r0 + n) * a.Do + kw;
    abase = a.attn + kw;
    ld = a.Do;
    nks = a.Do / 128;
  } else {
    const int b = blockIdx.x - n_wo;
    r0 = (b / kBatchQkvSplit) * 16;
    split = b % kBatchQkvSplit;
    const int kq = a.H / (kBatchQkvSplit * kWavesPerBlock);
    const int kw = split * (a.H / kBatchQkvSplit) + wv * kq + 8 * g;
    wp = a.w_qkv + (size_t)min(r0 + n, a.Dq - 1) * a.H + kw;
    abase = a.x + kw;
    ld = a.H;
    nks = kq / 32;
  }
  by_chunks((B + 15) >> 4, [&](auto ncc) {
    constexpr int NC = decltype(ncc)::value;
    const uint16_t *ap[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) ap[c] = abase + (size_t)min(16 * c + n, B - 1) * ld;
    f32x4 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_rows<NC, (NC <= 2 ? 8 : 4)>(wp, ap, nks, acc);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wv][16 * c + 4 * g + i][n] = acc[c][i];
  });
  __syncthreads();
  if (wo) {
    for (int q = tid; q < B * 16; q += kBlock) {
      const int t = q >> 4, nn = q & 15, i = r0 + nn;
      const float s = ((red[0][t][nn] + red[1][t][nn]) + red[2][t][nn]) + red[3][t][nn];
      const size_t o = (size_t)t * a.H + i;
      const float r1 = a.resid_in[o] + s;
      a.resid_out[o] = r1;
      a.hg[o] = bf16_lo(a.gain[i]) * r1;
      sq[t][nn] = r1 * r1;
    }
    __syncthreads();
    if (tid < B) {
      float s = 0.f;
      for (int nn = 0; nn < 16; ++nn) s += sq[tid][nn];
      a.ss_part[(size_t)blockIdx.x * B + tid] = s;
    }
  } else {
    for (int q = tid; q < B * 16; q += kBlock) {
      const int t = q >> 4, nn = q & 15, j = r0 + nn;
      if (j < a.Dq)
        a.qkv_part[((size_t)split * B + t) * a.Dq + j] =
            ((red[0][t][nn] + red[1][t][nn]) + red[2][t][nn]) + red[3][t][nn];
    }
  }
}

// ================================================================ launch 2
// Lane layout of v_mfma_f32_16x16x4_f32: A[n][g], B[g][n], D[4g + i][n].
// The K axis is permuted the same way for both operands so that every lane
// reads 4 consecutive fp32 values: at sub-step s, MFMA K index g stands for
// k = kb + 4g + s.
__global__ void __launch_bounds__(kBlock) router_b(BatchArgs a) {
  __shared__ float red[kWavesPerBlock][4 * 2 * 256];  // [wave][chunk][tile][m * 16 + n]
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int B = a.B, H = a.H, E = a.E;
  const int e0 = blockIdx.x * kBatchRtrExperts, ky = blockIdx.y;
  const int kb = ky * kBatchRtrK + wv * (kBatchRtrK / kWavesPerBlock) + 4 * g;
  const float *w0 = a.w_router + (size_t)min(e0 + n, E - 1) * H + kb;
  const float *w1 = a.w_router + (size_t)min(e0 + 16 + n, E - 1) * H + kb;
  by_chunks((B + 15) >> 4, [&](auto ncc) {
    constexpr int NC = decltype(ncc)::value;
    float4 b0[4], b1[4], av[4][NC];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      b0[it] = ld16f(w0 + 16 * it);
      b1[it] = ld16f(w1 + 16 * it);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float *ap = a.hg + (size_t)min(16 * c + n, B - 1) * H + kb;
#pragma unroll
      for (int it = 0; it < 4; ++it) av[it][c] = ld16f(ap + 16 * it);
    }
    DL_SCHED_FENCE();
    f32x4 acc[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c][0] = acc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float wa[4] = {b0[it].x, b0[it].y, b0[it].z, b0[it].w};
      const float wb[4] = {b1[it].x, b1[it].y, b1[it].z, b1[it].w};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float x[4] = {av[it][c].x, av[it][c].y, av[it][c].z, av[it][c].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc[c][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], wa[s], acc[c][0], 0, 0, 0);
          acc[c][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], wb[s], acc[c][1], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wv][(c * 2 + nt) * 256 + (4 * g + i) * 16 + n] = acc[c][nt][i];
  });
  __syncthreads();
  for (int q = tid; q < B * kBatchRtrExperts; q += kBlock) {
    const int t = q >> 5, el = q & 31;
    const int idx = ((t >> 4) * 2 + (el >> 4)) * 256 + (t & 15) * 16 + (el & 15);
    if (e0 + el < E)
      a.rlog_part[((size_t)ky * B + t) * E + e0 + el] =
          ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
  }
  // qkv = sum of the K-split partials, spread over the grid
  const int nblk = gridDim.x * gridDim.y, bl = blockIdx.y * gridDim.x + blockIdx.x;
  const size_t nq = (size_t)B * a.Dq, plane = nq;
  for (size_t q = (size_t)bl * kBlock + tid; q < nq; q += (size_t)nblk * kBlock) {
    const float *p = a.qkv_part + q;
    a.qkv[q] = ((p[0] + p[plane]) + p[2 * plane]) + p[3 * plane];
  }
}

// ================================================================ launch 3
__global__ void __launch_bounds__(kBlock) topk_b(BatchArgs a, int n_ow, int n_rk) {
  __shared__ float lg[kMaxExperts];
  __shared__ float wred[kWavesPerBlock];
  __shared__ int cnt[kMaxExperts], off[kMaxExperts];
  __shared__ unsigned msk[kMaxExperts][2];
  __shared__ int sa[kBlock], sc[kBlock];
  __shared__ int slot_nch[kMaxExperts];
  __shared__ int last_flag;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int B = a.B, H = a.H, E = a.E, K = a.K, t = blockIdx.x;
  // 1/rms from the out-projection workgroups' partial sums
  float ss = 0.f;
  for (int q = tid; q < n_ow; q += kBlock) ss += a.ss_part[(size_t)q * B + t];
  ss = wave_sum(ss);
  if (lane == 0) wred[wv] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf(((wred[0] + wred[1]) + (wred[2] + wred[3])) / (float)H + a.eps);
  // h = hg / rms: fp32 copy, optional output, bf16 hi/lo planes
  for (int i = tid * 8; i < H; i += kBlock * 8) {
    const size_t o = (size_t)t * H + i;
    float x[8];
    load8f(a.hg + o, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= inv;
    const float4 u = make_float4(x[0], x[1], x[2], x[3]), v = make_float4(x[4], x[5], x[6], x[7]);
    *reinterpret_cast<float4 *>(a.hn + o) = u;
    *reinterpret_cast<float4 *>(a.hn + o + 4) = v;
    if (a.h_out) {
      *reinterpret_cast<float4 *>(a.h_out + o) = u;
      *reinterpret_cast<float4 *>(a.h_out + o + 4) = v;
    }
    uint4 hi, lo;
    split8(x, hi, lo);
    *reinterpret_cast<uint4 *>(a.hp + o) = hi;
    *reinterpret_cast<uint4 *>(a.hp + (size_t)B * H + o) = lo;
  }
  // logits: K chunks summed in ascending order, then scaled
  for (int e = tid; e < E; e += kBlock) {
    float d = 0.f;
    const float *p = a.rlog_part + (size_t)t * E + e;
    const size_t stride = (size_t)B * E;
    for (int ky0 = 0; ky0 < n_rk; ky0 += 8) {  // 8 independent loads per batch
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p[min(ky0 + j, n_rk - 1) * stride];
#pragma unroll
      for (int j = 0; j < 8; ++j) d += ky0 + j < n_rk ? v[j] : 0.f;
    }
    const float l = d * inv;
    lg[e] = l;
    if (a.logits_out) a.logits_out[(size_t)t * E + e] = l;
  }
  __syncthreads();
  if (wv == 0) {  // lane holds experts lane, lane + 64, ...
    constexpr int NCAND = kMaxExperts / kWave;
    float lv[NCAND];
#pragma unroll
    for (int c = 0; c < NCAND; ++c) {
      const int e = lane + 64 * c;
      lv[c] = e < E ? lg[e] : 0.f;
    }
    int my_idx;
    float my_l;
    wave_topk<NCAND>(lv, E, K, my_idx, my_l);
    const float s = lane < K ? 1.0f / (1.0f + expf(-my_l)) : 0.f;
    const float ssum = wave_sum(s);
    if (lane < K) {  // written through: the last workgroup reads them back
      __hip_atomic_store(a.topk_idx + (size_t)t * K + lane, my_idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.topk_w + (size_t)t * K + lane, s / ssum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!arrive_last_wt(a.counter, B, &last_flag)) return;

  // ---- the last workgroup: per-expert token lists ----
  for (int q = tid; q < E; q += kBlock) {
    cnt[q] = 0;
    msk[q][0] = msk[q][1] = 0u;
  }
  __syncthreads();
  const int P = B * K;
  for (int i = tid; i < P; i += kBlock) {
    const int e = __hip_atomic_load(a.topk_idx + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), tt = i / K;
    atomicAdd(&cnt[e], 1);
    atomicOr(&msk[e][tt >> 5], 1u << (tt & 31));
  }
  __syncthreads();
  // exclusive scans over experts: active-slot index and pair offset
  const int seg = (E + kBlock - 1) / kBlock;
  const int q0 = tid * seg, q1 = min(E, q0 + seg);
  int la = 0, lc = 0;
  for (int q = q0; q < q1; ++q) { la += cnt[q] > 0; lc += cnt[q]; }
  sa[tid] = la;
  sc[tid] = lc;
  __syncthreads();
  for (int o = 1; o < kBlock; o <<= 1) {
    const int va = tid >= o ? sa[tid - o] : 0, vc = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sa[tid] += va;
    sc[tid] += vc;
    __syncthreads();
  }
  int pa = sa[tid] - la, pc = sc[tid] - lc;
  for (int q = q0; q < q1; ++q) {
    const int c = cnt[q];
    off[q] = pc;
    if (c > 0) {
      a.act_exp[pa] = q;
      a.act_cnt[pa] = c;
      a.act_off[pa] = pc;
      // gate/up work per slot: 16-token chunks on the matrix cores, else one VALU entry
      slot_nch[pa] = c >= kBatchMfmaMin ? (c + 15) >> 4 : 0;
      ++pa;
      pc += c;
    }
  }
  const int n_act = sa[kBlock - 1];
  if (tid == kBlock - 1) *a.n_active = n_act;
  __syncthreads();
  // gate/up work lists: matrix-core entries (slot, 16-token chunk), then VALU
  // entries (slot, all of its fewer than 16 tokens); slots ascending in each
  {
    const int seg2 = (n_act + kBlock - 1) / kBlock;
    const int s0 = tid * seg2, s1 = min(n_act, s0 + seg2);
    int lm = 0, lv = 0;
    for (int q = s0; q < s1; ++q) {
      lm += slot_nch[q];
      lv += slot_nch[q] == 0;
    }
    sa[tid] = lm;
    sc[tid] = lv;
    __syncthreads();
    for (int o = 1; o < kBlock; o <<= 1) {
      const int vm = tid >= o ? sa[tid - o] : 0, vv = tid >= o ? sc[tid - o] : 0;
      __syncthreads();
      sa[tid] += vm;
      sc[tid] += vv;
      __syncthreads();
    }
    const int n_qm = sa[kBlock - 1], n_qv = sc[kBlock - 1];
    int pm = sa[tid] - lm, pv = n_qm + sc[tid] - lv;
    for (int q = s0; q < s1; ++q) {
      for (int c = 0; c < slot_nch[q]; ++c) a.gu_q[pm++] = q | (c << 16);
      if (slot_nch[q] == 0) a.gu_q[pv++] = q;
    }
    if (tid == kBlock - 1) {
      a.n_q[0] = n_qm;
      a.n_q[1] = n_qv;
    }
  }
  __syncthreads();
  // a pair's place inside its expert = number of lower tokens with that expert
  for (int i = tid; i < P; i += kBlock) {
    const int e = __hip_atomic_load(a.topk_idx + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), tt = i / K;
    const unsigned m0 = msk[e][0], m1 = msk[e][1];
    const int r = tt < 32 ? __popc(m0 & ((1u << tt) - 1u)) : __popc(m0) + __popc(m1 & ((1u << (tt - 32)) - 1u));
    const int pos = off[e] + r;
    a.pair_tok[pos] = tt;
    a.pair_w[pos] = __hip_atomic_load(a.topk_w + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ================================================================ launch 4
struct GuItem {
  const uint16_t *w1, *w3;  // first of the item's 16 rows, row stride H
  const int *toks;          // token of row m (nullptr: tok0 + m)
  int tok0;
  float *out;               // row m of the output at out + m * ld, 16 columns
  int ld, cnt;              // cnt <= 16 rows on the matrix cores, < 16 on the VALU
  __device__ int tok(int m) const { return toks ? toks[m] : tok0 + m; }
};

// Fewer than 16 tokens: wave w takes rows 4w .. 4w+3 of the item, one
// (W1 row, W3 row) pair at a time over the full K, up to 8 tokens per pass.
__device__ void gateup_valu(const BatchArgs &a, const GuItem &it) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H;
  for (int t0 = 0; t0 < it.cnt; t0 += 8) {
    const int nt = min(8, it.cnt - t0);
    auto pass = [&](auto ntc) {
      constexpr int NT = decltype(ntc)::value;
      constexpr int CPB = NT <= 2 ? 4 : NT <= 4 ? 2 : 1;
      HgGather<NT> act;
      act.base = a.hn;
      act.ld = H;
#pragma unroll
      for (int t = 0; t < NT; ++t) act.tok[t] = it.tok(t0 + min(t, nt - 1));
      for (int r = 0; r < 4; ++r) {
        const int f = 4 * wv + r;
        const uint16_t *w[2] = {it.w1 + (size_t)f * H, it.w3 + (size_t)f * H};
        float o[2][NT];
        wave_rows_dot<2, NT, CPB>(w, 0, H / 8, act, o);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (lane == t && t < nt) it.out[(size_t)(t0 + t) * it.ld + f] = silu_mul(o[0][t], o[1][t]);
      }
    };
    if (nt == 1) pass(std::integral_constant<int, 1>{});
    else if (nt == 2) pass(std::integral_constant<int, 2>{});
    else if (nt <= 4) pass(std::integral_constant<int, 4>{});
    else pass(std::integral_constant<int, 8>{});
  }
}

// Matrix-core units.  A group is 16 NTL rows (NTL <= 4) of W1 and the same
// rows of W3 applied to one 16-token chunk: a chunk of a routed expert with
// 16 or more tokens, or of the shared expert when B >= 16.  A unit is one
// group over kGuKc K steps of 32 (448 K elements at H = 7168; a group has
// ceil(H / (32 kGuKc)) units, its K chunks).  The workgroup stages the
// chunk's activations for the unit's K range (bf16 hi and lo planes of h)
// in LDS with contiguous loads; wave w < NTL then streams the 16 rows of
// tile w of W1 and of W3, 7 K steps (448 bytes of each row) per load batch,
// taking its activation fragments from LDS.  The sums go to the group's
// slot for that K chunk, written through to the device coherence point; the
// last unit of the group to arrive adds the slots in K-chunk order (so the
// result does not depend on arrival order) and writes silu(u) * v.
// VALU units.  (expert, 16-row tile) of experts with fewer than 16 tokens,
// and of the shared expert below 16 tokens, after the matrix-core units.
constexpr int kGuPad = 8;                  // bf16 elements of padding per LDS row
constexpr int kGuLd = 32 * kGuKc + kGuPad; // LDS row of one staged token
constexpr int kGuLds = 2 * 16 * kGuLd * 2; // bytes: [hi | lo][16 tokens][kGuLd]
constexpr unsigned kGuSc1 = 16;            // cache policy: coherent at agent scope

struct GuUnit {
  const uint16_t *w1, *w3;  // row 0 of the group, row stride H
  float *out;               // output row m at out + m * ld, columns [0, 16 NTL)
  float *slots;             // the group's slots, kGuSlotFloatsR floats each
  unsigned *arrivals;       // the group's arrival counter
  int ld, cnt, k0, k1, kc, nck, ntl, group;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gu_rsrc(const float *p, int floats) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, floats * 4, 0x00020000);
}

// One matrix-core unit: sums over its K chunk into its slot, as
// [W1 | W3][tile][row][token] (a lane's 4 tokens are contiguous).
template <int NTL>
__device__ void gu_unit(const BatchArgs &a, const GuUnit &s, const uint16_t *lds) {
  constexpr int U = 7;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  if (wv >= NTL) return;
  const int H = a.H, kb = 32 * s.k0, nks = s.k1 - s.k0;
  const uint16_t *p1 = s.w1 + (size_t)(16 * wv + n) * H + kb + 8 * g;
  const uint16_t *p3 = s.w3 + (size_t)(16 * wv + n) * H + kb + 8 * g;
  const uint16_t *lh = lds + n * kGuLd + 8 * g, *ll = lh + 16 * kGuLd;
  f32x4 acc1 = {0.f, 0.f, 0.f, 0.f}, acc3 = acc1;
  for (int ks = 0; ks < nks; ks += U) {
    uint4 w1v[U], w3v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(ks + u, nks - 1) * 32;
      w1v[u] = ld16(p1 + k);
      w3v[u] = ld16(p3 + k);
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(ks + u, nks - 1) * 32;
      const bool on = ks + u < nks;
      const uint4 b1 = zero_unless(on, w1v[u]), b3 = zero_unless(on, w3v[u]);
      const uint4 hv = *reinterpret_cast<const uint4 *>(lh + k), lv = *reinterpret_cast<const uint4 *>(ll + k);
      acc1 = mfma_bf16(hv, b1, acc1);
      acc3 = mfma_bf16(hv, b3, acc3);
      acc1 = mfma_bf16(lv, b1, acc1);
      acc3 = mfma_bf16(lv, b3, acc3);
    }
  }
  const __amdgpu_buffer_rsrc_t r = gu_rsrc(s.slots, s.nck * kGuSlotFloatsR);
  const int base = s.kc * kGuSlotFloatsR + (wv * 16 + n) * 16 + 4 * g;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc1), r, base * 4, 0, kGuSc1);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc3), r, (base + NTL * 256) * 4, 0, kGuSc1);
}

// The group's last unit: u and v summed over the K-chunk slots in order.
template <int NTL>
__device__ void gu_combine(const GuUnit &s) {
  constexpr int ROWS = 16 * NTL;
  const int q = threadIdx.x;
  if (q >= ROWS * 4) return;
  const int r = q % ROWS, mq = q / ROWS, t = r >> 4, nn = r & 15;
  const __amdgpu_buffer_rsrc_t rs = gu_rsrc(s.slots, s.nck * kGuSlotFloatsR);
  const int i1 = ((0 * NTL + t) * 16 + nn) * 16 + 4 * mq, i3 = ((NTL + t) * 16 + nn) * 16 + 4 * mq;
  f32x4 u = {0.f, 0.f, 0.f, 0.f}, v = u;
  for (int s0 = 0; s0 < s.nck; s0 += 8) {
    f32x4 pu[8], pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int o = min(s0 + j, s.nck - 1) * kGuSlotFloatsR;
      pu[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (o + i1) * 4, 0, kGuSc1));
      pv[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (o + i3) * 4, 0, kGuSc1));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < s.nck) {
        u += pu[j];
        v += pv[j];
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * mq + i;
    if (m < s.cnt) s.out[(size_t)m * s.ld + r] = silu_mul(u[i], v[i]);
  }
}

// The staged activations of one unit: 16-byte words of [hi | lo][token][K].
constexpr int kGuStW = (2 * 16 * (32 * kGuKc / 8) + kBlock - 1) / kBlock;  // words per thread

__device__ __forceinline__ int gu_token(const int *toks, int tok0, int m, int cnt) {
  m = min(m, cnt - 1);
  return toks ? toks[m] : tok0 + m;
}

__device__ __forceinline__ void gu_stage_load(const BatchArgs &a, const int *tok_l, const GuUnit &s,
                                              uint4 (&st)[kGuStW]) {
  const int kbeg = 32 * s.k0, wpr = 4 * (s.k1 - s.k0), nw = 32 * wpr;
  const size_t plane = (size_t)a.B * a.H;
#pragma unroll
  for (int j = 0; j < kGuStW; ++j) {
    const int w = min((int)threadIdx.x + kBlock * j, nw - 1);
    const int pl = w / (16 * wpr), m = (w / wpr) & 15, c = w % wpr;
    st[j] = ld16(a.hp + pl * plane + (size_t)tok_l[m] * a.H + kbeg + 8 * c);
  }
}

__device__ __forceinline__ void gu_stage_store(const uint4 (&st)[kGuStW], const GuUnit &s, uint16_t *lds) {
  const int wpr = 4 * (s.k1 - s.k0), nw = 32 * wpr;
#pragma unroll
  for (int j = 0; j < kGuStW; ++j) {
    const int w = (int)threadIdx.x + kBlock * j;
    if (w < nw) {
      const int pl = w / (16 * wpr), m = (w / wpr) & 15, c = w % wpr;
      *reinterpret_cast<uint4 *>(lds + (pl * 16 + m) * kGuLd + 8 * c) = st[j];
    }
  }
}

struct GuGeom {
  int NK, NCK, F, Fs, B, rg_r, ngr, rg_s, ng_r, nch_s;
};

// Unit u: its group's weights, output, slots and tokens (toks[m], or tok0 + m).
__device__ __forceinline__ void gu_meta(const BatchArgs &a, const GuGeom &q, int u, GuUnit &s, const int *&toks,
                                        int &tok0) {
  const int gi = u / q.NCK, H = a.H;
  s.group = gi;
  s.nck = q.NCK;
  if (gi < q.ng_r) {
    const int e = gi / q.ngr, r0 = (gi % q.ngr) * q.rg_r;
    const int qe = a.gu_q[e], slot = qe & 0xffff, c0 = 16 * (qe >> 16);
    const int ex = a.act_exp[slot], off = a.act_off[slot] + c0;
    s.w1 = a.w1 + ((size_t)ex * q.F + r0) * H;
    s.w3 = a.w3 + ((size_t)ex * q.F + r0) * H;
    s.cnt = min(16, a.act_cnt[slot] - c0);
    s.out = a.act + (size_t)off * q.F + r0;
    s.ld = q.F;
    s.ntl = q.rg_r >> 4;
    s.slots = a.gu_part + (size_t)gi * q.NCK * kGuSlotFloatsR;
    s.arrivals = a.gu_cnt + gi;
    toks = a.pair_tok + off;
    tok0 = 0;
  } else {
    const int gs = gi - q.ng_r, r0 = (gs / q.nch_s) * q.rg_s, c = gs % q.nch_s;
    s.w1 = a.s1 + (size_t)r0 * H;
    s.w3 = a.s3 + (size_t)r0 * H;
    s.cnt = min(16, q.B - 16 * c);
    s.out = a.act_s + (size_t)(16 * c) * q.Fs + r0;
    s.ld = q.Fs;
    s.ntl = q.rg_s >> 4;
    s.slots = a.gu_part_s + (size_t)gs * q.NCK * kGuSlotFloatsR;
    s.arrivals = a.gu_cnt_s + gs;
    toks = nullptr;
    tok0 = 16 * c;
  }
}

__device__ __forceinline__ void gu_chunk(GuUnit &s, int u, int NK) {
  s.kc = u % s.nck;
  s.k0 = s.kc * kGuKc;
  s.k1 = min(NK, s.k0 + kGuKc);
}

// Matrix-core units laid end to end (group by group, K chunks in order) are
// cut into one contiguous run per workgroup (two workgroups per CU), so
// consecutive units of a workgroup mostly share a group and its tokens.
// While a unit streams its weights, the next unit's activations are loaded
// into registers and then written to the other LDS buffer, so staging does
// not stall the weight stream.  VALU units are dealt round-robin after.
__global__ void __launch_bounds__(kBlock, 2) gateup_b(BatchArgs a) {
  __shared__ __align__(16) uint16_t lds[2][kGuLds / 2];
  __shared__ int tok_l[2][16];
  __shared__ int s_flag;
  const int tid = threadIdx.x;
  const int n_qm = a.n_q[0], n_qv = a.n_q[1];
  GuGeom q;
  q.B = a.B;
  q.F = a.F;
  q.Fs = a.Fs;
  q.NK = a.H >> 5;
  q.NCK = (q.NK + kGuKc - 1) / kGuKc;
  const bool s_mfma = q.Fs > 0 && q.B >= kBatchMfmaMin;
  q.nch_s = s_mfma ? (q.B + 15) >> 4 : 0;
  q.rg_r = min(kBatchGuRows, q.F);
  q.ngr = q.F / q.rg_r;
  q.rg_s = q.Fs > 0 ? min(kBatchGuRows, q.Fs) : 16;
  q.ng_r = n_qm * q.ngr;
  const int ng = q.ng_r + q.nch_s * (q.Fs / q.rg_s);
  const int n_mfma = ng * q.NCK;
  const int G = gridDim.x, w = blockIdx.x;
  // workgroups w and w + G/2 are dispatched to the same CU: give them
  // neighbouring runs, so that every CU holds the same number of units
  const int half = G >> 1, r = (G & 1) ? w : 2 * (w % half) + w / half;
  const int ub = (int)((long)r * n_mfma / G), ue = (int)((long)(r + 1) * n_mfma / G);
  if (ub < ue) {
    GuUnit cur;
    const int *toks;
    int tok0;
    gu_meta(a, q, ub, cur, toks, tok0);
    gu_chunk(cur, ub, q.NK);
    if (tid < 16) tok_l[0][tid] = gu_token(toks, tok0, tid, cur.cnt);
    __syncthreads();
    {
      uint4 st[kGuStW];
      gu_stage_load(a, tok_l[0], cur, st);
      gu_stage_store(st, cur, lds[0]);
    }
    __syncthreads();
    int b = 0;
    for (int u = ub; u < ue; ++u) {
      const bool more = u + 1 < ue;
      GuUnit nx = cur;
      if (more) {
        if ((u + 1) % q.NCK == 0) {  // the next unit starts a new group
          gu_meta(a, q, u + 1, nx, toks, tok0);
          if (tid < 16) tok_l[b ^ 1][tid] = gu_token(toks, tok0, tid, nx.cnt);
        } else if (tid < 16) {
          tok_l[b ^ 1][tid] = tok_l[b][tid];
        }
        gu_chunk(nx, u + 1, q.NK);
      }
      __syncthreads();
      uint4 st[kGuStW];
      if (more) gu_stage_load(a, tok_l[b ^ 1], nx, st);
      asm volatile("" ::: "memory");  // issue the staging loads ahead of the weight stream
      if (cur.ntl == 4) gu_unit<4>(a, cur, lds[b]);
      else gu_unit<2>(a, cur, lds[b]);
      if (more) gu_stage_store(st, nx, lds[b ^ 1]);
      // arrival: this workgroup's slot stores have completed before it is counted
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(cur.arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = prev == (unsigned)q.NCK - 1;
        if (s_flag) __hip_atomic_store(cur.arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (s_flag) {
        if (cur.ntl == 4) gu_combine<4>(cur);
        else gu_combine<2>(cur);
      }
      cur = nx;
      b ^= 1;
    }
  }
  const int n_vr = n_qv * (q.F / 16), n_vs = (q.Fs > 0 && !s_mfma) ? q.Fs / 16 : 0;
  for (int i = (w - (n_mfma > 0 ? n_mfma % G : 0) + G) % G; i < n_vr + n_vs; i += G) {
    GuItem it;
    if (i < n_vr) {
      const int slot = a.gu_q[n_qm + i / (q.F / 16)], tile = i % (q.F / 16);
      const int ex = a.act_exp[slot], off = a.act_off[slot];
      it.w1 = a.w1 + ((size_t)ex * q.F + tile * 16) * a.H;
      it.w3 = a.w3 + ((size_t)ex * q.F + tile * 16) * a.H;
      it.toks = a.pair_tok + off;
      it.tok0 = 0;
      it.out = a.act + (size_t)off * q.F + tile * 16;
      it.ld = q.F;
      it.cnt = a.act_cnt[slot];
    } else {
      const int tile = i - n_vr;
      it.w1 = a.s1 + (size_t)tile * 16 * a.H;
      it.w3 = a.s3 + (size_t)tile * 16 * a.H;
      it.toks = nullptr;
      it.tok0 = 0;
      it.out = a.act_s + tile * 16;
      it.ld = q.Fs;
      it.cnt = q.B;
    }
    gateup_valu(a, it);
  }
}

// ================================================================ launch 5
// Weights of one item for this lane: row n = lane % 16 of the 16-row tile,
// K positions 32 s + 8 g (g = lane / 16) for s < NKS = Fd / 32.  MFMA items
// use them as the B operand; VALU items reduce the four g lanes of a row.
template <int NKS>
__device__ __forceinline__ void down_load_w(const uint16_t *tile, uint4 (&wv)[NKS]) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const uint16_t *p = tile + (size_t)n * (32 * NKS) + 8 * g;
#pragma unroll
  for (int s = 0; s < NKS; ++s) wv[s] = ld16(p + 32 * s);
}

struct DnItem {
  const float *act;   // row m at act + m * Fd
  const int *toks;    // token of row m (nullptr: m itself)
  const float *wts;   // weight of row m (nullptr: 1)
  int cnt;
  __device__ int tok(int m) const { return toks ? toks[m] : m; }
  __device__ float wt(int m) const { return wts ? wts[m] : 1.f; }
};

// Rows [c0, c0 + 16) of an item on the matrix cores: load, then compute.
template <int NKS>
struct MfmaChunk {
  float4 xv[NKS][2];
  __device__ __forceinline__ void load(const DnItem &it, int c0) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const float *ap = it.act + (size_t)min(c0 + n, it.cnt - 1) * (32 * NKS) + 8 * g;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      xv[s][0] = ld16f(ap + 32 * s);
      xv[s][1] = ld16f(ap + 32 * s + 4);
    }
  }
  __device__ __forceinline__ void compute(const DnItem &it, int c0, const uint4 (&wv)[NKS], float (*y)[16]) const {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const float x[8] = {xv[s][0].x, xv[s][0].y, xv[s][0].z, xv[s][0].w,
                          xv[s][1].x, xv[s][1].y, xv[s][1].z, xv[s][1].w};
      uint4 hi, lo;
      split8(x, hi, lo);
      acc = mfma_bf16(hi, wv[s], acc);
      acc = mfma_bf16(lo, wv[s], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = c0 + 4 * g + i;
      if (m < it.cnt) y[it.tok(m)][n] += it.wt(m) * acc[i];
    }
  }
};

// Rows m0 .. m0 + TB - 1 (below cnt) of an item on the VALU.
template <int NKS>
struct ValuRows {
  static constexpr int TB = 8 / NKS;   // 64 VGPRs of activations per batch
  float4 xv[TB][NKS][2];
  __device__ __forceinline__ void load(const DnItem &it, int m0) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const float *ap = it.act + (size_t)min(m0 + tb, it.cnt - 1) * (32 * NKS) + 8 * g;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        xv[tb][s][0] = ld16f(ap + 32 * s);
        xv[tb][s][1] = ld16f(ap + 32 * s + 4);
      }
    }
  }
  __device__ __forceinline__ void compute(const DnItem &it, int m0, const uint4 (&wv)[NKS], float (*y)[16]) const {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        float wf[8];
        unpack8(wv[s], wf);
        const float x[8] = {xv[tb][s][0].x, xv[tb][s][0].y, xv[tb][s][0].z, xv[tb][s][0].w,
                            xv[tb][s][1].x, xv[tb][s][1].y, xv[tb][s][1].z, xv[tb][s][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], x[e], acc);
      }
      acc += __shfl_xor(acc, 16, kWave);   // lanes g, g ^ 1
      acc += __shfl_xor(acc, 32, kWave);   // (v0 + v1) + (v2 + v3)
      const int m = m0 + tb;
      if (g == 0 && m < it.cnt) y[it.tok(m)][n] += it.wt(m) * acc;
    }
  }
};

// One item with weights wv; if `next` is set, the next item's weights are
// requested right after this item's first activation batch, so the wait
// for those activations does not include them (a wave's loads complete in
// issue order).
template <int NKS>
__device__ __forceinline__ void down_item(const DnItem &it, const uint4 (&wv)[NKS], float (*y)[16],
                                          const uint16_t *next, uint4 (&wn)[NKS]) {
  if (it.cnt >= kBatchMfmaMin) {
    for (int c0 = 0; c0 < it.cnt; c0 += 16) {
      MfmaChunk<NKS> ch;
      ch.load(it, c0);
      if (c0 == 0 && next) down_load_w<NKS>(next, wn);
      DL_SCHED_FENCE();
      ch.compute(it, c0, wv, y);
    }
  } else {
    for (int m0 = 0; m0 < it.cnt; m0 += ValuRows<NKS>::TB) {
      ValuRows<NKS> rw;
      rw.load(it, m0);
      if (m0 == 0 && next) down_load_w<NKS>(next, wn);
      DL_SCHED_FENCE();
      rw.compute(it, m0, wv, y);
    }
  }
}

// Routed items of this wave: active slots wv, wv + 4, ... (metadata in LDS).
template <int NKS>
__device__ void down_routed(const BatchArgs &a, int i0, int n_act, const int *exp_, const int *cnt_,
                            const int *off_, float (*y)[16]) {
  constexpr int Fd = 32 * NKS;
  const int wv = threadIdx.x >> 6;
  if (wv >= n_act) return;
  auto tile = [&](int slot) { return a.w2 + ((size_t)exp_[slot] * a.H + i0) * Fd; };
  uint4 wc[NKS], wn[NKS];
  down_load_w<NKS>(tile(wv), wc);
  for (int i = wv; i < n_act; i += kWavesPerBlock) {
    const int off = off_[i];
    const DnItem it{a.act + (size_t)off * Fd, a.pair_tok + off, a.pair_w + off, cnt_[i]};
    const int nx = i + kWavesPerBlock;
    down_item<NKS>(it, wc, y, nx < n_act ? tile(nx) : nullptr, wn);
#pragma unroll
    for (int s = 0; s < NKS; ++s) wc[s] = wn[s];
  }
}

// The shared expert (weight 1, every token): with 16 or more tokens wave w
// takes the 16-token chunk w on the matrix cores; below that one wave takes
// all tokens on the VALU.
template <int NKS>
__device__ void down_shared(const BatchArgs &a, int i0, int n_act, float (*y)[16]) {
  const int wv = threadIdx.x >> 6, B = a.B;
  const DnItem it{a.act_s, nullptr, nullptr, B};
  const uint16_t *tile = a.s2 + (size_t)i0 * (32 * NKS);
  uint4 wv_[NKS];
  if (B >= kBatchMfmaMin) {
    if (16 * wv < B) {
      down_load_w<NKS>(tile, wv_);
      MfmaChunk<NKS> ch;
      ch.load(it, 16 * wv);
      DL_SCHED_FENCE();
      ch.compute(it, 16 * wv, wv_, y);
    }
  } else if (wv == n_act % kWavesPerBlock) {
    down_load_w<NKS>(tile, wv_);
    for (int m0 = 0; m0 < B; m0 += ValuRows<NKS>::TB) {
      ValuRows<NKS> rw;
      rw.load(it, m0);
      DL_SCHED_FENCE();
      rw.compute(it, m0, wv_, y);
    }
  }
}

template <class Fn>
__device__ __forceinline__ void by_nks(int Fd, Fn fn) {
  switch (Fd) {
    case 32: fn(std::integral_constant<int, 1>{}); break;
    case 64: fn(std::integral_constant<int, 2>{}); break;
    case 128: fn(std::integral_constant<int, 4>{}); break;
    default: fn(std::integral_constant<int, 8>{}); break;
  }
}

// Workgroup: rows [16 b, 16 b + 16) of y for every token.  Each wave adds its
// items into its own LDS accumulator; the four are added in wave order.
__global__ void __launch_bounds__(kBlock) down_b(BatchArgs a) {
  __shared__ float yw[kWavesPerBlock][kMaxBatch][16];
  __shared__ int s_exp[kMaxExperts], s_cnt[kMaxExperts], s_off[kMaxExperts];
  const int tid = threadIdx.x, wv = tid >> 6;
  const int B = a.B, H = a.H, i0 = blockIdx.x * 16;
  const int n_act = *a.n_active;
  for (int q = tid; q < kWavesPerBlock * kMaxBatch * 16; q += kBlock) (&yw[0][0][0])[q] = 0.f;
  for (int q = tid; q < n_act; q += kBlock) {
    s_exp[q] = a.act_exp[q];
    s_cnt[q] = a.act_cnt[q];
    s_off[q] = a.act_off[q];
  }
  __syncthreads();
  by_nks(a.F, [&](auto k) { down_routed<decltype(k)::value>(a, i0, n_act, s_exp, s_cnt, s_off, yw[wv]); });
  if (a.Fs > 0) by_nks(a.Fs, [&](auto k) { down_shared<decltype(k)::value>(a, i0, n_act, yw[wv]); });
  __syncthreads();
  for (int q = tid; q < B * 16; q += kBlock) {
    const int t = q >> 4, nn = q & 15;
    a.moe_out[(size_t)t * H + i0 + nn] = ((yw[0][t][nn] + yw[1][t][nn]) + yw[2][t][nn]) + yw[3][t][nn];
  }
}

}  // namespace

hipError_t launch_batched(const BatchArgs &a, hipStream_t s, hipEvent_t (*ev)[2]) {
  const int n_wo = a.H / 16;
  const int n_q = (a.Dq + 15) / 16 * kBatchQkvSplit;
  const int n_rk = a.H / kBatchRtrK;
  hipError_t e;
  auto rec = [&](int i, int j) { return ev ? hipEventRecord(ev[i][j], s) : hipSuccess; };
#define DL_TRY(x) do { if ((e = (x)) != hipSuccess) return e; } while (0)
  DL_TRY(rec(0, 0));
  hipLaunchKernelGGL(proj_b, dim3(n_wo + n_q), dim3(kBlock), 0, s, a, n_wo);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(0, 1));
  DL_TRY(rec(1, 0));
  hipLaunchKernelGGL(router_b, dim3((a.E + kBatchRtrExperts - 1) / kBatchRtrExperts, n_rk), dim3(kBlock), 0, s, a);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(1, 1));
  DL_TRY(rec(2, 0));
  hipLaunchKernelGGL(topk_b, dim3(a.B), dim3(kBlock), 0, s, a, n_wo, n_rk);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(2, 1));
  DL_TRY(rec(3, 0));
  hipLaunchKernelGGL(gateup_b, dim3(a.gu_grid), dim3(kBlock), 0, s, a);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(3, 1));
  DL_TRY(rec(4, 0));
  hipLaunchKernelGGL(down_b, dim3(n_wo), dim3(kBlock), 0, s, a);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(4, 1));
#undef DL_TRY
  return hipSuccess;
}

}  // namespace dl
