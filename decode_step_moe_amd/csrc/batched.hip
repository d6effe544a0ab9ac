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
//  4 gateup_b  items (active expert or shared expert, 16 ffn rows):
//              a[p, f] = silu(W1[e, f] . h[t_p]) * (W3[e, f] . h[t_p]).
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
// its 8g K position).  U K-steps of loads are issued before their MFMAs.
template <int NC, int U>
__device__ __forceinline__ void mfma_rows(const uint16_t *wp, const uint16_t *const (&ap)[NC], int nks,
                                          f32x4 (&acc)[NC]) {
  int ks = 0;
  for (; ks + U <= nks; ks += U) {
    uint4 wv[U], av[U][NC];
#pragma unroll
    for (int u = 0; u < U; ++u) wv[u] = ld_stream16(wp + (ks + u) * 32);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c) av[u][c] = ld16(ap[c] + (ks + u) * 32);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = mfma_bf16(av[u][c], wv[u], acc[c]);
  }
  for (; ks < nks; ++ks) {
    const uint4 wv = ld_stream16(wp + ks * 32);
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = mfma_bf16(ld16(ap[c] + ks * 32), wv, acc[c]);
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
      b0[it] = ld_stream16f(w0 + 16 * it);
      b1[it] = ld_stream16f(w1 + 16 * it);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float *ap = a.hg + (size_t)min(16 * c + n, B - 1) * H + kb;
#pragma unroll
      for (int it = 0; it < 4; ++it) av[it][c] = ld16f(ap + 16 * it);
    }
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
    for (int ky = 0; ky < n_rk; ++ky) d += a.rlog_part[((size_t)ky * B + t) * E + e];
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
    if (lane < K) {
      a.topk_idx[(size_t)t * K + lane] = my_idx;
      a.topk_w[(size_t)t * K + lane] = s / ssum;
    }
  }
  if (!arrive_last(a.counter, B, &last_flag)) return;

  // ---- the last workgroup: per-expert token lists ----
  for (int q = tid; q < E; q += kBlock) {
    cnt[q] = 0;
    msk[q][0] = msk[q][1] = 0u;
  }
  __syncthreads();
  const int P = B * K;
  for (int i = tid; i < P; i += kBlock) {
    const int e = a.topk_idx[i], tt = i / K;
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
      ++pa;
      pc += c;
    }
  }
  if (tid == kBlock - 1) *a.n_active = sa[kBlock - 1];
  __syncthreads();
  // a pair's place inside its expert = number of lower tokens with that expert
  for (int i = tid; i < P; i += kBlock) {
    const int e = a.topk_idx[i], tt = i / K;
    const unsigned m0 = msk[e][0], m1 = msk[e][1];
    const int r = tt < 32 ? __popc(m0 & ((1u << tt) - 1u)) : __popc(m0) + __popc(m1 & ((1u << (tt - 32)) - 1u));
    const int pos = off[e] + r;
    a.pair_tok[pos] = tt;
    a.pair_w[pos] = a.topk_w[i];
  }
}

// ================================================================ launch 4
struct GuItem {
  const uint16_t *w1, *w3;  // first of the item's 16 rows, row stride H
  const int *toks;          // token of row m (nullptr: m itself)
  float *out;               // row m of the output at out + m * ld, 16 columns
  int ld, cnt;
  __device__ int tok(int m) const { return toks ? toks[m] : m; }
};

// 16 tokens per chunk on the matrix cores; the 4 waves split K.
template <int NC>
__device__ void gateup_mfma(const BatchArgs &a, const GuItem &it, float (*red)[4 * 2 * 256]) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int H = a.H, kw = wv * (H / 4) + 8 * g, nks = H / 128;
  const uint16_t *p1 = it.w1 + (size_t)n * H + kw, *p3 = it.w3 + (size_t)n * H + kw;
  const uint16_t *ph[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) ph[c] = a.hp + (size_t)it.tok(min(16 * c + n, it.cnt - 1)) * H + kw;
  const size_t plane = (size_t)a.B * H;
  f32x4 acc1[NC], acc3[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc1[c] = acc3[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = NC <= 2 ? 4 : 2;
  int ks = 0;
  for (; ks + U <= nks; ks += U) {
    uint4 w1v[U], w3v[U], hv[U][NC], lv[U][NC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w1v[u] = ld_stream16(p1 + (ks + u) * 32);
      w3v[u] = ld_stream16(p3 + (ks + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        hv[u][c] = ld16(ph[c] + (ks + u) * 32);
        lv[u][c] = ld16(ph[c] + plane + (ks + u) * 32);
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc1[c] = mfma_bf16(hv[u][c], w1v[u], acc1[c]);
        acc1[c] = mfma_bf16(lv[u][c], w1v[u], acc1[c]);
        acc3[c] = mfma_bf16(hv[u][c], w3v[u], acc3[c]);
        acc3[c] = mfma_bf16(lv[u][c], w3v[u], acc3[c]);
      }
  }
  for (; ks < nks; ++ks) {
    const uint4 w1v = ld_stream16(p1 + ks * 32), w3v = ld_stream16(p3 + ks * 32);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 hv = ld16(ph[c] + ks * 32), lv = ld16(ph[c] + plane + ks * 32);
      acc1[c] = mfma_bf16(hv, w1v, acc1[c]);
      acc1[c] = mfma_bf16(lv, w1v, acc1[c]);
      acc3[c] = mfma_bf16(hv, w3v, acc3[c]);
      acc3[c] = mfma_bf16(lv, w3v, acc3[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[wv][(c * 2) * 256 + (4 * g + i) * 16 + n] = acc1[c][i];
      red[wv][(c * 2 + 1) * 256 + (4 * g + i) * 16 + n] = acc3[c][i];
    }
  __syncthreads();
  for (int q = tid; q < it.cnt * 16; q += kBlock) {
    const int m = q >> 4, nn = q & 15;
    const int i1 = ((m >> 4) * 2) * 256 + (m & 15) * 16 + nn;
    const float u = ((red[0][i1] + red[1][i1]) + red[2][i1]) + red[3][i1];
    const float v = ((red[0][i1 + 256] + red[1][i1 + 256]) + red[2][i1 + 256]) + red[3][i1 + 256];
    it.out[(size_t)m * it.ld + nn] = silu_mul(u, v);
  }
}

// Fewer than 16 tokens: wave w takes rows 4w .. 4w+3 of the item, one
// (W1 row, W3 row) pair at a time over the full K, up to 8 tokens per pass.
__device__ void gateup_valu(const BatchArgs &a, const GuItem &it) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H;
  for (int t0 = 0; t0 < it.cnt; t0 += 8) {
    const int nt = min(8, it.cnt - t0);
    auto pass = [&](auto ntc) {
      constexpr int NT = decltype(ntc)::value;
      constexpr int CPB = NT <= 4 ? 4 : 2;
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

// Items: (active slot, 16-row tile) for the routed experts, then the shared
// expert's tiles.  Block b runs on XCD b % 8; each XCD takes a contiguous
// range of items, so an expert's tiles (which read the same token rows of h)
// mostly share one L2.
__global__ void __launch_bounds__(kBlock) gateup_b(BatchArgs a) {
  __shared__ float red[kWavesPerBlock][4 * 2 * 256];
  const int n_act = *a.n_active;
  const int ntr = a.F / 16, nts = a.Fs / 16;
  const int n_items = n_act * ntr + nts;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3, nloc = gridDim.x >> 3;
  const int per = (n_items + 7) >> 3;
  const int beg = xcd * per, end = min(beg + per, n_items);
  for (int i = beg + loc; i < end; i += nloc) {
    GuItem it;
    if (i < n_act * ntr) {
      const int slot = i / ntr, tile = i % ntr;
      const int e = a.act_exp[slot], off = a.act_off[slot];
      it.w1 = a.w1 + ((size_t)e * a.F + tile * 16) * a.H;
      it.w3 = a.w3 + ((size_t)e * a.F + tile * 16) * a.H;
      it.toks = a.pair_tok + off;
      it.out = a.act + (size_t)off * a.F + tile * 16;
      it.ld = a.F;
      it.cnt = a.act_cnt[slot];
    } else {
      const int tile = i - n_act * ntr;
      it.w1 = a.s1 + (size_t)tile * 16 * a.H;
      it.w3 = a.s3 + (size_t)tile * 16 * a.H;
      it.toks = nullptr;
      it.out = a.act_s + tile * 16;
      it.ld = a.Fs;
      it.cnt = a.B;
    }
    if (it.cnt >= kBatchMfmaMin)
      by_chunks((it.cnt + 15) >> 4, [&](auto ncc) { gateup_mfma<decltype(ncc)::value>(a, it, red); });
    else
      gateup_valu(a, it);
    __syncthreads();  // red is reused by the next item
  }
}

// ================================================================ launch 5
struct DnItem {
  const uint16_t *w;  // row r0 of the item's [H][Fd] matrix
  const float *act;   // row m at act + m * Fd
  const int *toks;    // token of row m (nullptr: m itself)
  const float *wts;   // weight of row m (nullptr: 1)
  int Fd, cnt;
};

__device__ void down_mfma(const DnItem &it, float (*y)[16]) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int nks = it.Fd / 32;
  uint4 wv[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    if (s < nks) wv[s] = ld_stream16(it.w + (size_t)n * it.Fd + 32 * s + 8 * g);
  for (int c0 = 0; c0 < it.cnt; c0 += 16) {
    const float *ap = it.act + (size_t)min(c0 + n, it.cnt - 1) * it.Fd + 8 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < nks) {
        float x[8];
        load8f(ap + 32 * s, x);
        uint4 hi, lo;
        split8(x, hi, lo);
        acc = mfma_bf16(hi, wv[s], acc);
        acc = mfma_bf16(lo, wv[s], acc);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = c0 + 4 * g + i;
      if (m < it.cnt) {
        const int t = it.toks ? it.toks[m] : m;
        const float w = it.wts ? it.wts[m] : 1.f;
        y[t][n] += w * acc[i];
      }
    }
  }
}

// Lane l: row l / 4 of the tile, K chunks (l % 4) + 4j of 8 values; the 4
// lanes of a row reduce with quad permutes.
__device__ void down_valu(const DnItem &it, float (*y)[16]) {
  const int lane = threadIdx.x & 63, r = lane >> 2, q = lane & 3;
  const int nch = it.Fd / 32;
  uint4 wv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < nch) wv[j] = ld_stream16(it.w + (size_t)r * it.Fd + 8 * q + 32 * j);
  for (int m = 0; m < it.cnt; ++m) {
    const float *ap = it.act + (size_t)m * it.Fd + 8 * q;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < nch) {
        float x[8], wf[8];
        load8f(ap + 32 * j, x);
        unpack8(wv[j], wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], x[e], acc);
      }
    acc += dpp_mov<kDppXor1>(acc);
    acc += dpp_mov<kDppXor2>(acc);
    if (q == 0) {
      const int t = it.toks ? it.toks[m] : m;
      const float w = it.wts ? it.wts[m] : 1.f;
      y[t][r] += w * acc;
    }
  }
}

// Workgroup: rows [16 b, 16 b + 16) of y for every token.  Wave w takes items
// w, w + 4, ... (active slots, then the shared expert) into its own LDS
// accumulator; the four accumulators are added in wave order at the end.
__global__ void __launch_bounds__(kBlock) down_b(BatchArgs a) {
  __shared__ float yw[kWavesPerBlock][kMaxBatch][16];
  const int tid = threadIdx.x, wv = tid >> 6;
  const int B = a.B, H = a.H, i0 = blockIdx.x * 16;
  for (int q = tid; q < kWavesPerBlock * kMaxBatch * 16; q += kBlock) (&yw[0][0][0])[q] = 0.f;
  __syncthreads();
  const int n_act = *a.n_active;
  const int n_items = n_act + (a.Fs > 0 ? 1 : 0);
  for (int i = wv; i < n_items; i += kWavesPerBlock) {
    DnItem it;
    if (i < n_act) {
      const int e = a.act_exp[i], off = a.act_off[i];
      it.w = a.w2 + ((size_t)e * H + i0) * a.F;
      it.act = a.act + (size_t)off * a.F;
      it.toks = a.pair_tok + off;
      it.wts = a.pair_w + off;
      it.Fd = a.F;
      it.cnt = a.act_cnt[i];
    } else {
      it.w = a.s2 + (size_t)i0 * a.Fs;
      it.act = a.act_s;
      it.toks = nullptr;
      it.wts = nullptr;
      it.Fd = a.Fs;
      it.cnt = B;
    }
    if (it.cnt >= kBatchMfmaMin) down_mfma(it, yw[wv]);
    else down_valu(it, yw[wv]);
  }
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
  const int max_items = min(a.E, a.B * a.K) * (a.F / 16) + a.Fs / 16;
  const int g4 = min(kBatchGateupGrid, (max_items + 7) & ~7);
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
  hipLaunchKernelGGL(gateup_b, dim3(g4), dim3(kBlock), 0, s, a);
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
