// Launch 2 of the step: router scores, top-k selection and the
// token-to-expert permutation (wireai.ir "vLLM's speed jump on NVIDIA
// Blackwell servers; record 842 tokens/s for Kimi K3", section "Four key
// changes behind the jump", bullet 3: router scores before the shared and
// routed experts).
//
// Workgroup e computes, for every token, the fp32 logit of expert e:
//   l[t, e] = inv_rms[t] * sum_i Wr[e, i] hg[t, i]    (= h[t] . Wr[e])
// with K = H split over its 4 waves and reduced through LDS.  The last
// workgroup to finish (cross-workgroup hand-off in common.h) then, per token,
// picks the k largest logits with a wave64 shuffle arg-max (descending, ties
// to the lower expert id), computes s = sigmoid(l) and w = s / sum s over the
// k picks, and builds the per-expert token lists the expert kernels walk:
//   act_exp[a], act_cnt[a], act_off[a]  for active experts a < n_active
//                                       (ascending expert id),
//   pair_tok[p], pair_w[p]              token and weight of pair p, grouped
//                                       by expert, tokens ascending inside.
#include "common.h"
#include "kernels.h"

namespace dl {

template <int NT>
__device__ void router_chunk(const RouterArgs &a, int e, int t0, int nt, float (&red)[4][kTokChunk]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float *w = a.w_router + (size_t)e * a.H;
  const float *hb = a.hg + (size_t)t0 * a.H;
  float acc[NT] = {};
  // each lane visit covers 8 consecutive fp32 weights (two 16-byte loads)
  const int kstride = kBlock * 8;
  int k = (wave * 64 + lane) * 8;
  for (; k + kstride < a.H; k += 2 * kstride) {
    float4 w0 = ld_stream16f(w + k), w1 = ld_stream16f(w + k + 4);
    float4 w2 = ld_stream16f(w + k + kstride), w3 = ld_stream16f(w + k + kstride + 4);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int tt = t < nt ? t : nt - 1;
      const float *p = hb + (size_t)tt * a.H + k;
      float4 h0 = ld16f(p), h1 = ld16f(p + 4), h2 = ld16f(p + kstride), h3 = ld16f(p + kstride + 4);
      float s = acc[t];
      s = fmaf(w0.x, h0.x, s); s = fmaf(w0.y, h0.y, s); s = fmaf(w0.z, h0.z, s); s = fmaf(w0.w, h0.w, s);
      s = fmaf(w1.x, h1.x, s); s = fmaf(w1.y, h1.y, s); s = fmaf(w1.z, h1.z, s); s = fmaf(w1.w, h1.w, s);
      s = fmaf(w2.x, h2.x, s); s = fmaf(w2.y, h2.y, s); s = fmaf(w2.z, h2.z, s); s = fmaf(w2.w, h2.w, s);
      s = fmaf(w3.x, h3.x, s); s = fmaf(w3.y, h3.y, s); s = fmaf(w3.z, h3.z, s); s = fmaf(w3.w, h3.w, s);
      acc[t] = s;
    }
  }
  for (; k < a.H; k += kstride) {
    float4 w0 = ld_stream16f(w + k), w1 = ld_stream16f(w + k + 4);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int tt = t < nt ? t : nt - 1;
      const float *p = hb + (size_t)tt * a.H + k;
      float4 h0 = ld16f(p), h1 = ld16f(p + 4);
      float s = acc[t];
      s = fmaf(w0.x, h0.x, s); s = fmaf(w0.y, h0.y, s); s = fmaf(w0.z, h0.z, s); s = fmaf(w0.w, h0.w, s);
      s = fmaf(w1.x, h1.x, s); s = fmaf(w1.y, h1.y, s); s = fmaf(w1.z, h1.z, s); s = fmaf(w1.w, h1.w, s);
      acc[t] = s;
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float v = wave_sum(acc[t]);
    if (lane == 0) red[wave][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    int t = threadIdx.x;
    float d = red[0][t] + red[1][t] + red[2][t] + red[3][t];
    float l = d * a.inv_rms[t0 + t];
    a.logits[(size_t)(t0 + t) * a.E + e] = l;
    if (a.logits_out) a.logits_out[(size_t)(t0 + t) * a.E + e] = l;
  }
  __syncthreads();
}

// Per-token top-k over the logits in global memory (wave_topk in common.h:
// descending, ties to the lower expert id, always k distinct valid ids).
__device__ void topk_token(const RouterArgs &a, int t, int *s_sel, float *s_w) {
  const int lane = threadIdx.x & 63;
  constexpr int NC = kMaxExperts / 64;
  const float *lg = a.logits + (size_t)t * a.E;
  float lv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e = lane + 64 * c;
    lv[c] = e < a.E ? lg[e] : 0.f;
  }
  int my_idx;
  float my_l;
  wave_topk<NC>(lv, a.E, a.K, my_idx, my_l);
  const float w = pick_weights(my_l, a.K);
  if (lane < a.K) {
    a.topk_idx[(size_t)t * a.K + lane] = my_idx;
    a.topk_w[(size_t)t * a.K + lane] = w;
    s_sel[t * a.K + lane] = my_idx;
    s_w[t * a.K + lane] = w;
  }
}

__global__ void __launch_bounds__(kBlock) router_kernel(RouterArgs a) {
  __shared__ float red[4][kTokChunk];
  __shared__ int last_flag;
  __shared__ int s_sel[kMaxBatch * kMaxTopK];
  __shared__ float s_w[kMaxBatch * kMaxTopK];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_sa[kBlock], s_sc[kBlock];
  const int e = blockIdx.x;
  for (int t0 = 0; t0 < a.B; t0 += kTokChunk) {
    int nt = min(kTokChunk, a.B - t0);
    if (nt == 1) router_chunk<1>(a, e, t0, nt, red);
    else if (nt == 2) router_chunk<2>(a, e, t0, nt, red);
    else if (nt <= 4) router_chunk<4>(a, e, t0, nt, red);
    else router_chunk<8>(a, e, t0, nt, red);
  }
  if (a.h_out) {  // optional copy of h = hg * inv_rms, spread over the grid
    const size_t n = (size_t)a.B * a.H;
    for (size_t q = (size_t)e * kBlock + threadIdx.x; q < n; q += (size_t)gridDim.x * kBlock)
      a.h_out[q] = a.hg[q] * a.inv_rms[q / a.H];
  }
  if (!arrive_last(a.counter, gridDim.x, &last_flag)) return;

  // ---- tail: one workgroup ----
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int t = wave; t < a.B; t += 4) topk_token(a, t, s_sel, s_w);
  for (int q = tid; q < a.E; q += kBlock) s_cnt[q] = 0;
  __syncthreads();
  const int n = a.B * a.K;
  for (int i = tid; i < n; i += kBlock) atomicAdd(&s_cnt[s_sel[i]], 1);
  __syncthreads();
  // exclusive scans over experts: active-expert slots and pair offsets
  const int seg = (a.E + kBlock - 1) / kBlock;
  const int e0 = tid * seg, e1 = min(a.E, e0 + seg);
  int la = 0, lc = 0;
  for (int q = e0; q < e1; ++q) { int c = s_cnt[q]; la += c > 0; lc += c; }
  s_sa[tid] = la;
  s_sc[tid] = lc;
  __syncthreads();
  for (int o = 1; o < kBlock; o <<= 1) {  // Hillis-Steele inclusive scan
    int va = tid >= o ? s_sa[tid - o] : 0, vc = tid >= o ? s_sc[tid - o] : 0;
    __syncthreads();
    s_sa[tid] += va;
    s_sc[tid] += vc;
    __syncthreads();
  }
  int pa = s_sa[tid] - la, pc = s_sc[tid] - lc;
  for (int q = e0; q < e1; ++q) {
    int c = s_cnt[q];
    s_off[q] = pc;
    if (c > 0) {
      a.act_exp[pa] = q;
      a.act_cnt[pa] = c;
      a.act_off[pa] = pc;
      ++pa;
      pc += c;
    }
  }
  if (tid == kBlock - 1) *a.n_active = s_sa[kBlock - 1];
  __syncthreads();
  for (int i = tid; i < n; i += kBlock) {
    int ex = s_sel[i], r = 0;
    for (int i2 = 0; i2 < i; ++i2) r += s_sel[i2] == ex;
    int pos = s_off[ex] + r;
    a.pair_tok[pos] = i / a.K;
    a.pair_w[pos] = s_w[i];
  }
}

hipError_t launch_router(const RouterArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(router_kernel, dim3(a.E), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace dl
