// Launches 3-5 of the step: the SwiGLU experts.
//
// gateup_kernel (routed experts on the caller's stream; the shared expert on
// the handle's second stream, overlapping the router and the routed experts -
// wireai.ir "vLLM's speed jump on NVIDIA Blackwell servers; record 842
// tokens/s for Kimi K3", section "Four key changes behind the jump", bullet 3):
//   for every (expert, token) pair p and ffn row f,
//     u = inv_rms[t] * sum_i W1[e, f, i] hg[t, i]      (= W1 h)
//     v = inv_rms[t] * sum_i W3[e, f, i] hg[t, i]      (= W3 h)
//     act[p, f] = silu(u) * v
//   Each wave owns one ffn row f and streams W1 row f and W3 row f once for
//   all of the expert's tokens.  Work items (active expert, 4-row tile) are
//   strided over the grid because the number of active experts is only known
//   on the device.
//
// down_kernel (caller's stream, after joining the shared expert):
//   y[t, i] = sum_s1 S2[i, :] . act_s[t, :] + sum_p w_p W2[e_p, i, :] . act[p, :]
//   Output-stationary: a workgroup owns 16 rows of y for all tokens and walks
//   every active expert (waves take experts round-robin), so each y element
//   is summed in a fixed order in LDS without atomics, and y needs no
//   zeroing.  The shared expert's contribution enters with weight one.
#include "common.h"
#include "kernels.h"

namespace dl {

template <int NT>
__device__ void gateup_chunk(const GateUpArgs &a, const uint16_t *w1row, const uint16_t *w3row,
                             const int *tok_list, int tok_base, int nt, size_t act_row0, int f) {
  const int lane = threadIdx.x & 63;
  ActF32Gather<NT> act;
  act.base = a.hg;
  act.ld = a.H;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int tt = t < nt ? t : nt - 1;
    act.tok[t] = tok_list ? tok_list[tt] : tok_base + tt;
  }
  const uint16_t *w[2] = {w1row, w3row};
  float acc[2][NT] = {};
  stream_rows_bf16<2, NT, 7>(w, act, lane * 8, kWave * 8, a.H, acc);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float u = wave_sum(acc[0][t]);
    float v = wave_sum(acc[1][t]);
    if (lane == t && t < nt) {
      float inv = a.inv_rms[act.tok[t]];
      u *= inv;
      v *= inv;
      float s = u / (1.0f + expf(-u));
      a.act[(act_row0 + t) * a.F + f] = s * v;
    }
  }
}

__device__ void gateup_tokens(const GateUpArgs &a, const uint16_t *w1row, const uint16_t *w3row,
                              const int *tok_list, int tok_base, int cnt, size_t act_row0, int f) {
  for (int p0 = 0; p0 < cnt; p0 += kTokChunk) {
    int nt = min(kTokChunk, cnt - p0);
    const int *tl = tok_list ? tok_list + p0 : nullptr;
    if (nt == 1) gateup_chunk<1>(a, w1row, w3row, tl, tok_base + p0, nt, act_row0 + p0, f);
    else if (nt == 2) gateup_chunk<2>(a, w1row, w3row, tl, tok_base + p0, nt, act_row0 + p0, f);
    else if (nt <= 4) gateup_chunk<4>(a, w1row, w3row, tl, tok_base + p0, nt, act_row0 + p0, f);
    else gateup_chunk<8>(a, w1row, w3row, tl, tok_base + p0, nt, act_row0 + p0, f);
  }
}

__global__ void __launch_bounds__(kBlock) gateup_kernel(GateUpArgs a) {
  const int wave = threadIdx.x >> 6;
  const int ntile = a.F / kGateRowsPerBlock;
  if (a.shared) {
    for (int it = blockIdx.x; it < ntile; it += gridDim.x) {
      int f = it * kGateRowsPerBlock + wave;
      gateup_tokens(a, a.w1 + (size_t)f * a.H, a.w3 + (size_t)f * a.H, nullptr, 0, a.B, 0, f);
    }
    return;
  }
  const int n_items = *a.n_active * ntile;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    int slot = it / ntile, f = (it % ntile) * kGateRowsPerBlock + wave;
    int e = a.act_exp[slot], cnt = a.act_cnt[slot], off = a.act_off[slot];
    size_t row = (size_t)e * a.F + f;
    gateup_tokens(a, a.w1 + row * a.H, a.w3 + row * a.H, a.pair_tok + off, 0, cnt, (size_t)off, f);
  }
}

// One expert slot's contribution to the workgroup's 16 output rows.
// LPR lanes share one row of W2 (F = 8 * LPR); a wave load covers 64/LPR rows.
template <int LPR, int NT>
__device__ void down_slot_chunk(const uint16_t *w2e, int F, int i0, int H, const float *actb,
                                const int *toks, const float *wts, int nt, float *yacc /* [B][16] */) {
  constexpr int RPL = 64 / LPR;                 // rows per wave load
  constexpr int NLD = kDownRows / RPL;          // loads per lane
  const int lane = threadIdx.x & 63;
  const int rg = lane / LPR, fc = lane % LPR;
  uint4 wv[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    int i = min(i0 + rg + RPL * j, H - 1);
    wv[j] = ld_stream16(w2e + (size_t)i * F + fc * 8);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int tt = t < nt ? t : nt - 1;
    const float *p = actb + (size_t)tt * F + fc * 8;
    float4 u = ld16f(p), v = ld16f(p + 4);
    float av[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      float wf[8];
      unpack8(wv[j], wf);
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) s = fmaf(wf[q], av[q], s);
      s = group_sum(s, LPR);
      if (fc == 0 && t < nt) {
        int r = rg + RPL * j;
        yacc[toks[tt] * kDownRows + r] += wts[tt] * s;
      }
    }
  }
}

template <int LPR>
__device__ void down_slot(const uint16_t *w2e, int F, int i0, int H, const float *act0, const int *toks,
                          const float *wts, int cnt, float *yacc) {
  for (int p0 = 0; p0 < cnt; p0 += kTokChunk) {
    int nt = min(kTokChunk, cnt - p0);
    const float *ab = act0 + (size_t)p0 * F;
    if (nt == 1) down_slot_chunk<LPR, 1>(w2e, F, i0, H, ab, toks + p0, wts + p0, nt, yacc);
    else if (nt == 2) down_slot_chunk<LPR, 2>(w2e, F, i0, H, ab, toks + p0, wts + p0, nt, yacc);
    else if (nt <= 4) down_slot_chunk<LPR, 4>(w2e, F, i0, H, ab, toks + p0, wts + p0, nt, yacc);
    else down_slot_chunk<LPR, 8>(w2e, F, i0, H, ab, toks + p0, wts + p0, nt, yacc);
  }
}

__device__ void down_dispatch(const uint16_t *w2e, int F, int i0, int H, const float *act0, const int *toks,
                              const float *wts, int cnt, float *yacc) {
  switch (F) {
    case 32: down_slot<4>(w2e, F, i0, H, act0, toks, wts, cnt, yacc); break;
    case 64: down_slot<8>(w2e, F, i0, H, act0, toks, wts, cnt, yacc); break;
    case 128: down_slot<16>(w2e, F, i0, H, act0, toks, wts, cnt, yacc); break;
    default: down_slot<32>(w2e, F, i0, H, act0, toks, wts, cnt, yacc); break;  // 256
  }
}

__global__ void __launch_bounds__(kBlock) down_kernel(DownArgs a) {
  __shared__ float yacc[4][kMaxBatch * kDownRows];
  __shared__ int s_iota[kMaxBatch];
  __shared__ float s_one[kMaxBatch];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int i0 = blockIdx.x * kDownRows;
  for (int q = tid; q < 4 * kMaxBatch * kDownRows; q += kBlock) (&yacc[0][0])[q] = 0.f;
  if (tid < kMaxBatch) { s_iota[tid] = tid; s_one[tid] = 1.0f; }
  __syncthreads();
  const int n_active = *a.n_active;
  const int nslots = n_active + (a.Fs > 0 ? 1 : 0);
  for (int slot = wave; slot < nslots; slot += 4) {
    if (slot < n_active) {
      int e = a.act_exp[slot], cnt = a.act_cnt[slot], off = a.act_off[slot];
      down_dispatch(a.w2 + (size_t)e * a.H * a.F, a.F, i0, a.H, a.act + (size_t)off * a.F,
                    a.pair_tok + off, a.pair_w + off, cnt, yacc[wave]);
    } else {
      down_dispatch(a.s2, a.Fs, i0, a.H, a.act_s, s_iota, s_one, a.B, yacc[wave]);
    }
  }
  __syncthreads();
  for (int q = tid; q < a.B * kDownRows; q += kBlock) {
    int t = q / kDownRows, r = q % kDownRows;
    if (i0 + r < a.H) {
      int o = t * kDownRows + r;
      a.y[(size_t)t * a.H + i0 + r] = ((yacc[0][o] + yacc[1][o]) + yacc[2][o]) + yacc[3][o];
    }
  }
}

hipError_t launch_gateup(const GateUpArgs &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gateup_kernel, dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down(const DownArgs &a, hipStream_t s) {
  int grid = (a.H + kDownRows - 1) / kDownRows;
  hipLaunchKernelGGL(down_kernel, dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace dl
