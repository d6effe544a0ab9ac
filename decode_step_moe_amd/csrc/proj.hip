// Launch 1 of the step: the attention input projection and the attention
// output projection fused with the residual add and the RMSNorm statistics,
// as one horizontally fused grid.
//
// Workgroups [0, nblk_o) own 16 rows of Wo each:
//   r1[t, i] = r[t, i] + sum_j attn[t, j] Wo[i, j]      -> resid_out
//   hg[t, i] = g[i] r1[t, i]                            -> scratch (gained, not yet normalised)
//   per-workgroup partial sum of r1^2 per token         -> ss_part
// and the last of them to finish turns the partials into
//   inv_rms[t] = 1 / sqrt(sum_i r1[t, i]^2 / H + eps).
// Consumers form h = hg * inv_rms on the fly (h = g r1 / rms(r1)).
// (Out-projection into the residual work: wireai.ir "vLLM's speed jump on
// NVIDIA Blackwell servers; record 842 tokens/s for Kimi K3", section "Four
// key changes behind the jump", bullet 2; the cross-GPU reduction between
// them is the identity on one shard.)
//
// Workgroups [nblk_o, nblk_o + nblk_qkv) own 2 rows of Wqkv each and split
// K = H over their 4 waves, reducing through LDS (the split-K form the same
// section's bullet 1 uses beyond two tokens; at one or two tokens it is the
// same loop with a single token chunk):
//   qkv[t, j] = sum_i x[t, i] Wqkv[j, i].
#include "common.h"
#include "kernels.h"

namespace dl {

template <int NT>
__device__ void qkv_chunk(const ProjArgs &a, int j0, int t0, int nt, float (&red)[4][kQkvRowsPerBlock][kTokChunk]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t *w[kQkvRowsPerBlock];
#pragma unroll
  for (int r = 0; r < kQkvRowsPerBlock; ++r) {
    int j = min(j0 + r, a.Dq - 1);
    w[r] = a.w_qkv + (size_t)j * a.H;
  }
  struct Act {
    const uint16_t *base; int ld; int tmax;
    __device__ __forceinline__ void load8(int t, int k, float (&v)[8]) const {
      int tt = t < tmax ? t : tmax;
      unpack8(ld16(base + (size_t)tt * ld + k), v);
    }
  } act{a.x + (size_t)t0 * a.H, a.H, nt - 1};
  float acc[kQkvRowsPerBlock][NT] = {};
  stream_rows_bf16<kQkvRowsPerBlock, NT, 2>(w, act, (wave * 64 + lane) * 8, kBlock * 8, a.H, acc);
#pragma unroll
  for (int r = 0; r < kQkvRowsPerBlock; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float v = wave_sum(acc[r][t]);
      if (lane == 0) red[wave][r][t] = v;
    }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < kQkvRowsPerBlock * nt) {
    int r = tid / nt, t = tid % nt;
    int j = j0 + r;
    if (j < a.Dq) {
      float v = red[0][r][t] + red[1][r][t] + red[2][r][t] + red[3][r][t];
      a.qkv[(size_t)(t0 + t) * a.Dq + j] = v;
    }
  }
  __syncthreads();
}

template <int NT>
__device__ void oproj_chunk(const ProjArgs &a, int i0, int t0, int nt,
                            float (&ored)[kORowsPerBlock][kTokChunk], float *ssum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t *w[kORowsPerWave];
#pragma unroll
  for (int r = 0; r < kORowsPerWave; ++r) {
    int i = min(i0 + wave * kORowsPerWave + r, a.H - 1);
    w[r] = a.w_o + (size_t)i * a.Do;
  }
  struct Act {
    const uint16_t *base; int ld; int tmax;
    __device__ __forceinline__ void load8(int t, int k, float (&v)[8]) const {
      int tt = t < tmax ? t : tmax;
      unpack8(ld16(base + (size_t)tt * ld + k), v);
    }
  } act{a.attn + (size_t)t0 * a.Do, a.Do, nt - 1};
  float acc[kORowsPerWave][NT] = {};
  stream_rows_bf16<kORowsPerWave, NT, 2>(w, act, lane * 8, kWave * 8, a.Do, acc);
#pragma unroll
  for (int r = 0; r < kORowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float v = wave_sum(acc[r][t]);
      if (lane == 0) ored[wave * kORowsPerWave + r][t] = v;
    }
  __syncthreads();
  // one thread per (row, token): residual add, gained copy, r1^2
  const int tid = threadIdx.x;
  if (tid < kORowsPerBlock * nt) {
    int rl = tid / nt, t = tid % nt;
    int i = i0 + rl;
    float sq = 0.f;
    if (i < a.H) {
      size_t o = (size_t)(t0 + t) * a.H + i;
      float r1 = a.resid_in[o] + ored[rl][t];
      a.resid_out[o] = r1;
      a.hg[o] = bf16_lo(a.gain[i]) * r1;
      sq = r1 * r1;
    }
    ored[rl][t] = sq;  // reuse: this slot is read only by this thread above
  }
  __syncthreads();
  if (tid < nt) {  // fixed-order sum over the block's 16 rows
    float s = 0.f;
    for (int rl = 0; rl < kORowsPerBlock; ++rl) s += ored[rl][tid];
    ssum[t0 + tid] = s;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kBlock) proj_kernel(ProjArgs a) {
  __shared__ float red[4][kQkvRowsPerBlock][kTokChunk];
  __shared__ float ored[kORowsPerBlock][kTokChunk];
  __shared__ float ssum[kMaxBatch];
  __shared__ int last_flag;
  const int b = blockIdx.x;
  if (b < a.nblk_o) {
    const int i0 = b * kORowsPerBlock;
    for (int t0 = 0; t0 < a.B; t0 += kTokChunk) {
      int nt = min(kTokChunk, a.B - t0);
      if (nt == 1) oproj_chunk<1>(a, i0, t0, nt, ored, ssum);
      else if (nt == 2) oproj_chunk<2>(a, i0, t0, nt, ored, ssum);
      else if (nt <= 4) oproj_chunk<4>(a, i0, t0, nt, ored, ssum);
      else oproj_chunk<8>(a, i0, t0, nt, ored, ssum);
    }
    if (threadIdx.x < a.B) a.ss_part[(size_t)b * a.B + threadIdx.x] = ssum[threadIdx.x];
    if (arrive_last(a.counter, a.nblk_o, &last_flag)) {
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      for (int t = wave; t < a.B; t += 4) {
        float s = 0.f;
        for (int q = lane; q < a.nblk_o; q += 64) s += a.ss_part[(size_t)q * a.B + t];
        s = wave_sum(s);
        if (lane == 0) a.inv_rms[t] = 1.0f / sqrtf(s / (float)a.H + a.eps);
      }
    }
  } else {
    const int j0 = (b - a.nblk_o) * kQkvRowsPerBlock;
    for (int t0 = 0; t0 < a.B; t0 += kTokChunk) {
      int nt = min(kTokChunk, a.B - t0);
      if (nt == 1) qkv_chunk<1>(a, j0, t0, nt, red);
      else if (nt == 2) qkv_chunk<2>(a, j0, t0, nt, red);
      else if (nt <= 4) qkv_chunk<4>(a, j0, t0, nt, red);
      else qkv_chunk<8>(a, j0, t0, nt, red);
    }
  }
}

hipError_t launch_proj(const ProjArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(proj_kernel, dim3(a.nblk_o + a.nblk_qkv), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace dl
