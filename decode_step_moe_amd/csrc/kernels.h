// Kernel argument blocks and launchers of the decode-layer step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dl {

// Out-projection rows per workgroup (4 waves x 4 rows) and attention-input
// projection rows per workgroup (split-K over the 4 waves).
constexpr int kORowsPerWave = 4;
constexpr int kORowsPerBlock = kORowsPerWave * 4;
constexpr int kQkvRowsPerBlock = 2;
// Gate/up: one ffn row pair (W1 row f, W3 row f) per wave.
constexpr int kGateRowsPerBlock = 4;
// Down projection: output rows of H per workgroup.
constexpr int kDownRows = 16;
// Token chunk handled per pass by the VALU paths.
constexpr int kTokChunk = 8;
// Router tail limits (LDS sizing).
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxBatch = 64;

struct ProjArgs {
  const uint16_t *x, *w_qkv;
  float *qkv;
  const uint16_t *attn, *w_o, *gain;
  const float *resid_in;
  float *resid_out, *hg, *ss_part, *inv_rms;
  unsigned *counter;
  int B, H, Dq, Do;
  float eps;
  int nblk_o, nblk_qkv;
};

struct RouterArgs {
  const float *w_router, *hg, *inv_rms;
  float *logits, *logits_out, *h_out;
  int32_t *topk_idx;
  float *topk_w;
  int *n_active, *act_exp, *act_cnt, *act_off, *pair_tok;
  float *pair_w;
  unsigned *counter;
  int B, H, E, K;
};

struct GateUpArgs {
  const uint16_t *w1, *w3;      // routed [E][F][H] or shared [F][H]
  const float *hg, *inv_rms;
  float *act;                   // routed [pairs][F] or shared [B][F]
  const int *n_active, *act_exp, *act_cnt, *act_off, *pair_tok;
  int B, H, F, shared;
};

struct DownArgs {
  const uint16_t *w2;           // routed [E][H][F]
  const uint16_t *s2;           // shared [H][Fs] or nullptr
  const float *act, *act_s, *pair_w;
  const int *n_active, *act_exp, *act_cnt, *act_off, *pair_tok;
  float *y;
  int B, H, F, Fs;
};

hipError_t launch_proj(const ProjArgs &a, hipStream_t s);
hipError_t launch_router(const RouterArgs &a, hipStream_t s);
hipError_t launch_gateup(const GateUpArgs &a, int grid, hipStream_t s);
hipError_t launch_down(const DownArgs &a, hipStream_t s);

}  // namespace dl
