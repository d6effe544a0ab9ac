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
constexpr int kMaxTopK = 64;
constexpr int kMaxBatch = 64;

// Single-launch path (fused.hip): one 512-thread workgroup per CU, all
// resident at once.  Limits of its LDS layout.
constexpr int kFusedThreads = 512;
constexpr int kFusedMaxB = 8;         // tokens
constexpr int kFusedMaxSlice = 32;    // rows of H per workgroup
constexpr int kFusedMaxPairs = 64;    // B * k
constexpr int kFusedBig = 8192;       // B * E logits, then B * k * F activations
constexpr int kFusedActS = 4096;      // B * Fs shared activations
constexpr int kFusedMaxH = 8192;      // router / shared rows held in registers
constexpr int kFusedMaxE = 512;       // experts (top-k candidates per lane)
constexpr int kFusedMaxGrid = 256;    // workgroups (one poll per control thread)
constexpr int kFusedQkvRows = 8;      // input-projection rows per workgroup
constexpr int kFusedW2Words = 4096;   // 16-byte words of down-projection rows staged in LDS (64 KB)

struct FusedArgs {
  const uint16_t *x, *w_qkv;
  float *qkv;
  const uint16_t *attn, *w_o, *gain;
  const float *resid_in;
  float *resid_out;
  const float *w_router;
  float *logits_out;
  int32_t *topk_idx;
  float *topk_w;
  const uint16_t *w1, *w3, *w2, *s1, *s3, *s2;
  float *moe_out, *h_out;
  // scratch: gained residual and the tagged hand-off arrays
  float *hg;          // [B][H]
  uint64_t *pss;      // [G][B]     partial sums of r1^2
  uint64_t *logit;    // [B][E]
  uint64_t *act;      // [B*k][F]   routed SwiGLU activations, pairs grouped by expert
  uint64_t *act_s;    // [B][Fs]    shared SwiGLU activations
  unsigned *epoch;    // tag of the last step on this handle (0: none yet)
  unsigned *status;   // bit 0: a hand-off wait expired
  uint64_t *tag_base; // the hand-off slots (pss .. act_s, contiguous), cleared at the tag wrap
  size_t tag_words;
  unsigned *wrap;     // arrivals at the wrap step's grid barrier (monotonic)
  int B, H, Dq, Do, E, K, F, Fs;
  int slice;          // rows of H per workgroup, a multiple of 4
  float eps;
  int spin_limit;
  uint64_t *trace;    // optional [G][kTracePoints] wall-clock stamps (nullptr: off)
  // cross-layer prefetch: the dense weights of the next layer (same shapes);
  // pf_w_o == nullptr: off
  const uint16_t *pf_w_o, *pf_w_qkv, *pf_s1, *pf_s3, *pf_s2;
  const float *pf_w_router;
};
constexpr int kTracePoints = 16;

// Batched path (batched.hip): five launches for batches the single-launch
// path does not take (up to 64 tokens); MFMA wherever 16 or more tokens share
// a weight matrix.  Needs H % 512 == 0 and Do % 128 == 0.
constexpr int kBatchQkvSplit = 8;     // K splits of the attention input projection (at most)
constexpr int kBatchRtrExperts = 48;  // router experts per workgroup (3 tiles of 16)
constexpr int kBatchRtrK = 256;       // router K per workgroup
constexpr int kBatchMfmaMin = 16;     // an expert with at least this many tokens uses MFMA
constexpr int kBatchGuRows = 64;      // gate/up rows of W1 (and of W3) per matrix-core group
constexpr int kGuKc = 14;             // K steps (of 32) of one matrix-core gate/up work unit
// K chunks (units, and partial-sum slots) of one gate/up group.
constexpr int batch_gu_chunks(int H) { return (H / 32 + kGuKc - 1) / kGuKc; }
// Partial y tiles per 64-row group of the down projection: the most
// workgroups one group's units can be spread over with a grid of G.
constexpr int kDnMaxGrid = 512;  // workgroups of the down launch at most
constexpr int batch_dn_slots(int H) { return (kDnMaxGrid + H / 64 - 1) / (H / 64) + 2; }
constexpr int kGuSlotFloatsR = 2 * 4 * 16 * 16;  // [W1 | W3][16-row tile][row][token], one 16-token chunk
constexpr int kBatchLaunches = 5;

struct BatchArgs {
  const uint16_t *x, *w_qkv;
  float *qkv;
  const uint16_t *attn, *w_o, *gain;
  const float *resid_in;
  float *resid_out;
  const float *w_router;
  float *logits_out;
  int32_t *topk_idx;
  float *topk_w;
  const uint16_t *w1, *w3, *w2, *s1, *s3, *s2;
  float *moe_out, *h_out;
  // scratch
  float *hg;          // [B][H]        g * r1
  float *ss_part;     // [H/64][B]     partial sums of r1^2 per out-projection workgroup
  float *qkv_part;    // [qkv_split][B][Dq]
  float *rlog_part;   // [H/kBatchRtrK][B][E]  router dot products per K chunk
  float *hn;          // [B][H]        normalised h (fp32)
  uint16_t *hp;       // [2][B][H]     h as bf16 hi + lo planes (MFMA operands)
  float *act;         // [B*k][F]      routed SwiGLU activations, pairs grouped by expert
  float *act_s;       // [B][Fs]
  int *n_active;      // [1]
  int *act_exp, *act_cnt, *act_off;  // [E] per active slot
  int *pair_tok;      // [B*k]
  float *pair_w;      // [B*k]
  int *gu_q;          // [4 E] gate/up work lists: matrix-core entries slot | (16-token chunk << 16),
                      //       then VALU entries (slot)
  int *n_q;           // [2]   their lengths
  float *gu_part;     // [routed groups][K chunks][kGuSlotFloatsR] partial gate/up sums
  float *gu_part_s;   // [shared groups][K chunks][kGuSlotFloatsR]
  unsigned *gu_cnt;   // [routed groups] arrivals of a group's units (re-armed by the last)
  unsigned *gu_cnt_s; // [shared groups]
  int gu_grid;        // workgroups of the gate/up and down launches (two per CU)
  float *dn_part;     // [H/64][dn_slots][64][64] partial y tiles of the down projection
  unsigned *dn_cnt;   // [H/64] arrivals of a row group's workgroups (re-armed by the last)
  int dn_slots;       // batch_dn_slots(H)
  unsigned *gu_done;  // [1] gate/up workgroups finished (re-armed by the last)
  int *dn_runs;       // [kDnMaxGrid + 3]: a group's unit cost, its cost before its last entry, first unit of each run
  unsigned *counter;  // [1] arrivals of the top-k workgroups (re-armed by the last)
  int B, H, Dq, Do, E, K, F, Fs;
  int qkv_split;      // K splits of the input projection: 8 when H % 1024 == 0, else 4
  float eps;
};

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
hipError_t launch_fused(const FusedArgs &a, int grid, hipStream_t s);
// ev: kBatchLaunches event pairs recorded around the launches, or nullptr.
hipError_t launch_batched(const BatchArgs &a, hipStream_t s, hipEvent_t (*ev)[2]);
// Resident workgroups of the single-launch kernel per CU (0 if it cannot run).
int fused_blocks_per_cu();

}  // namespace dl
