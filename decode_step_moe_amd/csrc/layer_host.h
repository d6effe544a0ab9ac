// Host-side pieces of the library shared by its C-ABI source files: the
// execution-path plan, the scratch layout and the launch sequence of one
// step.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "../../include/decode_layer.h"
#include "kernels.h"

namespace dl {
namespace host {

constexpr int kDefaultSpinLimit = 1 << 20;  // polling rounds of a hand-off wait: about a second

// Single-launch path: grid size and the largest batch its LDS layout allows.
struct SinglePlan {
  int grid = 0;       // workgroups = CUs
  int slice = 0;      // rows of H per workgroup
  int max_batch = 0;  // 0: path unavailable
};

struct Scratch {
  // hand-off state: tagged words, counters (configuration-independent offsets)
  uint64_t *pss = nullptr, *logit = nullptr, *act64 = nullptr, *act_s64 = nullptr;
  unsigned *epoch = nullptr;     // [1] tag of the last single-launch step
  unsigned *status = nullptr;    // [1]
  unsigned *wrap = nullptr;      // [1] arrivals at the tag-wrap grid barrier
  unsigned *counters = nullptr;  // [4]: out-projection, router, batched top-k, batched gate/up finished
  unsigned *gu_cnt = nullptr;    // routed group counters, then shared group counters
  unsigned *dn_cnt = nullptr;    // [H/64]
  size_t tag_words = 0;          // 64-bit words from pss to the end of act_s64
  // step data, written before it is read within every step
  float *hg = nullptr;        // [maxB][H]   g * r1
  float *ss_part = nullptr;   // [nblk_o][maxB]
  float *inv_rms = nullptr;   // [maxB]
  float *logits = nullptr;    // [maxB][E]
  int *pair_tok = nullptr;    // [maxB*k]
  float *pair_w = nullptr;    // [maxB*k]
  int *act_exp = nullptr;     // [E]
  int *act_cnt = nullptr;     // [E]
  int *act_off = nullptr;     // [E]
  int *n_active = nullptr;    // [1]
  float *act = nullptr;       // [maxB*k][F]
  float *act_s = nullptr;     // [maxB][Fs]
  // batched path (empty when no step can take it)
  float *qkv_part = nullptr;     // [kBatchQkvSplit][maxB][Dq]
  float *rlog_part = nullptr;    // [H/kBatchRtrK][maxB][E]
  float *hn = nullptr;           // [maxB][H]
  uint16_t *hp = nullptr;        // [2][maxB][H]
  int *gu_q = nullptr;           // [4 E] gate/up work lists
  int *n_q = nullptr;            // [2]
  float *gu_part = nullptr;      // routed group slots, then shared group slots
  float *dn_part = nullptr;      // [H/64][dn slots][64][64] partial y tiles
  int *dn_runs = nullptr;        // [kDnMaxGrid + 3] down-projection run bounds
};

// the most gate/up groups and down row groups any configuration in the envelope has
constexpr size_t kMaxGuGroups = (size_t)(kMaxBatch * kMaxTopK + 7) / 8 * (256 / 32) + (kMaxBatch + 15) / 16 * (256 / 32);
constexpr size_t kMaxDnGroups = 16384 / 64;

// Scratch layout.  The hand-off state - tagged words that may only ever hold
// tags of earlier steps, and arrival counters that start every step at zero -
// comes first, at offsets and sizes that do not depend on the configuration,
// so that calls with different configurations sharing one scratch area never
// mistake one another's data for their own.  Everything after it is written
// before it is read within a step.
enum Buf {
  kBPss, kBLogit64, kBAct64, kBActS64, kBEpoch, kBStatus, kBWrap, kBCounters, kBGuCnt, kBDnCnt,
  kBHg, kBSsPart, kBInvRms, kBLogits, kBPairTok, kBPairW, kBActExp, kBActCnt, kBActOff, kBNActive,
  kBAct, kBActS, kBQkvPart, kBRlogPart, kBHn, kBHp, kBGuQ, kBNQ, kBGuPart, kBDnPart, kBDnRuns, kNumBuf
};
struct Layout {
  size_t off[kNumBuf];
  size_t total;
};

// Everything one step needs besides its per-step I/O.
struct StepCtx {
  const decode_layer_config *c;
  const decode_layer_weights *w;
  const Scratch *s;
  const SinglePlan *single;
  int gu_grid;
  hipStream_t side;            // second stream of the multi-launch path (nullptr: the caller's stream)
  hipEvent_t ev_fork, ev_join;
  int spin_limit;
  void *trace;
  const decode_layer_weights *prefetch;  // next layer's weights to prefetch (nullptr: none)
  decode_layer *h;             // error text and profiling (nullptr: thread-local error, no profiling)
};

SinglePlan plan_single(const decode_layer_config &c, int n_cu);
bool batched_ok(const decode_layer_config &c);
Layout layout_of(const decode_layer_config &c, const SinglePlan &sp);
Scratch bind_scratch(char *base, const Layout &L);
int cu_count(int device);
// Sets the error text of `h` (or the calling thread's when h is NULL) and returns `code`.
int fail(decode_layer *h, int code, const char *fmt, ...);
int check_config(const decode_layer_config *c, decode_layer *h);
int check_weights(const decode_layer_config *c, const decode_layer_weights *w, decode_layer *h);
int check_io(const decode_layer_config *c, const decode_layer_io *io, decode_layer *h);
// Enqueues one step of batch io->batch >= 1 on `st` (validated already).
int enqueue_step(const StepCtx &x, const decode_layer_io *io, hipStream_t st);

}  // namespace host
}  // namespace dl
