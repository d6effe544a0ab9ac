// Host side of the C ABI declared in include/decode_layer.h: validation,
// the handle (scratch, second stream, events), the static scratch of the
// entry point that allocates nothing, and the launch sequence of one step.
// Nothing here computes layer math; every step of the layer runs in the
// kernels of fused.hip, batched.hip, proj.hip, router.hip and experts.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>
#include <new>
#include <string>

#include "../../include/decode_layer.h"
#include "kernels.h"
#include "layer_host.h"

using namespace dl;

namespace dl {
namespace host {

thread_local std::string g_thread_err = "no error";

int single_max_batch_for(const decode_layer_config &c, int grid, int slice) {
  if (grid < 1 || grid > kFusedMaxGrid || slice > kFusedMaxSlice) return 0;
  // each workgroup computes at most kFusedQkvRows rows of the input projection
  if (c.qkv_out > kFusedQkvRows * grid) return 0;
  // each workgroup holds at most 2 router rows in LDS
  if (c.hidden > kFusedMaxH || c.n_experts > kFusedMaxE || c.n_experts > 2 * grid) return 0;
  if (c.shared_ffn != 0 && c.shared_ffn != c.expert_ffn) return 0;
  int best = 0;
  for (int b = 1; b <= kFusedMaxB && b <= c.max_batch; ++b) {
    if (b * c.top_k > kFusedMaxPairs || b * c.n_experts > kFusedBig ||
        b * c.top_k * c.expert_ffn > kFusedBig || b * c.shared_ffn > kFusedActS)
      break;
    best = b;
  }
  return best;
}

SinglePlan plan_single(const decode_layer_config &c, int n_cu) {
  SinglePlan p;
  if (c.path == DL_PATH_MULTI || c.path == DL_PATH_BATCHED || n_cu < 1) return p;
  p.grid = n_cu;
  int sl = (c.hidden + n_cu - 1) / n_cu;
  p.slice = (sl + 3) & ~3;
  p.max_batch = single_max_batch_for(c, p.grid, p.slice);
  return p;
}

// Batched path: shape requirements of its tilings (K splits of 4 waves x 32
// for the projections and gate/up, 256-wide router K chunks).
bool batched_ok(const decode_layer_config &c) { return c.hidden % 512 == 0 && c.attn_dim % 128 == 0; }

// Whether some step of this configuration takes the batched path.
bool batched_used(const decode_layer_config &c, const SinglePlan &sp) {
  if (c.path == DL_PATH_BATCHED) return true;
  return c.path == DL_PATH_AUTO && batched_ok(c) && c.max_batch > sp.max_batch;
}

// Batched gate/up matrix-core groups: 16-token chunks of the routed experts
// with >= 16 tokens (at most B*k/8 chunks) times the row groups of one
// expert, and the shared expert's 16-token chunks (at most 4) times its row
// groups.
size_t gu_groups_routed(const decode_layer_config &c) {
  return ((size_t)c.max_batch * c.top_k + 7) / 8 * (c.expert_ffn / std::min(kBatchGuRows, c.expert_ffn));
}
size_t gu_groups_shared(const decode_layer_config &c) {
  return c.shared_ffn > 0 ? (size_t)(c.max_batch + 15) / 16 * (c.shared_ffn / std::min(kBatchGuRows, c.shared_ffn)) : 0;
}
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int nblk_o_of(const decode_layer_config &c) { return (c.hidden + kORowsPerBlock - 1) / kORowsPerBlock; }

Layout layout_of(const decode_layer_config &c, const SinglePlan &sp) {
  const size_t B = c.max_batch, H = c.hidden, E = c.n_experts, K = c.top_k;
  const size_t Bb = batched_used(c, sp) ? B : 0;
  (void)sp;
  const size_t sizes[kNumBuf] = {
      // hand-off state
      (size_t)kFusedMaxGrid * kFusedMaxB * 8, (size_t)kFusedBig * 8, (size_t)kFusedBig * 8, (size_t)kFusedActS * 8,
      4, 4, 4, 4 * 4, kMaxGuGroups * 4, kMaxDnGroups * 4,
      // step data
      B * H * 4, (size_t)nblk_o_of(c) * B * 4, B * 4, B * E * 4, B * K * 4, B * K * 4,
      E * 4, E * 4, E * 4, 4, B * K * (size_t)c.expert_ffn * 4, B * (size_t)(c.shared_ffn > 0 ? c.shared_ffn : 1) * 4,
      // batched arrays
      (size_t)kBatchQkvSplit * Bb * c.qkv_out * 4, (H / kBatchRtrK) * Bb * E * 4, Bb * H * 4, 2 * Bb * H * 2,
      Bb ? 4 * E * 4 : size_t(0), Bb ? size_t(8) : size_t(0),
      Bb ? (gu_groups_routed(c) + gu_groups_shared(c)) * batch_gu_chunks(c.hidden) * kGuSlotFloatsR * 4 : size_t(0),
      Bb ? (H / 64) * batch_dn_slots(c.hidden) * kMaxBatch * 64 * 4 : size_t(0), Bb ? (kDnMaxGrid + 3) * 4 : size_t(0)};
  Layout L;
  size_t o = 0;
  for (int i = 0; i < kNumBuf; ++i) { L.off[i] = o; o += align256(sizes[i]); }
  L.total = o;
  return L;
}

Scratch bind_scratch(char *b, const Layout &L) {
  Scratch s;
  s.pss = (uint64_t *)(b + L.off[kBPss]);
  s.logit = (uint64_t *)(b + L.off[kBLogit64]);
  s.act64 = (uint64_t *)(b + L.off[kBAct64]);
  s.act_s64 = (uint64_t *)(b + L.off[kBActS64]);
  s.epoch = (unsigned *)(b + L.off[kBEpoch]);
  s.status = (unsigned *)(b + L.off[kBStatus]);
  s.wrap = (unsigned *)(b + L.off[kBWrap]);
  s.counters = (unsigned *)(b + L.off[kBCounters]);
  s.gu_cnt = (unsigned *)(b + L.off[kBGuCnt]);
  s.dn_cnt = (unsigned *)(b + L.off[kBDnCnt]);
  s.tag_words = (L.off[kBEpoch] - L.off[kBPss]) / 8;
  s.hg = (float *)(b + L.off[kBHg]);
  s.ss_part = (float *)(b + L.off[kBSsPart]);
  s.inv_rms = (float *)(b + L.off[kBInvRms]);
  s.logits = (float *)(b + L.off[kBLogits]);
  s.pair_tok = (int *)(b + L.off[kBPairTok]);
  s.pair_w = (float *)(b + L.off[kBPairW]);
  s.act_exp = (int *)(b + L.off[kBActExp]);
  s.act_cnt = (int *)(b + L.off[kBActCnt]);
  s.act_off = (int *)(b + L.off[kBActOff]);
  s.n_active = (int *)(b + L.off[kBNActive]);
  s.act = (float *)(b + L.off[kBAct]);
  s.act_s = (float *)(b + L.off[kBActS]);
  s.qkv_part = (float *)(b + L.off[kBQkvPart]);
  s.rlog_part = (float *)(b + L.off[kBRlogPart]);
  s.hn = (float *)(b + L.off[kBHn]);
  s.hp = (uint16_t *)(b + L.off[kBHp]);
  s.gu_q = (int *)(b + L.off[kBGuQ]);
  s.n_q = (int *)(b + L.off[kBNQ]);
  s.gu_part = (float *)(b + L.off[kBGuPart]);
  s.dn_part = (float *)(b + L.off[kBDnPart]);
  s.dn_runs = (int *)(b + L.off[kBDnRuns]);
  return s;
}

int cu_count(int device) {
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
  return n;
}

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace host
}  // namespace dl

using namespace dl::host;

struct decode_layer {
  decode_layer_config cfg;
  decode_layer_weights w;
  int device = 0;
  void *scratch_base = nullptr;
  Scratch s;
  SinglePlan single;
  int gu_grid = 0;         // workgroups of the batched gate/up launch
  int spin_limit = kDefaultSpinLimit;
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  void *trace = nullptr;   // caller's device buffer for the phase trace
  bool has_next = false;   // cross-layer prefetch of next_w
  decode_layer_weights next_w{};
  bool profiling = false;
  bool profiled_step = false;
  hipEvent_t ev_prof[DECODE_LAYER_N_LAUNCHES][2] = {};
  bool launched[DECODE_LAYER_N_LAUNCHES] = {};
  std::string err = "no error";
};

namespace dl {
namespace host {

// Event pair around launch `i` when profiling is on (h may be NULL: no profiling).
struct ProfScope {
  decode_layer *h;
  int i;
  hipStream_t s;
  hipError_t begin() {
    if (!h || !h->profiling) return hipSuccess;
    h->launched[i] = true;
    return hipEventRecord(h->ev_prof[i][0], s);
  }
  hipError_t end() { return h && h->profiling ? hipEventRecord(h->ev_prof[i][1], s) : hipSuccess; }
};

int fail(decode_layer *h, int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (h) h->err = buf;
  g_thread_err = buf;
  return code;
}

int check_config(const decode_layer_config *c, decode_layer *h) {
  if (!c) return fail(h, DL_ERR_INVALID_ARG, "config is NULL");
  if (c->hidden < 8 || c->hidden > 16384 || c->hidden % 8)
    return fail(h, DL_ERR_UNSUPPORTED, "hidden=%d: need 8..16384 and a multiple of 8", c->hidden);
  if (c->qkv_out < 1 || c->qkv_out > 65536)
    return fail(h, DL_ERR_UNSUPPORTED, "qkv_out=%d: need 1..65536", c->qkv_out);
  if (c->attn_dim < 8 || c->attn_dim > 16384 || c->attn_dim % 8)
    return fail(h, DL_ERR_UNSUPPORTED, "attn_dim=%d: need 8..16384 and a multiple of 8", c->attn_dim);
  if (c->n_experts < 1 || c->n_experts > kMaxExperts)
    return fail(h, DL_ERR_UNSUPPORTED, "n_experts=%d: need 1..%d", c->n_experts, kMaxExperts);
  if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > kMaxTopK)
    return fail(h, DL_ERR_UNSUPPORTED, "top_k=%d: need 1..min(n_experts, %d)", c->top_k, kMaxTopK);
  if (c->expert_ffn < 32 || c->expert_ffn > 256 || !pow2(c->expert_ffn))
    return fail(h, DL_ERR_UNSUPPORTED, "expert_ffn=%d: need 32, 64, 128 or 256", c->expert_ffn);
  if (c->shared_ffn != 0 && (c->shared_ffn < 32 || c->shared_ffn > 256 || !pow2(c->shared_ffn)))
    return fail(h, DL_ERR_UNSUPPORTED, "shared_ffn=%d: need 0, 32, 64, 128 or 256", c->shared_ffn);
  if (c->max_batch < 1 || c->max_batch > kMaxBatch)
    return fail(h, DL_ERR_UNSUPPORTED, "max_batch=%d: need 1..%d", c->max_batch, kMaxBatch);
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps))
    return fail(h, DL_ERR_UNSUPPORTED, "rms_eps must be positive and finite");
  if (c->score_fn != 0) return fail(h, DL_ERR_UNSUPPORTED, "score_fn=%d: only 0 (sigmoid) is supported", c->score_fn);
  if (c->renormalize != 1)
    return fail(h, DL_ERR_UNSUPPORTED, "renormalize=%d: only 1 is supported", c->renormalize);
  if (c->path < DL_PATH_AUTO || c->path > DL_PATH_BATCHED)
    return fail(h, DL_ERR_UNSUPPORTED, "path=%d: need DL_PATH_AUTO, DL_PATH_MULTI, DL_PATH_SINGLE or DL_PATH_BATCHED",
                c->path);
  return DL_OK;
}

int check_weights(const decode_layer_config *c, const decode_layer_weights *w, decode_layer *h) {
  if (!w) return fail(h, DL_ERR_INVALID_ARG, "weights is NULL");
  const void *req[] = {w->w_qkv, w->w_o, w->norm_gain, w->w_router, w->w1, w->w3, w->w2};
  const char *names[] = {"w_qkv", "w_o", "norm_gain", "w_router", "w1", "w3", "w2"};
  for (int i = 0; i < 7; ++i) {
    if (!req[i]) return fail(h, DL_ERR_INVALID_ARG, "weights.%s is NULL", names[i]);
    if (!aligned16(req[i])) return fail(h, DL_ERR_INVALID_ARG, "weights.%s is not 16-byte aligned", names[i]);
  }
  const void *sh[] = {w->s1, w->s3, w->s2};
  const char *shn[] = {"s1", "s3", "s2"};
  for (int i = 0; i < 3; ++i) {
    if (c->shared_ffn > 0 && !sh[i]) return fail(h, DL_ERR_INVALID_ARG, "weights.%s is NULL but shared_ffn > 0", shn[i]);
    if (sh[i] && !aligned16(sh[i])) return fail(h, DL_ERR_INVALID_ARG, "weights.%s is not 16-byte aligned", shn[i]);
  }
  return DL_OK;
}

int check_io(const decode_layer_config *c, const decode_layer_io *io, decode_layer *h) {
  if (!io) return fail(h, DL_ERR_INVALID_ARG, "io is NULL");
  if (io->batch < 0) return fail(h, DL_ERR_INVALID_ARG, "batch=%d is negative", io->batch);
  if (io->batch > c->max_batch)
    return fail(h, DL_ERR_UNSUPPORTED, "batch=%d exceeds max_batch=%d", io->batch, c->max_batch);
  if (io->batch == 0) return DL_OK;
  const void *req[] = {io->x, io->attn, io->resid_in, io->qkv, io->resid_out, io->topk_idx, io->topk_w, io->moe_out};
  const char *names[] = {"x", "attn", "resid_in", "qkv", "resid_out", "topk_idx", "topk_w", "moe_out"};
  for (int i = 0; i < 8; ++i) {
    if (!req[i]) return fail(h, DL_ERR_INVALID_ARG, "io.%s is NULL", names[i]);
    if (!aligned16(req[i])) return fail(h, DL_ERR_INVALID_ARG, "io.%s is not 16-byte aligned", names[i]);
  }
  if (io->router_logits && !aligned16(io->router_logits))
    return fail(h, DL_ERR_INVALID_ARG, "io.router_logits is not 16-byte aligned");
  if (io->h_out && !aligned16(io->h_out)) return fail(h, DL_ERR_INVALID_ARG, "io.h_out is not 16-byte aligned");
  if (io->resid_out != io->resid_in) {
    // partial overlap of the residual buffers would race; exact aliasing is allowed
    const char *a0 = (const char *)io->resid_in, *b0 = (const char *)io->resid_out;
    size_t n = (size_t)io->batch * c->hidden * 4;
    if (a0 < b0 + n && b0 < a0 + n) return fail(h, DL_ERR_INVALID_ARG, "io.resid_out partially overlaps io.resid_in");
  }
  return DL_OK;
}

}  // namespace host
}  // namespace dl

#define HIP_TRY(h, expr)                                                                         \
  do {                                                                                           \
    hipError_t e_ = (expr);                                                                      \
    if (e_ != hipSuccess) return fail(h, DL_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

namespace dl {
namespace host {

int enqueue_step(const StepCtx &x, const decode_layer_io *io, hipStream_t st) {
  decode_layer *h = x.h;
  const decode_layer_config &c = *x.c;
  const decode_layer_weights &W = *x.w;
  const Scratch &S = *x.s;
  const int B = io->batch;
  const bool single = (c.path == DL_PATH_AUTO || c.path == DL_PATH_SINGLE) && B <= x.single->max_batch;
  if (c.path == DL_PATH_SINGLE && !single)
    return fail(h, DL_ERR_UNSUPPORTED, "batch=%d exceeds the single-launch limit %d", B, x.single->max_batch);
  const bool batched = !single && batched_used(c, *x.single);
  const bool prof = h && h->profiling;
  if (prof)
    for (int i = 0; i < DECODE_LAYER_N_LAUNCHES; ++i) h->launched[i] = false;
  if (single) {
    FusedArgs fa{};
    fa.x = (const uint16_t *)io->x;
    fa.w_qkv = (const uint16_t *)W.w_qkv;
    fa.qkv = io->qkv;
    fa.attn = (const uint16_t *)io->attn;
    fa.w_o = (const uint16_t *)W.w_o;
    fa.gain = (const uint16_t *)W.norm_gain;
    fa.resid_in = io->resid_in;
    fa.resid_out = io->resid_out;
    fa.w_router = W.w_router;
    fa.logits_out = io->router_logits;
    fa.topk_idx = io->topk_idx;
    fa.topk_w = io->topk_w;
    fa.w1 = (const uint16_t *)W.w1;
    fa.w3 = (const uint16_t *)W.w3;
    fa.w2 = (const uint16_t *)W.w2;
    fa.s1 = (const uint16_t *)W.s1;
    fa.s3 = (const uint16_t *)W.s3;
    fa.s2 = (const uint16_t *)W.s2;
    fa.moe_out = io->moe_out;
    fa.h_out = io->h_out;
    fa.hg = S.hg;
    fa.pss = S.pss;
    fa.logit = S.logit;
    fa.act = S.act64;
    fa.act_s = S.act_s64;
    fa.epoch = S.epoch;
    fa.status = S.status;
    fa.tag_base = S.pss;
    fa.tag_words = S.tag_words;
    fa.wrap = S.wrap;
    fa.B = B;
    fa.H = c.hidden;
    fa.Dq = c.qkv_out;
    fa.Do = c.attn_dim;
    fa.E = c.n_experts;
    fa.K = c.top_k;
    fa.F = c.expert_ffn;
    fa.Fs = c.shared_ffn;
    fa.slice = x.single->slice;
    fa.eps = c.rms_eps;
    fa.spin_limit = x.spin_limit;
    fa.trace = (uint64_t *)x.trace;
    if (x.prefetch) {
      fa.pf_w_o = (const uint16_t *)x.prefetch->w_o;
      fa.pf_w_qkv = (const uint16_t *)x.prefetch->w_qkv;
      fa.pf_s1 = (const uint16_t *)x.prefetch->s1;
      fa.pf_s3 = (const uint16_t *)x.prefetch->s3;
      fa.pf_s2 = (const uint16_t *)x.prefetch->s2;
      fa.pf_w_router = x.prefetch->w_router;
    }
    ProfScope p5{h, 5, st};
    HIP_TRY(h, p5.begin());
    HIP_TRY(h, launch_fused(fa, x.single->grid, st));
    HIP_TRY(h, p5.end());
    if (prof) h->profiled_step = true;
    return DL_OK;
  }
  if (batched) {
    BatchArgs ba{};
    ba.x = (const uint16_t *)io->x;
    ba.w_qkv = (const uint16_t *)W.w_qkv;
    ba.qkv = io->qkv;
    ba.attn = (const uint16_t *)io->attn;
    ba.w_o = (const uint16_t *)W.w_o;
    ba.gain = (const uint16_t *)W.norm_gain;
    ba.resid_in = io->resid_in;
    ba.resid_out = io->resid_out;
    ba.w_router = W.w_router;
    ba.logits_out = io->router_logits;
    ba.topk_idx = io->topk_idx;
    ba.topk_w = io->topk_w;
    ba.w1 = (const uint16_t *)W.w1;
    ba.w3 = (const uint16_t *)W.w3;
    ba.w2 = (const uint16_t *)W.w2;
    ba.s1 = (const uint16_t *)W.s1;
    ba.s3 = (const uint16_t *)W.s3;
    ba.s2 = (const uint16_t *)W.s2;
    ba.moe_out = io->moe_out;
    ba.h_out = io->h_out;
    ba.hg = S.hg;
    ba.ss_part = S.ss_part;
    ba.qkv_part = S.qkv_part;
    ba.rlog_part = S.rlog_part;
    ba.hn = S.hn;
    ba.hp = S.hp;
    ba.act = S.act;
    ba.act_s = S.act_s;
    ba.n_active = S.n_active;
    ba.act_exp = S.act_exp;
    ba.act_cnt = S.act_cnt;
    ba.act_off = S.act_off;
    ba.pair_tok = S.pair_tok;
    ba.pair_w = S.pair_w;
    ba.gu_q = S.gu_q;
    ba.n_q = S.n_q;
    ba.gu_part = S.gu_part;
    ba.gu_part_s = S.gu_part + gu_groups_routed(c) * batch_gu_chunks(c.hidden) * kGuSlotFloatsR;
    ba.gu_cnt = S.gu_cnt;
    ba.gu_cnt_s = S.gu_cnt + gu_groups_routed(c);
    ba.gu_grid = x.gu_grid;
    ba.qkv_split = c.hidden % 1024 == 0 ? kBatchQkvSplit : kBatchQkvSplit / 2;
    ba.dn_part = S.dn_part;
    ba.dn_cnt = S.dn_cnt;
    ba.dn_slots = batch_dn_slots(c.hidden);
    ba.counter = S.counters + 2;
    ba.gu_done = S.counters + 3;
    ba.dn_runs = S.dn_runs;
    ba.B = B;
    ba.H = c.hidden;
    ba.Dq = c.qkv_out;
    ba.Do = c.attn_dim;
    ba.E = c.n_experts;
    ba.K = c.top_k;
    ba.F = c.expert_ffn;
    ba.Fs = c.shared_ffn;
    ba.eps = c.rms_eps;
    if (prof)
      for (int i = 0; i < kBatchLaunches; ++i) h->launched[6 + i] = true;
    HIP_TRY(h, launch_batched(ba, st, prof ? &h->ev_prof[6] : nullptr));
    if (prof) h->profiled_step = true;
    return DL_OK;
  }

  ProjArgs pa{};
  pa.x = (const uint16_t *)io->x;
  pa.w_qkv = (const uint16_t *)W.w_qkv;
  pa.qkv = io->qkv;
  pa.attn = (const uint16_t *)io->attn;
  pa.w_o = (const uint16_t *)W.w_o;
  pa.gain = (const uint16_t *)W.norm_gain;
  pa.resid_in = io->resid_in;
  pa.resid_out = io->resid_out;
  pa.hg = S.hg;
  pa.ss_part = S.ss_part;
  pa.inv_rms = S.inv_rms;
  pa.counter = S.counters + 0;
  pa.B = B;
  pa.H = c.hidden;
  pa.Dq = c.qkv_out;
  pa.Do = c.attn_dim;
  pa.eps = c.rms_eps;
  pa.nblk_o = nblk_o_of(c);
  pa.nblk_qkv = (c.qkv_out + kQkvRowsPerBlock - 1) / kQkvRowsPerBlock;
  ProfScope p0{h, 0, st};
  HIP_TRY(h, p0.begin());
  HIP_TRY(h, launch_proj(pa, st));
  HIP_TRY(h, p0.end());

  // the shared expert's gate/up on the second stream (forked from and joined
  // back into the caller's stream), or in order on the caller's stream
  const hipStream_t sst = x.side ? x.side : st;
  if (c.shared_ffn > 0) {
    if (x.side) {
      HIP_TRY(h, hipEventRecord(x.ev_fork, st));
      HIP_TRY(h, hipStreamWaitEvent(x.side, x.ev_fork, 0));
    }
    GateUpArgs ga{};
    ga.w1 = (const uint16_t *)W.s1;
    ga.w3 = (const uint16_t *)W.s3;
    ga.hg = S.hg;
    ga.inv_rms = S.inv_rms;
    ga.act = S.act_s;
    ga.B = B;
    ga.H = c.hidden;
    ga.F = c.shared_ffn;
    ga.shared = 1;
    ProfScope p1{h, 1, sst};
    HIP_TRY(h, p1.begin());
    HIP_TRY(h, launch_gateup(ga, c.shared_ffn / kGateRowsPerBlock, sst));
    HIP_TRY(h, p1.end());
    if (x.side) HIP_TRY(h, hipEventRecord(x.ev_join, x.side));
  }

  RouterArgs ra{};
  ra.w_router = W.w_router;
  ra.hg = S.hg;
  ra.inv_rms = S.inv_rms;
  ra.logits = S.logits;
  ra.logits_out = io->router_logits;
  ra.h_out = io->h_out;
  ra.topk_idx = io->topk_idx;
  ra.topk_w = io->topk_w;
  ra.n_active = S.n_active;
  ra.act_exp = S.act_exp;
  ra.act_cnt = S.act_cnt;
  ra.act_off = S.act_off;
  ra.pair_tok = S.pair_tok;
  ra.pair_w = S.pair_w;
  ra.counter = S.counters + 1;
  ra.B = B;
  ra.H = c.hidden;
  ra.E = c.n_experts;
  ra.K = c.top_k;
  ProfScope p2{h, 2, st};
  HIP_TRY(h, p2.begin());
  HIP_TRY(h, launch_router(ra, st));
  HIP_TRY(h, p2.end());

  GateUpArgs ga{};
  ga.w1 = (const uint16_t *)W.w1;
  ga.w3 = (const uint16_t *)W.w3;
  ga.hg = S.hg;
  ga.inv_rms = S.inv_rms;
  ga.act = S.act;
  ga.n_active = S.n_active;
  ga.act_exp = S.act_exp;
  ga.act_cnt = S.act_cnt;
  ga.act_off = S.act_off;
  ga.pair_tok = S.pair_tok;
  ga.B = B;
  ga.H = c.hidden;
  ga.F = c.expert_ffn;
  ga.shared = 0;
  {
    int max_active = B * c.top_k < c.n_experts ? B * c.top_k : c.n_experts;
    long items = (long)max_active * (c.expert_ffn / kGateRowsPerBlock);
    int grid = (int)(items < 2048 ? items : 2048);
    ProfScope p3{h, 3, st};
    HIP_TRY(h, p3.begin());
    HIP_TRY(h, launch_gateup(ga, grid, st));
    HIP_TRY(h, p3.end());
  }

  if (c.shared_ffn > 0 && x.side) HIP_TRY(h, hipStreamWaitEvent(st, x.ev_join, 0));

  DownArgs da{};
  da.w2 = (const uint16_t *)W.w2;
  da.s2 = (const uint16_t *)W.s2;
  da.act = S.act;
  da.act_s = S.act_s;
  da.pair_w = S.pair_w;
  da.n_active = S.n_active;
  da.act_exp = S.act_exp;
  da.act_cnt = S.act_cnt;
  da.act_off = S.act_off;
  da.pair_tok = S.pair_tok;
  da.y = io->moe_out;
  da.B = B;
  da.H = c.hidden;
  da.F = c.expert_ffn;
  da.Fs = c.shared_ffn;
  ProfScope p4{h, 4, st};
  HIP_TRY(h, p4.begin());
  HIP_TRY(h, launch_down(da, st));
  HIP_TRY(h, p4.end());
  if (prof) h->profiled_step = true;
  return DL_OK;
}

}  // namespace host
}  // namespace dl

extern "C" {

int decode_layer_check_config(const decode_layer_config *cfg) { return check_config(cfg, nullptr); }

int decode_layer_check_io(const decode_layer_config *cfg, const decode_layer_io *io) {
  int rc = check_config(cfg, nullptr);
  if (rc != DL_OK) return rc;
  return check_io(cfg, io, nullptr);
}

size_t decode_layer_scratch_bytes(const decode_layer_config *cfg, int n_cu) {
  if (check_config(cfg, nullptr) != DL_OK) return 0;
  return layout_of(*cfg, plan_single(*cfg, n_cu)).total;
}

const char *decode_layer_last_error(const decode_layer *h) {
  return h ? h->err.c_str() : g_thread_err.c_str();
}

int decode_layer_init(const decode_layer_config *cfg, const decode_layer_weights *w, int device,
                      decode_layer **out) {
  if (!out) return fail(nullptr, DL_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg, nullptr);
  if (rc != DL_OK) return rc;
  rc = check_weights(cfg, w, nullptr);
  if (rc != DL_OK) return rc;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0)
    return fail(nullptr, DL_ERR_HIP, "no HIP device available");
  if (device < 0 || device >= ndev) return fail(nullptr, DL_ERR_INVALID_ARG, "device %d out of range (%d devices)", device, ndev);
  decode_layer *h = new (std::nothrow) decode_layer;
  if (!h) return fail(nullptr, DL_ERR_OOM, "host allocation failed");
  h->cfg = *cfg;
  h->w = *w;
  h->device = device;
  auto cleanup = [&](int code) {
    g_thread_err = h->err;
    decode_layer_destroy(h);
    return code;
  };
  if (hipSetDevice(device) != hipSuccess) return cleanup(fail(h, DL_ERR_HIP, "hipSetDevice(%d) failed", device));
  h->single = plan_single(*cfg, cu_count(device));
  if (h->single.max_batch > 0 && fused_blocks_per_cu() < 1) h->single = SinglePlan{};
  if (cfg->path == DL_PATH_SINGLE && h->single.max_batch == 0)
    return cleanup(fail(h, DL_ERR_UNSUPPORTED, "the single-launch path cannot run this configuration on this device"));
  if (cfg->path == DL_PATH_BATCHED && !batched_ok(*cfg))
    return cleanup(fail(h, DL_ERR_UNSUPPORTED,
                        "the batched path needs hidden %% 512 == 0 and attn_dim %% 128 == 0 (hidden=%d, attn_dim=%d)",
                        cfg->hidden, cfg->attn_dim));
  Layout L = layout_of(*cfg, h->single);
  if (hipMalloc(&h->scratch_base, L.total) != hipSuccess) {
    h->scratch_base = nullptr;
    return cleanup(fail(h, DL_ERR_OOM, "hipMalloc of %zu scratch bytes failed", L.total));
  }
  h->s = bind_scratch((char *)h->scratch_base, L);
  h->gu_grid = 2 * std::max(1, cu_count(device));
  // The hand-off counters start at zero and are re-armed by the kernels
  // themselves, and the tagged hand-off values start with tag 0, which no
  // step uses, so no step ever needs a memset.
  if (hipMemset(h->scratch_base, 0, L.total) != hipSuccess) return cleanup(fail(h, DL_ERR_HIP, "hipMemset failed"));
  if (hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess) {
    h->side = nullptr;
    return cleanup(fail(h, DL_ERR_HIP, "hipStreamCreateWithFlags failed"));
  }
  if (hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess) {
    h->ev_fork = nullptr;
    return cleanup(fail(h, DL_ERR_HIP, "hipEventCreate failed"));
  }
  if (hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess) {
    h->ev_join = nullptr;
    return cleanup(fail(h, DL_ERR_HIP, "hipEventCreate failed"));
  }
  if (hipDeviceSynchronize() != hipSuccess) return cleanup(fail(h, DL_ERR_HIP, "hipDeviceSynchronize failed"));
  *out = h;
  return DL_OK;
}

int decode_layer_step(decode_layer *h, const decode_layer_io *io, void *hip_stream) {
  if (!h) return fail(nullptr, DL_ERR_INVALID_ARG, "handle is NULL");
  int rc = check_io(&h->cfg, io, h);
  if (rc != DL_OK) return rc;
  if (io->batch == 0) return DL_OK;
  HIP_TRY(h, hipSetDevice(h->device));
  const StepCtx x{&h->cfg, &h->w, &h->s, &h->single, h->gu_grid, h->side, h->ev_fork, h->ev_join,
                  h->spin_limit, h->trace, h->has_next ? &h->next_w : nullptr, h};
  return enqueue_step(x, io, (hipStream_t)hip_stream);
}

int decode_layer_single_max_batch(const decode_layer *h) { return h ? h->single.max_batch : 0; }

int decode_layer_status(decode_layer *h, uint32_t *status, int clear) {
  if (!h || !status) return fail(h, DL_ERR_INVALID_ARG, "NULL handle or output");
  HIP_TRY(h, hipSetDevice(h->device));
  unsigned v = 0;
  HIP_TRY(h, hipMemcpy(&v, h->s.status, sizeof v, hipMemcpyDeviceToHost));
  *status = v;
  if (clear && v) {
    unsigned zero = 0;
    HIP_TRY(h, hipMemcpy(h->s.status, &zero, sizeof zero, hipMemcpyHostToDevice));
  }
  return DL_OK;
}

int decode_layer_set_spin_limit(decode_layer *h, int rounds) {
  if (!h) return fail(nullptr, DL_ERR_INVALID_ARG, "handle is NULL");
  if (rounds < 0) return fail(h, DL_ERR_INVALID_ARG, "rounds=%d is negative", rounds);
  h->spin_limit = rounds;
  return DL_OK;
}

int decode_layer_set_step_counter(decode_layer *h, uint32_t last_tag) {
  if (!h) return fail(nullptr, DL_ERR_INVALID_ARG, "handle is NULL");
  HIP_TRY(h, hipSetDevice(h->device));
  HIP_TRY(h, hipDeviceSynchronize());
  HIP_TRY(h, hipMemcpy(h->s.epoch, &last_tag, sizeof last_tag, hipMemcpyHostToDevice));
  return DL_OK;
}

int decode_layer_set_prefetch(decode_layer *h, const decode_layer *next) {
  if (!h) return fail(nullptr, DL_ERR_INVALID_ARG, "handle is NULL");
  if (!next) {
    h->has_next = false;
    return DL_OK;
  }
  if (next->device != h->device || std::memcmp(&next->cfg, &h->cfg, sizeof h->cfg) != 0)
    return fail(h, DL_ERR_INVALID_ARG, "the next layer's handle must have the same configuration and device");
  h->next_w = next->w;
  h->has_next = true;
  return DL_OK;
}

int decode_layer_set_trace(decode_layer *h, void *device_buffer) {
  if (!h) return fail(nullptr, DL_ERR_INVALID_ARG, "handle is NULL");
  if (device_buffer && !aligned16(device_buffer))
    return fail(h, DL_ERR_INVALID_ARG, "trace buffer is not 16-byte aligned");
  h->trace = device_buffer;
  return DL_OK;
}

int decode_layer_trace_points(void) { return kTracePoints; }

int decode_layer_grid(const decode_layer *h) { return h ? h->single.grid : 0; }

int decode_layer_set_profiling(decode_layer *h, int enable) {
  if (!h) return fail(nullptr, DL_ERR_INVALID_ARG, "handle is NULL");
  HIP_TRY(h, hipSetDevice(h->device));
  if (enable && !h->ev_prof[0][0]) {
    for (int i = 0; i < DECODE_LAYER_N_LAUNCHES; ++i)
      for (int j = 0; j < 2; ++j) HIP_TRY(h, hipEventCreate(&h->ev_prof[i][j]));
  }
  h->profiling = enable != 0;
  h->profiled_step = false;
  return DL_OK;
}

int decode_layer_kernel_times(decode_layer *h, float *ms, int capacity) {
  if (!h || !ms || capacity < 0) return fail(h, DL_ERR_INVALID_ARG, "NULL handle or output");
  if (!h->profiling || !h->profiled_step) return fail(h, DL_ERR_INVALID_ARG, "no profiled step to report");
  HIP_TRY(h, hipSetDevice(h->device));
  int n = capacity < DECODE_LAYER_N_LAUNCHES ? capacity : DECODE_LAYER_N_LAUNCHES;
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.f;
    if (!h->launched[i]) continue;
    HIP_TRY(h, hipEventSynchronize(h->ev_prof[i][1]));
    HIP_TRY(h, hipEventElapsedTime(&ms[i], h->ev_prof[i][0], h->ev_prof[i][1]));
  }
  return n;
}

int decode_layer_destroy(decode_layer *h) {
  if (!h) return DL_OK;
  (void)hipSetDevice(h->device);
  if (h->side) (void)hipStreamSynchronize(h->side);
  for (int i = 0; i < DECODE_LAYER_N_LAUNCHES; ++i)
    for (int j = 0; j < 2; ++j)
      if (h->ev_prof[i][j]) (void)hipEventDestroy(h->ev_prof[i][j]);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->scratch_base) {
    (void)hipDeviceSynchronize();
    (void)hipFree(h->scratch_base);
  }
  delete h;
  return DL_OK;
}

}  // extern "C"
