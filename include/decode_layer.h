/*
 * decode_layer.h - C ABI of an MI355X (gfx950) library that runs one decode
 * step of a mixture-of-experts transformer layer, for 1..64 tokens, on one
 * GPU's tensor-parallel shard.
 *
 * The step is the one the vLLM "latency_specialized" decode backend for
 * Kimi K3 specialises (bigchange.ai "Kimi K3 vLLM GPU inference benchmark",
 * section "Where the time was going"; wireai.ir "vLLM's speed jump on NVIDIA
 * Blackwell servers; record 842 tokens/s for Kimi K3", section "Four key
 * changes behind the jump"):
 *   1. attention input projection          qkv = x Wqkv^T
 *   2. attention output projection, fused with the residual add and RMSNorm
 *                                          r1 = r + attn Wo^T
 *                                          h  = g * r1 / sqrt(mean(r1^2) + eps)
 *   3. router scores and top-k selection   l = h Wr^T, s = sigmoid(l),
 *                                          idx = top-k of s, w = s_idx / sum s_idx
 *   4. routed SwiGLU experts and the always-on shared expert
 *        y[t] = FFN_shared(h[t]) + sum_j w[t,j] FFN_{idx[t,j]}(h[t]),
 *        FFN(v) = W2 (silu(W1 v) * (W3 v)).
 * On one shard the cross-GPU reductions that the pages fuse into the
 * out-projection and the MoE tail are the identity: the residual adds this
 * shard's projection, and y is returned as this shard's partial sum (it is
 * NOT added to the residual).
 *
 * Conventions for every entry point:
 *   - Matrices are row-major [out][in]: row j holds the weights of output j,
 *     and the input dimension is contiguous.
 *   - bf16 means IEEE bfloat16 bit patterns (uint16 storage).
 *   - All device pointers must be 16-byte aligned.
 *   - No exception crosses the ABI.  Functions return DL_OK (0) or a negative
 *     DL_ERR_* code; decode_layer_last_error() then describes the failure.
 *   - Argument and configuration errors are detected on the host before any
 *     HIP call is made.  Configurations outside the supported envelope return
 *     DL_ERR_UNSUPPORTED, so a caller can fall back to a generic path (the
 *     pages' backend is opt-in and falls back for unsupported steps:
 *     bigchange.ai, opening section; wireai.ir, "Conditions and limits for
 *     production deployment").
 */
#ifndef DECODE_LAYER_H
#define DECODE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the C ABI (the library is built with hidden visibility). */
#define DL_API __attribute__((visibility("default")))

enum {
  DL_OK = 0,
  DL_ERR_INVALID_ARG = -1, /* NULL or misaligned pointer, negative size        */
  DL_ERR_UNSUPPORTED = -2, /* shape or option outside the supported envelope   */
  DL_ERR_HIP = -3,         /* a HIP runtime call failed (no device, launch ...) */
  DL_ERR_OOM = -4          /* device allocation of the handle's scratch failed  */
};

/* Shapes and options, fixed when the handle is created.
 * Supported envelope (anything else -> DL_ERR_UNSUPPORTED):
 *   hidden H      : 8..16384, multiple of 8
 *   qkv_out Dq    : 1..65536
 *   attn_dim Do   : 8..16384, multiple of 8
 *   n_experts E   : 1..1024
 *   top_k k       : 1..min(E, 64) (each pick of a token is one lane of a
 *                   wave-wide top-k)
 *   expert_ffn F  : 32, 64, 128 or 256
 *   shared_ffn Fs : 0 (no shared expert) or 32, 64, 128 or 256
 *     (F is narrower than a generic MoE layer would need: the kernels map an
 *     expert's ffn row onto F/8 lanes of 16-byte loads, specialised for these
 *     four widths; the shapes this library is measured on use F = 128 or 256.
 *     Other values return DL_ERR_UNSUPPORTED, the pages' fallback case.)
 *   max_batch     : 1..64
 *   rms_eps       : > 0 and finite
 *   score_fn      : 0 = sigmoid (the only value supported)
 *   renormalize   : 1 = top-k weights divided by their sum (the only value supported)
 *   path          : DL_PATH_AUTO, DL_PATH_MULTI, DL_PATH_SINGLE or DL_PATH_BATCHED (below)
 *
 * Execution paths.  The pages' backend is shape-aware: small-batch kernels at
 * one or two tokens, split-K kernels beyond (wireai.ir "vLLM's speed jump on
 * NVIDIA Blackwell servers; record 842 tokens/s for Kimi K3", section "Four
 * key changes behind the jump", bullet 1).  This library has three:
 *   DL_PATH_SINGLE  the whole step in ONE launch: one workgroup per CU, all
 *                   resident, phases handing data to each other through
 *                   device memory (the shared expert's and the router's
 *                   weights stream while the norm is being exchanged, and
 *                   the attention input projection is computed while the
 *                   router logits are exchanged).
 *                   Available on devices with at most 256 CUs when
 *                   hidden <= 8192 and <= 32 * CUs, n_experts <= 512 and
 *                   <= 2 * CUs, qkv_out <= 8 * CUs, and shared_ffn == 0 or
 *                   == expert_ffn; for batches up to
 *                   decode_layer_single_max_batch(), which is at most 8 and
 *                   also bounded by B*k <= 64, B*E <= 8192, B*k*F <= 8192 and
 *                   B*Fs <= 4096.
 *   DL_PATH_BATCHED five launches on the caller's stream (projections,
 *                   router dot products, top-k + permutation, gate/up,
 *                   down + combine) that run every contraction whose
 *                   weights 16 or more tokens share on the matrix cores
 *                   (fp32 activations as bf16 hi + lo pairs) and the rest
 *                   as VALU GEMVs.  Available when hidden % 512 == 0 and
 *                   attn_dim % 128 == 0; any batch up to max_batch.
 *   DL_PATH_MULTI   five launches of VALU GEMVs (input/out-projection,
 *                   router + top-k + permutation, routed gate/up, down +
 *                   combine) with the shared expert's gate/up on the
 *                   handle's second stream.  Any configuration and batch
 *                   in the envelope.
 *   DL_PATH_AUTO    SINGLE when the step's batch allows it, else BATCHED
 *                   when available, else MULTI.
 * Forcing DL_PATH_SINGLE makes a step with a larger batch fail with
 * DL_ERR_UNSUPPORTED; forcing DL_PATH_BATCHED (or SINGLE) on a configuration
 * the path cannot run makes decode_layer_init fail with DL_ERR_UNSUPPORTED.
 */
enum { DL_PATH_AUTO = 0, DL_PATH_MULTI = 1, DL_PATH_SINGLE = 2, DL_PATH_BATCHED = 3 };
typedef struct {
  int32_t hidden;
  int32_t qkv_out;
  int32_t attn_dim;
  int32_t n_experts;
  int32_t top_k;
  int32_t expert_ffn;
  int32_t shared_ffn;
  int32_t max_batch;
  float rms_eps;
  int32_t score_fn;
  int32_t renormalize;
  int32_t path;
} decode_layer_config;

/* Weights of one layer shard: device pointers owned by the caller.  They
 * must stay allocated and unchanged while the handle is in use; the library
 * never writes them and keeps no copy. */
typedef struct {
  const void *w_qkv;     /* bf16 [Dq][H]                    */
  const void *w_o;       /* bf16 [H][Do]                    */
  const void *norm_gain; /* bf16 [H]                        */
  const float *w_router; /* fp32 [E][H]                     */
  const void *w1;        /* bf16 [E][F][H]  expert gate      */
  const void *w3;        /* bf16 [E][F][H]  expert up        */
  const void *w2;        /* bf16 [E][H][F]  expert down      */
  const void *s1;        /* bf16 [Fs][H]    shared gate (NULL iff Fs == 0) */
  const void *s3;        /* bf16 [Fs][H]    shared up        */
  const void *s2;        /* bf16 [H][Fs]    shared down      */
} decode_layer_weights;

/* Per-step tensors: device pointers owned by the caller, valid until the
 * work enqueued by decode_layer_step has completed on its stream. */
typedef struct {
  int32_t batch;          /* B tokens, 0..max_batch; 0 is a no-op          */
  const void *x;          /* bf16 [B][H]  attention input                   */
  const void *attn;       /* bf16 [B][Do] attention-core output             */
  const float *resid_in;  /* fp32 [B][H]  residual stream                   */
  float *qkv;             /* out fp32 [B][Dq]                               */
  float *resid_out;       /* out fp32 [B][H]  r + attn Wo^T; may equal resid_in */
  float *router_logits;   /* out fp32 [B][E]; may be NULL                   */
  int32_t *topk_idx;      /* out int32 [B][k], descending score, ties to the lower id */
  float *topk_w;          /* out fp32 [B][k], sums to 1 per token          */
  float *moe_out;         /* out fp32 [B][H]  shard-partial MoE output y    */
  float *h_out;           /* out fp32 [B][H]  normalised hidden h; may be NULL */
} decode_layer_io;

typedef struct decode_layer decode_layer; /* opaque handle */

/* Validate `cfg` and `w`, then create a handle on HIP device `device`:
 * allocates the handle's device scratch (decode_layer_scratch_bytes: under
 * 1 MB at batch 1 on the single-launch path, tens of MB when the batched path
 * can run at 64 tokens), a second HIP stream for the shared expert and the
 * events that fork and join it.  No kernel runs.  The weights stay the
 * caller's: the library reads them in place and never changes them (the
 * pages' backend leaves weights, scheduling, sampling and the KV cache as
 * they are: bigchange.ai "Kimi K3 vLLM GPU inference benchmark", opening
 * section; wireai.ir "vLLM's speed jump on NVIDIA Blackwell servers; record
 * 842 tokens/s for Kimi K3", "Conditions and limits for production
 * deployment").
 * On success *out receives the handle; on failure *out is set to NULL.
 * Errors: DL_ERR_INVALID_ARG (NULL pointers, misaligned weights),
 * DL_ERR_UNSUPPORTED (shape outside the envelope, or a forced path that
 * cannot run it), DL_ERR_HIP (no such device), DL_ERR_OOM. */
DL_API int decode_layer_init(const decode_layer_config *cfg, const decode_layer_weights *w,
                             int device, decode_layer **out);

/* Enqueue one layer-step - the attention input projection, the out-projection
 * fused with the residual add and RMSNorm, the router with top-k, and the
 * shared and routed SwiGLU experts (wireai.ir "vLLM's speed jump on NVIDIA
 * Blackwell servers; record 842 tokens/s for Kimi K3", "Four key changes
 * behind the jump", bullets 1-3; bigchange.ai "Kimi K3 vLLM GPU inference
 * benchmark", "Where the time was going") - on `hip_stream` (a hipStream_t;
 * NULL = the null stream) and return without synchronising.  Device work: on
 * the single-launch path one persistent kernel on `hip_stream`; on the
 * batched path five kernel launches on `hip_stream`; on the multi-launch path
 * up to five kernel launches, four on `hip_stream` and one (the shared
 * expert's gate/up projection) on the handle's second stream, which is forked
 * from and joined back into `hip_stream` with events.  Either can be captured
 * in a HIP graph.  No allocation, no host copy, no memset.
 * The single-launch kernel is correct only when all of its workgroups (one
 * per CU) are resident at once: it needs every CU of the device.  Work on
 * other streams that finishes on its own (ordinary kernels, copies) only
 * delays it.  Two single-launch steps in flight at once on one device (two
 * handles stepped on different streams, or a graph replayed on two streams)
 * can each hold part of the device while waiting for the rest: their
 * hand-off waits then expire (about a second each).  A caller that steps
 * handles concurrently must create them with DL_PATH_BATCHED or
 * DL_PATH_MULTI, whose kernels need no co-residency.
 * When a hand-off wait expires, the step still runs to completion, every
 * output it computes from a value it did not receive is written as NaN (a
 * topk_idx entry as -1), and decode_layer_status() reports bit 0; qkv and
 * resid_out depend on no hand-off and stay exact.
 * `io` is validated on the host first (DL_ERR_INVALID_ARG /
 * DL_ERR_UNSUPPORTED, nothing enqueued).  A failed launch returns DL_ERR_HIP;
 * faults inside kernels surface at the caller's next synchronisation.
 * One step per handle may be in flight at a time (the scratch is per
 * handle). */
DL_API int decode_layer_step(decode_layer *h, const decode_layer_io *io, void *hip_stream);

/* Largest batch the single-launch path accepts with this handle (0 if none). */
DL_API int decode_layer_single_max_batch(const decode_layer *h);

/* Device-side status of the handle, read synchronously (synchronise the
 * step's stream first).  Bit 0 (value 1): a single-launch hand-off wait
 * expired in some step since the last clear (that step's affected outputs
 * are NaN, see decode_layer_step).  The single-launch step counter is 32-bit
 * and wraps: the step that uses its last value clears every hand-off slot,
 * so the handle works indefinitely.  `clear` != 0 resets the word afterwards.
 * Returns DL_OK or DL_ERR_HIP / DL_ERR_INVALID_ARG. */
DL_API int decode_layer_status(decode_layer *h, uint32_t *status, int clear);

/* Wait for the handle's streams, free its scratch, stream and events (the
 * resources decode_layer_init took; the caller's weights are untouched).
 * NULL is a no-op.  Always returns DL_OK. */
DL_API int decode_layer_destroy(decode_layer *h);

/* Host-only check of a configuration (the validation decode_layer_init does
 * before touching the GPU).  Returns DL_OK, DL_ERR_INVALID_ARG or DL_ERR_UNSUPPORTED. */
DL_API int decode_layer_check_config(const decode_layer_config *cfg);

/* Host-only check of one step's arguments against a configuration (the
 * validation decode_layer_step does before enqueuing anything). */
DL_API int decode_layer_check_io(const decode_layer_config *cfg, const decode_layer_io *io);

/* Text of the last error on `h`, or of the calling thread's last error when
 * `h` is NULL (e.g. a failed decode_layer_init): the reason a caller falls
 * back to another backend for an unsupported step (wireai.ir "vLLM's speed
 * jump on NVIDIA Blackwell servers; record 842 tokens/s for Kimi K3",
 * "Conditions and limits for production deployment").  Never NULL; the
 * string is owned by the library and valid until the next call on the same
 * handle or thread. */
DL_API const char *decode_layer_last_error(const decode_layer *h);

/* Test support.  decode_layer_set_spin_limit sets the number of polling
 * rounds after which a single-launch hand-off wait gives up (default 2^20,
 * about a second); 0 makes every wait give up at its first unsatisfied poll,
 * so the failure behaviour of decode_layer_step can be exercised while every
 * kernel still finishes normally.  decode_layer_set_step_counter
 * synchronises the device and sets the handle's single-launch step counter
 * (the tag of the last step; the next step uses last_tag + 1, skipping 0),
 * e.g. to run the counter's wrap.  Both return DL_OK or DL_ERR_INVALID_ARG /
 * DL_ERR_HIP. */
DL_API int decode_layer_set_spin_limit(decode_layer *h, int rounds);
DL_API int decode_layer_set_step_counter(decode_layer *h, uint32_t last_tag);

/* Measurement support, not needed for normal use.  While profiling is
 * enabled on a handle, every decode_layer_step also records a HIP event pair
 * around each of its kernel launches, on the stream that launch uses.
 * decode_layer_kernel_times() waits for the last step's events and writes
 * the launches' durations in milliseconds, in the fixed order
 *   0 out-projection + input projection, 1 shared expert gate/up,
 *   2 router + top-k + permute, 3 routed expert gate/up, 4 expert down + combine,
 *   5 single-launch step,
 *   6 batched projections, 7 batched router, 8 batched top-k + permute,
 *   9 batched gate/up, 10 batched down + combine
 * (0 for a launch the last step did not make).  It returns the number of
 * entries written (<= capacity) or a negative DL_ERR_* code (DL_ERR_INVALID_ARG
 * if profiling is off or no step ran since it was enabled).  Enabling creates
 * the events (DL_ERR_HIP on failure); do not enable it while capturing a graph. */
#define DECODE_LAYER_N_LAUNCHES 11
DL_API int decode_layer_set_profiling(decode_layer *h, int enable);
DL_API int decode_layer_kernel_times(decode_layer *h, float *ms, int capacity);

/* Cross-layer weight prefetch.  In a decode step the layers of the model run
 * one after another; while one layer's single-launch step waits for its
 * router logits (a hand-off that leaves HBM mostly idle), the weights of the
 * next layer are already known.  After this call every single-launch step of
 * `h` also reads, once per 64-byte sector, the dense weights that the
 * workgroups of `next` read first in their own step (out-projection, router
 * and shared-expert rows, attention input projection, shared down-projection
 * rows), so that `next` finds them in this device's caches (the XCD's L2 and
 * the memory-side Infinity Cache).  The results are unchanged; only where
 * the next layer's reads are served from changes.  This is the single-GPU
 * form of the pages' weight prefetch during communication (wireai.ir "vLLM's
 * speed jump on NVIDIA Blackwell servers; record 842 tokens/s for Kimi K3",
 * "Four key changes behind the jump", bullet 4).  `next` must have the same
 * configuration and device (DL_ERR_INVALID_ARG otherwise) and must stay alive
 * while `h` steps; NULL turns the prefetch off.  Host-only. */
DL_API int decode_layer_set_prefetch(decode_layer *h, const decode_layer *next);

/* Phase trace of the single-launch kernel, for measurement.  With a non-NULL
 * device buffer of decode_layer_grid(h) * decode_layer_trace_points() uint64
 * values (caller-owned, 16-byte aligned), every later single-launch step has
 * thread 0 of each workgroup w write the device wall clock (100 MHz) into
 * buffer[w * points + p] at these points: 0 start, 1 out-projection done and
 * norm partials published, 2 every norm partial polled, 4 norm known,
 * 5 logits (and shared-expert activations) published, 7 all logits read,
 * 14 top-k start, 15 top-k selection done, 13 top-k done (batches above one
 * token), 12 expert lists built (wave 0), 8 lists visible to the workgroup,
 * 9 routed SwiGLU activations published, 10 activations read, 11 y written,
 * 3 end; others unused.
 * NULL turns it off.  Returns DL_OK or DL_ERR_INVALID_ARG. */
DL_API int decode_layer_set_trace(decode_layer *h, void *device_buffer);
DL_API int decode_layer_trace_points(void);
/* Workgroups of the single-launch kernel (the device's CU count; 0 if the path is unavailable). */
DL_API int decode_layer_grid(const decode_layer *h);

/* Bytes of device scratch a handle with this configuration allocates on a
 * device with `n_cu` compute units (0 if the configuration is invalid).  The
 * single-launch path's hand-off arrays grow with n_cu; n_cu = 0 gives the size
 * without them.  The batched path's arrays are included when a step of this
 * configuration can take that path.  Host-only. */
DL_API size_t decode_layer_scratch_bytes(const decode_layer_config *cfg, int n_cu);

/* ---- one step with no handle and no allocation ----------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * decode_layer_step_noalloc validates `cfg`, `w` and `io` exactly as
 * decode_layer_init and decode_layer_step do, then enqueues the same kernels
 * as decode_layer_step would on a handle made from `cfg` and `w`, on the
 * current HIP device (`hip_stream` must belong to it).  Instead of a handle's
 * scratch it uses a static device area of decode_layer_noalloc_max_scratch()
 * bytes (32 MiB), which every device the library runs on holds until the
 * process ends; a configuration whose scratch (decode_layer_scratch_bytes)
 * exceeds it returns DL_ERR_UNSUPPORTED with nothing enqueued (a smaller
 * max_batch or DL_PATH_MULTI needs less; the batched path at 64 tokens needs
 * more).  It calls no hipMalloc, hipFree or other allocating routine; the
 * multi-launch path runs its shared-expert projection on `hip_stream` itself
 * (there is no second stream).  The first call on a device looks up the
 * area's address and, unless the stream is being captured, clears its
 * hand-off state with a small kernel on `hip_stream`.
 * Every call on a device shares that device's area, which keeps the last
 * call's contents: calls whose work overlaps on one device (different
 * streams, threads or graphs in flight together) race and give undefined
 * results; calls ordered on one stream, or synchronised, are safe with any
 * mix of configurations.  Wait expiries are not reported through a status
 * word here; they show as NaN outputs (decode_layer_step).  Errors go to the
 * calling thread's decode_layer_last_error(NULL). */
DL_API int decode_layer_step_noalloc(const decode_layer_config *cfg, const decode_layer_weights *w,
                                     const decode_layer_io *io, void *hip_stream);
DL_API size_t decode_layer_noalloc_max_scratch(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_LAYER_H */
