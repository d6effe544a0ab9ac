/*
 * decode_attention.h - C ABI of the decode attention core of the MI355X
 * (gfx950) decode-layer library: one decode step of grouped-query attention
 * over an FP8 KV cache, for 1 to 8 query tokens per request (one verified
 * token plus up to 7 speculative drafts), on one GPU's tensor-parallel shard.
 *
 * The pages run decode with an FP8 KV cache and verify 3 to 7 draft tokens
 * of the DSpark speculative decoder in one step (bigchange.ai "Kimi K3 vLLM
 * GPU inference benchmark", section "Where the time was going").  They give
 * no head count, head size, cache layout or masking rule; this library takes
 * the plainest forms that fit the layer-step it serves (whose out-projection
 * reads 512 attention outputs per TP16 shard, i.e. 4 query heads of 128):
 *
 *   - grouped-query attention: query head h reads KV head h / (Hq / Hkv);
 *   - the cache holds OCP FP8 E4M3 codes (bias 7, no infinities, largest
 *     finite 448) and one fp32 scale per KV head: value = decode(code) * scale;
 *   - a step first writes its T tokens' keys and values to positions
 *     past_len[r] .. past_len[r] + T - 1 of request r's cache, each value
 *     quantised as x / scale in fp32 rounded to the nearest E4M3 value (ties
 *     to the even code, magnitudes beyond 448 clamped to 448, the sign kept);
 *   - query token j of request r then attends to positions 0 .. past_len[r] + j
 *     (causal among the step's tokens, reading them back as FP8):
 *       out = sum_p softmax_p(softmax_scale * q . k_p) * v_p.
 *
 * Conventions as in decode_layer.h: bf16 = IEEE bfloat16 bit patterns; all
 * device pointers 16-byte aligned; functions return DL_OK (0) or a negative
 * DL_ERR_* code (the values of decode_layer.h), with the text available from
 * decode_layer_last_error(NULL) on the calling thread; argument errors are
 * found on the host before any HIP call.
 */
#ifndef DECODE_ATTENTION_H
#define DECODE_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#include "decode_layer.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Shapes, fixed per call site.  Envelope (else DL_ERR_UNSUPPORTED):
 *   head_dim D      : 128
 *   n_kv_heads Hkv  : 1..64, dividing n_q_heads Hq (1..256)
 *   max_tokens T    : 1..8, with (Hq / Hkv) * T <= 32 query rows per KV head
 *   max_requests R  : 1..1024
 *   cache_len C     : 1..(1 << 20) positions per request and KV head
 *   softmax_scale   : finite and > 0
 *   max_splits      : 0 (automatic) or a cap on the workgroups that share one
 *                     request's positions (a caller that shares the GPU with
 *                     other work can keep the launch small); >= 0 */
typedef struct {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t max_tokens;
  int32_t max_requests;
  int32_t cache_len;
  float softmax_scale;
  int32_t max_splits;
} decode_attention_config;

/* One step.  Caller-owned device memory, valid until the enqueued work ends. */
typedef struct {
  int32_t n_requests;        /* R, 0..max_requests (0: no-op) */
  int32_t n_tokens;          /* T, 1..max_tokens, the same for every request */
  int32_t max_past;          /* host bound: past_len[r] <= max_past for every r (sizes the launch);
                                max_past + T <= cache_len */
  const int32_t *past_len;   /* device int32 [R]: positions already cached per request */
  const void *q;             /* bf16 [R][T][Hq][D] */
  const void *k_new;         /* bf16 [R][T][Hkv][D] */
  const void *v_new;         /* bf16 [R][T][Hkv][D] */
  uint8_t *k_cache;          /* E4M3 [max_requests][Hkv][C][D], appended in place */
  uint8_t *v_cache;          /* E4M3 [max_requests][Hkv][C][D], appended in place */
  const float *k_scale;      /* fp32 [Hkv] */
  const float *v_scale;      /* fp32 [Hkv] */
  float *out;                /* fp32 [R][T][Hq][D] */
  void *workspace;           /* decode_attention_workspace_bytes(cfg) bytes, 256-byte aligned, zeroed
                                once before first use (the kernels leave it as they found it) */
  void *out_bf16;            /* optional (NULL: not written): bf16 [R][T][Hq][D], each element out
                                rounded to nearest even - laid out as the decode layer step's attn
                                input [R*T][Hq*D] (token r*T + j), so a step can take it as is */
} decode_attention_io;

/* Bytes of workspace a call site with this configuration needs (0 if invalid).
 * It holds the partial results of the workgroups that share one request's
 * positions (at most min(64, ceil(C / 256)) per request and KV head) and one
 * arrival counter per request and KV head.  Host-only. */
DL_API size_t decode_attention_workspace_bytes(const decode_attention_config *cfg);

/* Host-only validation of a configuration and of one step's arguments. */
DL_API int decode_attention_check(const decode_attention_config *cfg, const decode_attention_io *io);

/* Enqueue one attention step on `hip_stream` (one kernel: workgroups take
 * consecutive tiles of 256 positions of one request and KV head, quantise and
 * write the step's own positions where they fall, and the last workgroup of a
 * request and KV head to finish combines their partial results) and return
 * without synchronising.  No allocation, no host copy, no memset; capturable in a HIP
 * graph.  A device-side past_len[r] above max_past, or with
 * past_len[r] + T > cache_len, makes request r's outputs NaN and writes none
 * of its cache positions.  Steps that share a workspace must not overlap. */
DL_API int decode_attention_step(const decode_attention_config *cfg, const decode_attention_io *io,
                                 void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTENTION_H */
