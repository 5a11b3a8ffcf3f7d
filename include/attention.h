/*
 * GQA attention with per-head sinks on one MI355X (gfx950) - C ABI.
 *
 * "GPT-OSS on day 0", section "Sink attention": each head has a learned sink
 * value that takes part in the softmax next to the scaled scores,
 *     attn = softmax(q . k^T * sm_scale + sink) . V,
 * computed online with the running maximum seeded by the sink; when the keys
 * are split into parts, the sink is counted in the first part only.  Section
 * "GPT-OSS on Hopper": the attention is GQA.  For one query q of head h
 * (key/value head h / (Hq / Hkv)) over its visible keys j:
 *
 *   s_j = sm_scale * q . k_j,   M = max(sink_h, max_j s_j)
 *   out = sum_j exp(s_j - M) v_j / (exp(sink_h - M) + sum_j exp(s_j - M))
 *
 * The sink has no value vector: it only enlarges the denominator.  Prefill
 * is causal (query i sees keys 0..i of its sequence); decode has one query
 * per sequence that sees all kv_len[b] cached keys.  Arithmetic: bf16 inputs,
 * fp32 scores and softmax, probabilities rounded to bf16 for the P.V product,
 * fp32 accumulation, bf16 output.
 *
 * Conventions are those of moe.h: device pointers, caller-owned, 16-byte
 * aligned; work is enqueued on `stream` without host synchronisation;
 * argument errors return a negative moe_status before anything is enqueued;
 * S == 0 or B == 0 is a no-op.  Head dimension D must be 64.
 */
#ifndef SPARSE_MOE_MI355_ATTENTION_H
#define SPARSE_MOE_MI355_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Causal prefill of one sequence of S tokens.
 *   q      bf16 [S, Hq, D]      token major (the QKV projection's layout)
 *   k, v   bf16 [S, Hkv, D]
 *   sinks  fp32 [Hq]
 *   out    bf16 [S, Hq, D]      written
 * Hq / Hkv must be 1, 2, 4 or a multiple of 8 (MOE_ERR_UNSUPPORTED otherwise);
 * Hq not a multiple of Hkv is MOE_ERR_SHAPE. */
moe_status attn_sink_prefill(const void* q, const void* k, const void* v, const float* sinks,
                             void* out, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                             float sm_scale, hipStream_t stream);

/* Bytes of device workspace attn_sink_decode needs (the partial results of
 * the sequence pieces the waves hold: min(1024 + 2 B, B (ceil(Lmax / 256) + 2))
 * * Hq records of 68 floats, then 2 B + 2 int32 of work plan). */
size_t attn_sink_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Lmax);

/* One query per sequence over a KV cache laid out heads major with each
 * head's tokens contiguous (the HND order of "Hosting Qwen on Blackwell",
 * in its opening part on disaggregated prefill).
 *   q        bf16 [B, Hq, D]
 *   k_cache  bf16 [B, Hkv, Lmax, D]
 *   v_cache  bf16 [B, Hkv, Lmax, D]
 *   kv_len   int32 [B]           visible keys per sequence (device; values outside
 *                                [0, Lmax] are clamped; 0 keys give a zero output)
 *   sinks    fp32 [Hq]
 *   out      bf16 [B, Hq, D]     written
 * For each key/value head the keys of all sequences are cut into equal
 * ranges of at least 256 keys, one wave each (one wave per SIMD of the chip
 * in all), so a wave may hold pieces of several sequences; a second kernel
 * merges each sequence's pieces; Hq / Hkv must be at most 16. */
moe_status attn_sink_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* kv_len, const float* sinks, void* out, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, float sm_scale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
