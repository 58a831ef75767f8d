/*
 * delta_rule.h - C ABI of the gated delta-rule recurrence (the model's linear-attention layers)
 * on gfx950.
 *
 * Source: "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for
 * Apple Silicon", section "The Model: Qwen3.6-35B-A3B in Focus" (thirty Gated DeltaNet layers
 * whose recurrence keeps a fixed-size state). The pages do not print the recurrence; it is the
 * gated delta rule of Yang, Kautz and Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with
 * Delta Rule" (ICLR 2025), with L2-normalised queries and keys. For value head j (query/key
 * head i = j / (Hv / Hk)) of sequence b and token t, with the state S a [Dv, Dk] matrix:
 *   kh = k / sqrt(|k|^2 + eps),  qh = scale * q / sqrt(|q|^2 + eps),  alpha = exp(g)
 *   S_t = alpha S_{t-1} (I - beta kh kh^T) + beta v kh^T,    o_t = S_t qh
 * computed as u = S_{t-1} kh, S_t = alpha S_{t-1} + beta (v - alpha u) kh^T,
 * o_t = alpha S_{t-1} qh + beta (v - alpha u) (kh . qh): the same quantities, in fp32.
 *
 * Conventions are those of moe_w4.h (device pointers, caller-owned buffers, enqueue-only,
 * graph-capturable, moe_status_t return codes, nothing allocated, no workspace).
 */
#ifndef DELTA_RULE_H
#define DELTA_RULE_H

#include <stddef.h>
#include <stdint.h>

#include "moe_w4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Supported: dk 64, 128 or 256; dv a multiple of 16; num_v_heads a multiple of num_k_heads.
 * Else MOE_UNSUPPORTED. */
typedef struct {
  int32_t num_k_heads;  /* Hk: query/key heads */
  int32_t num_v_heads;  /* Hv: value heads (state heads) */
  int32_t dk;           /* key size (state columns) */
  int32_t dv;           /* value size (state rows) */
  float scale;          /* query scale, usually 1/sqrt(dk) */
  float eps;            /* added to |q|^2 and |k|^2 before the square root */
} delta_rule_desc_t;

/* T tokens of B sequences, token after token (T = 1: one decode step).
 *   q, k      [B, T, Hk, dk] bf16;  v [B, T, Hv, dv] bf16
 *   g, beta   [B, T, Hv] fp32 (log of the decay alpha, and the write strength)
 *   state_in  [B, Hv, dv, dk] fp32, or NULL for a zero initial state
 *   state_out [B, Hv, dv, dk] fp32: the state after the last token (may equal state_in)
 *   o         [B, T, Hv, dv] fp32
 * Each state row is read once and written once; rows are independent given the token's
 * normalised key and query, so the work splits over rows with no synchronisation. */
int delta_rule_forward(const delta_rule_desc_t* desc, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const float* g, const float* beta,
                       const float* state_in, float* state_out, float* o, int32_t batch,
                       int32_t T, void* stream);

/* The same computation as delta_rule_forward (the same outputs up to fp32 rounding), over chunks
 * of 32 tokens: the chunkwise form of the gated delta rule (Yang, Kautz and Hatamizadeh,
 * section 3), in which each chunk's (I + M)^-1 and output-mixing matrix are formed for all
 * chunks at once and the state advances one chunk per step. For long T (prefill).
 *   workspace  device buffer of at least delta_rule_chunked_workspace_bytes(desc, batch, T)
 *              bytes, 16-byte aligned; its contents on entry do not matter and are overwritten
 *              (per (sequence, value head, chunk): the chunk's corrected keys and queries,
 *              its value terms, its normalised keys and its decays; 4 * (96 dk + 64 dv + 64)
 *              bytes per record). Calls that share a workspace must not overlap.
 * Returns MOE_WORKSPACE_TOO_SMALL when ws_bytes is below the size needed, else as
 * delta_rule_forward. */
size_t delta_rule_chunked_workspace_bytes(const delta_rule_desc_t* desc, int32_t batch, int32_t T);
int delta_rule_forward_chunked(const delta_rule_desc_t* desc, const uint16_t* q,
                               const uint16_t* k, const uint16_t* v, const float* g,
                               const float* beta, const float* state_in, float* state_out,
                               float* o, int32_t batch, int32_t T, void* workspace,
                               size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DELTA_RULE_H */
