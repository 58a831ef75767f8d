/*
 * attn_gqa.h - C ABI of grouped-query decode attention over a block-paged KV cache (gfx950).
 *
 * Source (cited by page title and section): "Perplexity's Lily: A Breakthrough Local Inference
 * Engine Tailored Exclusively for Apple Silicon", section "The Model: Qwen3.6-35B-A3B in Focus"
 * (ten full-attention layers with grouped-query attention, 16 query heads and two KV heads,
 * attending over a growing key-value cache) and section "How It Works: Prefill and Decode
 * Strategies" (coalesced reads of the key and value cache, GQA packing, a fixed-block cache
 * layout for long contexts; decode is bandwidth-bound).
 *
 * One decode step for B sequences: for query head h of sequence b, with g = h / (Hq / Hkv),
 *   out[b,h] = sum_j softmax_j(scale * q[b,h] . K_b,g[j]) V_b,g[j]      over j < seq_lens[b]
 * Token j of sequence b is row j % BS of physical block block_table[b, j / BS] of the cache.
 * q, K and V are bf16; scores, softmax and sums are fp32; out is fp32.
 *
 * Conventions are those of moe_w4.h (device pointers, caller-owned buffers, enqueue-only,
 * graph-capturable, moe_status_t return codes, nothing allocated).
 */
#ifndef ATTN_GQA_H
#define ATTN_GQA_H

#include <stddef.h>
#include <stdint.h>

#include "moe_w4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Supported: head_dim 64, 128 or 256; num_q_heads a multiple of num_kv_heads with at most 8
 * query heads per KV head; block_size 16, 32, 64, 128 or 256 tokens. Else MOE_UNSUPPORTED. */
typedef struct {
  int32_t num_q_heads;   /* Hq  */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* D   */
  int32_t block_size;    /* BS: tokens per cache block */
  float scale;           /* score scale, usually 1/sqrt(D) */
} attn_gqa_desc_t;

enum {
  /* one query head per workgroup instead of a KV head's whole group: every query head reads
   * the K and V rows again (the layout without GQA packing, kept to measure what packing buys) */
  ATTN_FLAG_UNPACKED = 1
};

/* Workspace for a call with these sizes (0 if the arguments are invalid): the per-span
 * partial results of the split over the context. 256-byte aligned, no initialisation. */
size_t attn_gqa_decode_workspace_bytes(const attn_gqa_desc_t* desc, int32_t batch,
                                       int32_t max_seq_len);

/* One decode step.
 *   q           [B, Hq, D] bf16 (the new token's queries)
 *   k_cache,
 *   v_cache     [num_blocks, Hkv, BS, D] bf16 (rows of D contiguous values)
 *   block_table [B, max_blocks_per_seq] int32 physical block ids
 *   seq_lens    [B] int32 on the device, each in [0, max_seq_len]; a sequence of length 0
 *               gets a zero output
 *   out         [B, Hq, D] fp32
 * max_seq_len <= max_blocks_per_seq * BS bounds the grid (the lengths stay on the device).
 * Device-side guards: lengths are clamped to max_seq_len and block ids to [0, num_blocks), so
 * that no access leaves the buffers (a wrong id gives a wrong result, not a fault).
 * flags: ATTN_FLAG_*. workspace: attn_gqa_decode_workspace_bytes(desc, B, max_seq_len).
 * Deterministic: the context is split into spans of whole chunks (sized from B, the heads and
 * max_seq_len only) whose partial results are merged in a fixed order. */
int attn_gqa_decode(const attn_gqa_desc_t* desc, const uint16_t* q, const uint16_t* k_cache,
                    const uint16_t* v_cache, int32_t num_blocks, const int32_t* block_table,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                    int32_t max_seq_len, float* out, int32_t flags, void* workspace,
                    size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GQA_H */
