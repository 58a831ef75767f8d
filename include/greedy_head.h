/*
 * greedy_head.h - C ABI of the greedy decode step on gfx950: the LM head, the argmax over the
 * vocabulary, and the chosen token's embedding written as the next step's input.
 *
 * Source: "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for
 * Apple Silicon", section "How It Works: Prefill and Decode Strategies" (the selected token is
 * written straight into the next step's GPU-resident input slot, with no CPU round trip per
 * token) and section "Frequently Asked Questions" (greedy decoding only). For token t:
 *   logits[t, v] = x[t] . W_head[v]         v < V; W_head [V, H] in the 4-bit group-64 affine
 *                                           format of moe_w4.h (one matrix), each weight
 *                                           s*q + b rounded to bf16, sums in fp32
 *   token[t]     = argmax_v logits[t, v]    (the lowest v among equal maxima)
 *   x_next[t]    = embedding row token[t]   E [V, H] in the same format, each value s*q + b
 *                                           rounded to bf16 (nearest, ties to even)
 * Conventions are those of moe_w4.h (device pointers, caller-owned buffers, enqueue-only,
 * graph-capturable, moe_status_t return codes, nothing allocated).
 */
#ifndef GREEDY_HEAD_H
#define GREEDY_HEAD_H

#include <stddef.h>
#include <stdint.h>

#include "moe_w4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace for V tokens of vocabulary and T tokens (0 if invalid): the fp32 logits [T, V] at
 * offset 0, then per-workgroup partial maxima. 256-byte aligned, no initialisation. */
size_t moe_greedy_workspace_bytes(int32_t V, int32_t T);

/* One greedy step for T tokens (1 <= T <= 16).
 *   head, embed  4-bit weights of V rows of H inputs (q [V, H/8], scale/bias [V, H/64]);
 *                q 16-byte aligned
 *   x            [T, H] bf16, the final normalised hidden state; 16-byte aligned
 *   token        [T] int32 (written)
 *   x_next       [T, H] bf16 (written; may be x: x is read in full before it is written)
 * H one of 512, 1024, 2048, 4096 (T <= 8 at 4096); 1 <= V < 2^31. On return the workspace starts with the fp32
 * logits [T, V]. Deterministic: the argmax does not depend on the order of the partial sums'
 * merge (ties go to the lowest index).
 * Returns MOE_INVALID_ARG / MOE_UNSUPPORTED / MOE_WORKSPACE_TOO_SMALL / MOE_HIP_ERROR, or MOE_OK. */
int moe_greedy_next_input(const moe_w4_t* head, const moe_w4_t* embed, int32_t V, int32_t H,
                          const uint16_t* x, int32_t T, int32_t* token, uint16_t* x_next,
                          void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GREEDY_HEAD_H */
