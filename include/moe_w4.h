/*
 * moe_w4.h - C ABI of the MI355X (gfx950) MoE-layer library: router, permutation,
 * 4-bit group-64 grouped GEMM, combine, and the whole layer.
 *
 * Sources (cited by page title and section):
 *   [P1] "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for
 *        Apple Silicon", sections "The Model: Qwen3.6-35B-A3B in Focus" (a router scores 256
 *        experts and picks 8, one shared expert sees every token; groupwise affine 4-bit
 *        weights with a scale and a bias per 64 weights; weights rebuilt tile by tile into
 *        bf16 for the tensor operations, fp32 accumulation) and "How It Works: Prefill and
 *        Decode Strategies" (4-bit reconstruction inside the grouped GEMM; histogram, prefix
 *        scan, scatter and block maps kept on the GPU with no CPU synchronisation; decode is
 *        bandwidth-bound).
 *   [P3] "Perplexity Open Sources Apple Chip Inference Engine Lily": the paragraph on the
 *        target weights (MLX affine 4-bit, group size 64; the loader verifies the exact
 *        quantisation layout and rejects other formats).
 *
 * The layer (fp32 output y for tokens x):
 *   y[t] = sum_{e in topk(t)} p[t,e] * Wd_e(silu(Wg_e x[t]) * (Wu_e x[t]))
 *        + sigmoid(wg . x[t]) * Wd_s(silu(Wg_s x[t]) * (Wu_s x[t]))
 * with p = softmax over the selected router logits, ties in the top-k going to the lower
 * expert index, and every W = scale * q + bias dequantised per group of 64 inputs. The
 * inputs of the two tensor operations of an expert are bf16 with fp32 accumulation
 * [P1 "The Model ..."]: the dequantised weights and the SwiGLU output. Each expert's output
 * stays fp32, and the weighted combine (a scalar-weighted sum) is computed in fp32.
 *
 * Conventions for every entry point:
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Tensor pointers are DEVICE pointers, row-major, 16-byte aligned, owned by the caller;
 *     the library keeps no pointer after a call returns and allocates no device memory.
 *     Scratch memory comes from a caller workspace sized by moe_workspace_bytes() and
 *     256-byte aligned; its contents need no initialisation and are not kept between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls validate
 *     their arguments on the host, then only enqueue work: no host synchronisation, no
 *     device-to-host copy, so the sequence can be captured into a HIP graph. Results are
 *     valid once the stream reaches that point.
 *   - Every call returns a moe_status_t; nothing is thrown and nothing aborts. On a non-OK
 *     return nothing was enqueued (except MOE_HIP_ERROR, which reports a failed launch).
 *   - T = 0 returns MOE_OK and enqueues nothing.
 *   - Calls are thread-safe provided concurrent calls use distinct workspaces and outputs.
 */
#ifndef MOE_W4_H
#define MOE_W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_INVALID_ARG = 1,          /* null/misaligned pointer, negative size, bad enum      */
  MOE_UNSUPPORTED = 2,          /* a layout the library does not implement (see below)   */
  MOE_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below what the call needs                    */
  MOE_HIP_ERROR = 4             /* a HIP launch failed                                   */
} moe_status_t;

/* One packed 4-bit projection family [P1 "The Model ..."], [P3 target weights]:
 *   q     [n_mat, N, Kin/8] uint32: element 8i+j of a row at bits [4j, 4j+4) of word i
 *   scale [n_mat, N, Kin/64] bf16, bias [n_mat, N, Kin/64] bf16
 *   weight(m, n, k) = scale[m, n, k/64] * q(m, n, k) + bias[m, n, k/64]
 * N is the output dimension and Kin the input dimension (rows are input-contiguous).
 * Each weight is formed as one fp32 fused multiply-add of scale, q and bias and rounded to
 * bf16; this holds for every finite scale of magnitude below 2^104 (larger scales are outside
 * what the kernels compute exactly). */
typedef struct {
  const uint32_t* q;
  const uint16_t* scale;
  const uint16_t* bias;
} moe_w4_t;

/* Layer descriptor. Read during a call, never retained.
 * Supported: bits == 4, group_size == 64, renormalize == 1, hidden and ffn multiples of 64,
 * shared_ffn 0 (no shared expert) or a multiple of 64, 1 <= top_k <= min(num_experts, 32),
 * num_experts <= 1024. Anything else returns MOE_UNSUPPORTED ([P3]: other layouts are
 * rejected). */
typedef struct {
  int32_t hidden;        /* H  */
  int32_t num_experts;   /* E  */
  int32_t top_k;         /* K  */
  int32_t ffn;           /* F  (routed expert intermediate size) */
  int32_t shared_ffn;    /* Fs (shared expert intermediate size, 0 = none) */
  int32_t bits;          /* must be 4  */
  int32_t group_size;    /* must be 64 */
  int32_t renormalize;   /* must be 1: top-k weights renormalised to sum to 1 */
  const float* router_w;      /* [E, H] fp32 */
  const float* router_bias;   /* [E] fp32, added to the logits before selection; or NULL */
  moe_w4_t gate, up;          /* n_mat = E, N = F, Kin = H */
  moe_w4_t down;              /* n_mat = E, N = H, Kin = F */
  moe_w4_t sh_gate, sh_up;    /* n_mat = 1, N = Fs, Kin = H (ignored when Fs == 0) */
  moe_w4_t sh_down;           /* n_mat = 1, N = H, Kin = Fs */
  const float* shared_gate_w; /* [H] fp32: the shared expert's scale is sigmoid(wg . x) */
} moe_layer_desc_t;

/* Routing plan: device arrays written by moe_permute(), read by the grouped GEMM.
 *   counts       [E]            tokens routed to each expert
 *   offsets      [E+1]          exclusive prefix sum of counts (offsets[E] = T*K)
 *   sorted_slots [T*K]          slot ids s = t*K + k grouped by expert, ascending inside a group
 *   slot_pos     [T*K]          inverse of sorted_slots: the grouped row of slot s
 *   blocks       [max_blocks*4] block map, one int32x4 {expert, m0, m_len, row0} per tile of
 *                               at most MOE_BLOCK_M rows: rows m0..m0+m_len-1 of `expert`,
 *                               which are rows row0.. of the grouped activations. Routed
 *                               experts come first in expert order; the shared expert (id E)
 *                               follows with its T rows (row0 = T*K + m0).
 *   num_blocks   [1]            number of valid entries in blocks
 * max_blocks = moe_plan_max_blocks(desc, T). */
typedef struct {
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slots;
  int32_t* slot_pos;
  int32_t* blocks;
  int32_t* num_blocks;
} moe_plan_t;

#define MOE_BLOCK_M 256

/* moe_grouped_gemm_w4 `which` */
enum {
  MOE_GEMM_GATE_UP = 0,             /* out = A [T*K*F + T*Fs] bf16: silu(G)*U per grouped row */
  MOE_GEMM_DOWN = 1,                /* out = Y [(T*K + T), H] fp32, unweighted, grouped rows  */
  MOE_GEMM_DOWN_COMBINE = 2,        /* out = y [T, H] fp32, the combined layer output         */
  MOE_GEMM_DOWN_COMBINE_ATOMIC = 3  /* as 2, combined with fp32 atomics (order not fixed)     */
};

/* moe_layer_forward flags. By default the prefill path (T > 16 or MOE_FLAG_FORCE_PREFILL)
 * stores the fp32 expert outputs Y [T*K + T, H] in the workspace and then combines them in a
 * fixed order (rank order, then the shared term): bit-reproducible. MOE_FLAG_ATOMIC_COMBINE
 * fuses the combine into the down GEMM's epilogue with fp32 atomics instead: no Y array (a
 * smaller workspace), but the summation order, hence the last bits of out, may vary between
 * runs, and on gfx950 the atomics cost more time than the Y round trip they save. The decode
 * path (T <= 16) is deterministic under every flag. */
enum {
  MOE_FLAG_ATOMIC_COMBINE = 1,  /* prefill: fuse the combine into the down GEMM with atomics */
  MOE_FLAG_FORCE_PREFILL = 2    /* use the MFMA grouped-GEMM path even for small T           */
};

/* Text for a status code (static storage; never NULL). */
const char* moe_status_str(int status);

/* Library version string, e.g. "moe_w4 1.0 gfx950". */
const char* moe_version(void);

/* Bytes of workspace that any entry point below needs for up to T_max tokens with these
 * flags. Returns 0 if the descriptor is invalid or unsupported. */
size_t moe_workspace_bytes(const moe_layer_desc_t* desc, int32_t T_max, int32_t flags);

/* Upper bound on plan->num_blocks for T tokens: ceil(T*K/BM) + min(E, T*K) + ceil(T/BM). */
int32_t moe_plan_max_blocks(const moe_layer_desc_t* desc, int32_t T);

/* Router [P1 "The Model ..."]: for each token the top_k experts by router logit (rank order,
 * ties to the lower expert index), their softmax-renormalised weights, the shared expert's
 * sigmoid gate, and the per-expert token counts.
 *   x [T, H] bf16 -> topk_idx [T, K] int32, topk_w [T, K] fp32, shared_gate [T] fp32
 *   (may be NULL when Fs == 0), counts [E] int32.
 * Logits are formed with fp32 accuracy (prefill: a three-part bf16 split of the fp32 router
 * weights on bf16 MFMA; decode: fp32 FMA). workspace: moe_workspace_bytes(desc, T, 0). */
int moe_route(const moe_layer_desc_t* desc, const uint16_t* x, int32_t T,
              int32_t* topk_idx, float* topk_w, float* shared_gate, int32_t* counts,
              void* workspace, size_t ws_bytes, void* stream);

/* Histogram, exclusive scan, stable scatter and block map [P1 "How It Works ..."], all on
 * the device. topk_idx [T, K] int32 with values in [0, E) (out-of-range values are counted
 * nowhere and flagged by setting *plan->num_blocks = -1). Fills every array of `plan`.
 * workspace: moe_workspace_bytes(desc, T, 0). */
int moe_permute(const moe_layer_desc_t* desc, const int32_t* topk_idx, int32_t T,
                const moe_plan_t* plan, void* workspace, size_t ws_bytes, void* stream);

/* Grouped GEMM over the plan's block map with the 4-bit weights dequantised to bf16 inside
 * the kernel and fp32 accumulation on MFMA [P1 "The Model ...", "How It Works ..."].
 *   GATE_UP: in = x [T, H] bf16 (rows gathered through plan->sorted_slots; the shared
 *            expert reads x in token order); out = A bf16, routed rows [T*K, F] in grouped
 *            order followed by shared rows [T, Fs]: A = bf16(silu(x Wg^T) * (x Wu^T)).
 *   DOWN:    in = A as above; out = Y [T*K + T, H] fp32 = A Wd^T per grouped row (fp32
 *            accumulation, not rounded).
 *   DOWN_COMBINE(_ATOMIC): in = A; out = y [T, H] fp32 =
 *            sum_k topk_w[t,k] Y[slot_pos[t*K+k]] + shared_gate[t] * Y[T*K + t]
 *            with Y the fp32 rows of DOWN, summed in fp32 (overwritten, not accumulated).
 *            Needs topk_w and, when Fs > 0, shared_gate. DOWN_COMBINE stores Y in the
 *            workspace and adds the terms in rank order, then the shared term; _ATOMIC adds
 *            them in the down GEMM's epilogue with fp32 atomics (no Y array).
 * For T <= 16 (and F, Fs <= 512, T*H <= 32768) GATE_UP and DOWN_COMBINE run the decode
 * path's GEMV kernels (the same ones moe_layer_forward uses for such T; DOWN_COMBINE is then
 * deterministic and needs no workspace).
 * workspace: moe_workspace_bytes(desc, T, 0) (DOWN_COMBINE with T > 16 stages Y in it). */
int moe_grouped_gemm_w4(const moe_layer_desc_t* desc, int32_t which, const void* in, int32_t T,
                        const moe_plan_t* plan, const float* topk_w, const float* shared_gate,
                        void* out, void* workspace, size_t ws_bytes, void* stream);

/* Weighted combine [P1 "The Model ..."]: y[t] = sum_k topk_w[t,k] * y_perm[slot_pos[t*K+k]]
 *                        + shared_gate[t] * shared_y[t]     (the shared term only if Fs > 0)
 * y_perm [T*K, H] fp32 (grouped rows, as moe_grouped_gemm_w4 DOWN writes them), shared_y
 * [T, H] fp32 (rows T*K.. of that array), out [T, H] fp32 (overwritten), products and sums
 * in fp32. Deterministic: terms are added in rank order k = 0..K-1, then the shared term. */
int moe_combine(const moe_layer_desc_t* desc, const float* y_perm, const int32_t* slot_pos,
                const float* topk_w, const float* shared_y, const float* shared_gate,
                int32_t T, float* out, void* stream);

/* The whole layer [P1 "The Model ..."]: router (256 experts scored, 8 kept, one shared expert
 * on every token), SwiGLU experts over 4-bit g64 weights, weighted combine -- with routing,
 * histogram, scan, scatter and block maps on the GPU and no host synchronisation
 * [P1 "How It Works ..."]. x [T, H] bf16 -> out [T, H] fp32. T <= 16 takes the decode path
 * (bandwidth-bound: each selected expert's weights streamed once), larger T the prefill path
 * (MFMA grouped GEMM with the weights rebuilt tile by tile). For H <= 2048 and F, Fs <= 512 the decode path is three
 * launches: (router logits + the shared expert's gate/up), (top-k in every workgroup + the
 * selected experts' gate/up), (down projection fused with the weighted combine); each selected
 * expert's weights are streamed once with 16-byte loads, and the combine is deterministic.
 * Other decode shapes run the same steps as separate GEMV kernels.
 * flags: MOE_FLAG_*. workspace: moe_workspace_bytes(desc, T, flags). */
int moe_layer_forward(const moe_layer_desc_t* desc, const uint16_t* x, int32_t T, float* out,
                      void* workspace, size_t ws_bytes, int32_t flags, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code under HIP-graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels, with the
 * scratch memory taken from a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that each GPU the library runs on holds until the process ends. 64 MiB covers every decode
 * batch and a 512-token prefill chunk of the full-size layer (moe_workspace_bytes gives what a
 * call needs). The call allocates nothing (no hipMalloc, no allocating library routine); it
 * looks up the array's device address once per GPU (hipGetSymbolAddress, on the first call
 * on that device).
 *   Returns MOE_WORKSPACE_TOO_SMALL if moe_workspace_bytes(desc, T, flags) exceeds
 *   MOE_NOALLOC_SCRATCH_BYTES, MOE_HIP_ERROR if the array's address cannot be obtained, and
 *   otherwise what moe_layer_forward returns.
 *   All calls on one GPU share its array, which keeps the last call's contents (no kernel
 *   needs it cleared): calls that may overlap on one GPU (several streams or host threads)
 *   race and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const moe_layer_desc_t* desc, const uint16_t* x, int32_t T,
                              float* out, int32_t flags, void* stream);

/* moe_layer_forward as its sequence of kernel launches, one launch per call, for measuring
 * and checking the kernels one at a time. moe_layer_num_phases(desc, T, flags) gives the
 * number of launches for this T and these flags (0 if the arguments are invalid); calling
 * moe_layer_forward_phase for phases 0, 1, ... in order on one stream and one workspace gives
 * the same result as moe_layer_forward (phase -1 runs all of them). A phase reads what the
 * previous phases left in the workspace. The launches are
 *   decode (T <= 16, H <= 2048, F, Fs <= 512): router + shared expert; top-k + gate/up of the
 *     selected experts; down projection + combine
 *   other decode shapes: router; top-k + permutation; gate/up; down + combine
 *   prefill: router; top-k; permutation; gate/up GEMM; down GEMM storing Y; combine
 *     (MOE_FLAG_ATOMIC_COMBINE: ...; gate/up GEMM; zero fill of out; down GEMM + combine). */
int32_t moe_layer_num_phases(const moe_layer_desc_t* desc, int32_t T, int32_t flags);
int moe_layer_forward_phase(const moe_layer_desc_t* desc, const uint16_t* x, int32_t T,
                            float* out, void* workspace, size_t ws_bytes, int32_t flags,
                            int32_t phase, void* stream);

/* Residual update and RMSNorm between stacked layers ([P1] "The Model ...": a 40-layer stack;
 * "How It Works ...": the next step's input stays in a GPU-resident slot):
 *   init == 0: resid += y, then x = bf16( resid / sqrt(mean(resid^2) + eps) ) per row
 *   init == 1: resid = x (bf16 widened to fp32), then x = bf16(RMSNorm(resid)); y unused
 * y, resid [T, H] fp32, x [T, H] bf16 (read in place when init == 1), unit norm weight.
 * H a multiple of 64, at most 16384; eps >= 0. */
int moe_residual_rmsnorm(const float* y, float* resid, uint16_t* x, int32_t T, int32_t H,
                         float eps, int32_t init, void* stream);

/* A stack of MoE layers with the residual stream between them (pre-norm):
 *   resid = x;  x = bf16(RMSNorm(resid));
 *   for each layer l:  y = moe_layer_forward(layers[l], x);  resid += y;  x = bf16(RMSNorm(resid))
 * On entry x [T, H] bf16 holds the tokens; on return resid [T, H] fp32 holds the final
 * residual stream and x its normalised bf16 copy -- the input of the next decode step, left on
 * the device. All layers must share `hidden`. workspace: moe_stack_workspace_bytes(...)
 * (0 if invalid). Enqueue only, graph-capturable like moe_layer_forward. For decode-sized
 * batches the residual update and the normalisation run inside the layers' own kernels (three
 * launches per layer instead of four); the results are the same bits as the composition of
 * moe_layer_forward and moe_residual_rmsnorm. */
size_t moe_stack_workspace_bytes(const moe_layer_desc_t* const* layers, int32_t n_layers,
                                 int32_t T_max, int32_t flags);
int moe_stack_forward(const moe_layer_desc_t* const* layers, int32_t n_layers, float* resid,
                      uint16_t* x, int32_t T, float eps, void* workspace, size_t ws_bytes,
                      int32_t flags, void* stream);

/* Test export: dequantise row `row` of matrix `mat` of a projection with input size Kin
 * using the same device code as the GEMM kernels. out_f32 [Kin] receives scale*q + bias
 * as computed in fp32, out_bf16 [Kin] its bf16 rounding (either may be NULL). */
int moe_debug_dequant_w4(const moe_w4_t* w, int32_t n_rows, int32_t Kin, int32_t mat,
                         int32_t row, float* out_f32, uint16_t* out_bf16, void* stream);

/* Test export: byte offsets of the workspace regions that moe_layer_forward_phase leaves for
 * the next phase, so that a test can check each launch on its own. offsets[i] receives, for
 * T tokens and these flags, the offset of region i in this order:
 *   0 logits   router logits [T, E] fp32 then the shared-gate logits [T] (decode path), or
 *              up to 8 split-K partial slices [T, E+1] (prefill path)
 *   1 topk_idx [T, K] int32      2 topk_w [T, K] fp32        3 sgate [T] fp32
 *   4 route    decode route record, int32 words: D, expert[T*K], rows[T*K], first grouped
 *              row[T*K], token mask[T*K], routing weight per grouped row[T*K] (fp32),
 *              shared gate[T] (fp32); D entries in ascending expert order (T = 1: rank order)
 *   5 counts [E]   6 offsets [E+1]   7 sorted_slots [T*K]   8 slot_pos [T*K]
 *   9 blocks [max_blocks*4]   10 num_blocks [1]
 *   11 A [T*K*F + T*Fs] bf16 (grouped routed rows, then the shared rows)
 *   12 Y [T*K + T, H] fp32 (not with MOE_FLAG_ATOMIC_COMBINE: then equal to the total)
 *   13 total bytes (= moe_workspace_bytes)
 * n: entries of offsets (at most 14 are written). Returns MOE_OK, or an error as
 * moe_workspace_bytes would return 0. */
int moe_debug_workspace_layout(const moe_layer_desc_t* desc, int32_t T, int32_t flags,
                               size_t* offsets, int32_t n);

/* Measurement export: enqueues `workgroups` workgroups of four waves, each wave issuing
 * iters x 8 independent bf16 MFMAs (32x32x16, fp32 accumulation) on register operands, and
 * writes the flops that launch performs to *flops. Timed by the caller (events on `stream`), it
 * gives the dense bf16 matrix rate the chip sustains, beside the datasheet peak. sink: device
 * buffer of workgroups*256 floats, written only in an impossible case (keeps the loop alive). */
int moe_bench_mfma_loop(int32_t workgroups, int32_t iters, float* sink, double* flops,
                        void* stream);

/* Measurement export: reads `bytes` (a multiple of 16) of the device buffer p once with 16-byte
 * loads over `workgroups` workgroups of 256 threads (four loads in flight per thread). Timed by
 * the caller, it gives the HBM read rate a streaming kernel reaches. sink: device buffer of
 * workgroups*256 uint32, written only in an impossible case. */
int moe_bench_stream_read(const void* p, size_t bytes, int32_t workgroups, uint32_t* sink,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_H */
