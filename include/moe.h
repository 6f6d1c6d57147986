/*
 * moe.h - C ABI of libmoe, a single-GPU Mixture-of-Experts layer forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is: router (gate logits, scoring, selection bias, optional group
 * limit, top-k, renormalisation) -> block alignment (per-expert histogram,
 * padding, scan, expert-sorted assignment ids, block table, padded length on
 * the device) -> grouped expert GEMM1 with the SwiGLU epilogue -> grouped
 * GEMM2 -> weighted combine back to token order.
 *
 * Sources (web pages, cited by title and section):
 *   [Router]  "How an MoE Model Picks Its Experts During LLM Inference"
 *   [MoE]     "Mixture of Experts" (mlinterviewnotes.com inference course 07-01)
 *   [Kernels] "MoE Kernels, in depth: the six kernels of an expert layer ..."
 *   [MegaMoE] "How GPUs Fuse Communication and Computation During LLM Inference"
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - All tensor pointers are DEVICE pointers, row-major, contiguous, 16-byte
 *    aligned.  bf16 tensors are passed as void* holding bf16 bit patterns.
 *  - Ownership: the caller allocates every input, output and workspace buffer
 *    and keeps it alive until the enqueued work has finished.  The library
 *    borrows pointers for the duration of the enqueue only; it never
 *    allocates or frees device memory, never copies between host and device,
 *    never synchronises and never reads device memory from the host (except
 *    moe_debug_error, which is documented as synchronising).
 *  - All work is enqueued on `stream` in order; the calls are capturable in a
 *    HIP graph.  The padded length produced by moe_align stays on the device
 *    and later kernels read it there ([Kernels] "Alignment": no host sync).
 *  - Workspace: each call takes a caller-provided workspace of at least the
 *    size reported by its *_workspace_size query.  Every workspace begins
 *    with a 64 KiB control block (router counters, alignment error bits)
 *    that no other region of any entry point overlaps.  The workspace must be
 *    ZERO-FILLED before its first use; every call leaves the control block's
 *    counters at zero again, so one workspace can be reused by any sequence
 *    of calls of any shapes on one stream.  Calls that overlap in time must
 *    not share a workspace.
 *  - Errors: arguments are validated on the host only (scalars and non-null
 *    pointers); a violation returns MOE_E_INVAL and enqueues nothing.  A
 *    workspace below the required size returns MOE_E_WORKSPACE.  An
 *    unsupported combination (e.g. a weight format with a dimension that is
 *    not a multiple of its scale block) returns MOE_E_UNSUPPORTED.  A launch
 *    failure reported by the HIP runtime returns MOE_E_HIP.  T = 0 is a valid
 *    no-op that returns MOE_OK.
 *  - The library is re-entrant and keeps no state between calls apart from
 *    per-device occupancy figures it queries once (thread-safe).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_E_INVAL = 1,        /* bad scalar argument or null required pointer   */
  MOE_E_UNSUPPORTED = 2,  /* valid but unsupported shape / format combination */
  MOE_E_WORKSPACE = 3,    /* workspace smaller than the query reports        */
  MOE_E_HIP = 4           /* the HIP runtime reported an error at launch      */
} moe_status;

/* Scoring of the router logits ([Router] §1.3 "The Rank Key and the Weight"):
 * softmax over the experts (Mixtral, Qwen3) or an independent sigmoid per
 * expert (DeepSeek-V3 and successors). */
typedef enum moe_scoring {
  MOE_SOFTMAX = 0,       /* softmax over the E logits                        */
  MOE_SIGMOID = 1,       /* sigmoid per expert                               */
  MOE_SQRTSOFTPLUS = 2   /* sqrt(softplus(logit)) per expert ([Router] §1.3:
                            the DeepSeek-V4 variant of the sigmoid score)    */
} moe_scoring;

/* Expert weight storage formats.
 *  MOE_W_BF16:          w13 bf16 [E, 2F, H], w2 bf16 [E, H, F]; scales unused.
 *  MOE_W_FP8_BLOCK128:  OCP e4m3 codes (uint8) w13 [E, 2F, H], w2 [E, H, F];
 *                       float32 scales w13_scale [E, 2F/128, H/128],
 *                       w2_scale [E, H/128, F/128] (one per 128x128 block;
 *                       [Kernels] "Combine, backward and low precision").
 *                       Activations are quantised to e4m3 with one float32
 *                       scale amax/448 per 1x128 group.  H, F multiples of 128.
 *  MOE_W_MXFP4:         OCP e2m1 codes packed two per byte along K (element 2j
 *                       in the low nibble of byte j): w13 uint8 [E, 2F, H/2],
 *                       w2 uint8 [E, H, F/2]; e8m0 scales (uint8, 2^(s-127))
 *                       w13_scale [E, 2F, H/32], w2_scale [E, H, F/32].
 *                       Activations are e4m3 with one power-of-two e8m0 scale
 *                       pow2_at_least(amax/448) per 32 ([MegaMoE] §1.1, §3.5).
 *                       H, F multiples of 128.
 *  In every format w13 holds the F gate rows first, then the F up rows
 *  ([MoE] "Shapes, sourced"; [MegaMoE] §3.5). */
typedef enum moe_wformat {
  MOE_W_BF16 = 0,
  MOE_W_FP8_BLOCK128 = 1,
  MOE_W_MXFP4 = 2
} moe_wformat;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(moe_status s);

/* Hash of the sources the library was built from (16 hex digits of a
 * sha256 over the HIP sources, headers and build script; static string).
 * The Python loader compares it with the sources beside the library and
 * refuses a library built from other sources. */
const char* moe_source_hash(void);

/* ------------------------------------------------------------------------
 * moe_route - the router ([Router] §1.1 "Three Steps", §1.3, §5.3;
 * [MoE] fused_topk and grouped_topk listings; [Kernels] "Router: one fused
 * kernel").
 *
 *  x        bf16 [T, H]      hidden states
 *  gate     [E, H]           gate weight (one row per expert): float32 if
 *                            gate_is_fp32 is 1, bf16 if it is 0 (the form
 *                            [Router] §1.1 / §2.4 / §5.1 describes engines
 *                            storing: bf16 rows, fp32 logits; half the bytes)
 *  bias     float32 [E]      selection bias added to the score to form the
 *                            rank key (NULL: rank key = score).  Only the
 *                            choice uses it; weights use the unbiased score.
 *  n_group, topk_group       group-limited routing: experts form n_group
 *                            equal groups; a group scores the sum of its two
 *                            largest rank keys; only the topk_group best
 *                            groups may be chosen.  n_group = 1 disables it.
 *  scoring                   moe_scoring
 *  renormalize               nonzero: w_j = s_j / (sum_j s_j + 1e-20)
 *  routed_scale              multiplies the weights after renormalising
 *  topk_ids   int32 [T, k]   out: chosen experts in round order (descending
 *                            rank key, lowest expert id first on ties)
 *  topk_weights float32 [T, k] out: their weights
 *  logits_out float32 [T, E] optional out (NULL allowed): the fp32 logits
 *
 * Arithmetic: logits accumulate bf16(x) * gate to fp32 accuracy (an fp32
 * gate split exactly into three bf16 planes on matrix cores; a bf16 gate
 * taken as it is) in one fixed order for every T: a token's logits and
 * choice do not depend on the batch it is in ([Router] §9).  Scores, keys
 * and weights are fp32.
 * Constraints: gate_is_fp32 in {0, 1}; 0 <= T <= 2^24, H >= 128 and a
 * multiple of 128,
 * 1 <= k <= E <= 1024, k <= 16; n_group divides E, E/n_group >= 2 when n_group > 1,
 * 1 <= topk_group <= n_group, k <= topk_group * E / n_group.
 * ------------------------------------------------------------------------ */
moe_status moe_route(const void* x, const void* gate, int gate_is_fp32, const float* bias,
                     int T, int H, int E, int k, int n_group, int topk_group,
                     int scoring, int renormalize, float routed_scale,
                     int32_t* topk_ids, float* topk_weights, float* logits_out,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream);
size_t moe_route_workspace_size(int T, int H, int E);

/* ------------------------------------------------------------------------
 * moe_align - block alignment ([MoE] "vLLM's Triton path: align, then
 * index"; [Kernels] "Alignment: making ragged routing tileable").
 *
 *  topk_ids       int32 [T, k]; assignment a = t*k + j routes to topk_ids[a].
 *                 An id of -1 is skipped (not a local expert).  Any other id
 *                 outside [0, E) is skipped and sets a sticky error bit in the
 *                 workspace (read with moe_debug_error).
 *  block_m        rows per block, 1..1024 (moe_expert_ffn and moe_layer
 *                 take 16, 32, 64 or 128)
 *  sorted_ids     int32 [moe_align_max_padded(T,k,E,block_m)] out: expert e's
 *                 assignments, ascending in a, start at the exclusive prefix
 *                 sum of ceil(count/block_m)*block_m over experts < e; every
 *                 other slot holds the sentinel T*k.
 *  block_expert   int32 [moe_align_max_blocks(T,k,E,block_m)] out: expert of
 *                 each block below the padded length, -1 after it.
 *  num_post_padded int32 [1] out (device): the padded length.
 * The result is deterministic (no atomics decide any position).
 * Constraints: T >= 0, 1 <= k <= 16, 1 <= E <= 1024, T*k <= 2^24.
 * ------------------------------------------------------------------------ */
moe_status moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m,
                     int32_t* sorted_ids, int32_t* block_expert,
                     int32_t* num_post_padded,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream);
size_t moe_align_workspace_size(int T, int k, int E);
/* Worst-case padded length T*k + E*(block_m-1), and its block count. */
int64_t moe_align_max_padded(int T, int k, int E, int block_m);
int64_t moe_align_max_blocks(int T, int k, int E, int block_m);

/* ------------------------------------------------------------------------
 * moe_route_align - moe_route followed by moe_align in one call, one
 * launch while T <= 4 ([Router] §6 and §6.1: one routing stage that
 * scores, selects, counts and sorts; [Router] §8.1: the gate product stays
 * expert-parallel, the selection row-parallel).
 *
 * Arguments as moe_route (without logits_out) and moe_align, with the same
 * layouts, ownership and results: topk_ids / topk_weights are written and
 * then aligned with block_m.  With n_shared = 0 the outputs equal those of
 * moe_route followed by moe_align on the same stream, bit for bit.  For
 * T <= 4, and for T <= 64 while ceil(T / 4) * E * H * 4 bytes (the gate
 * read once per 4-token tile) stay within 24 MiB, the router's workgroups
 * compute the gate product and each 4-token tile's last one selects its
 * tokens, one per wave; at T <= 4 that workgroup also aligns them in the
 * same launch, otherwise moe_align's launch follows.  Elsewhere the
 * router's two launches run (logits, then one wave per token), then
 * moe_align's.
 *  n_shared       0, or 1 for a shared expert as an always-selected slot
 *                 ([MoE] SGLang's fused shared expert: appended as expert
 *                 id E, top-k becomes top-(k+1); [MegaMoE] §3.8: its output
 *                 is added to the routed sum): topk_ids / topk_weights are
 *                 then [T, k+1] with slot k = (E, 1.0) for every token, and
 *                 the alignment covers E+1 experts (its buffers sized with
 *                 moe_align_max_*(T, k+1, E+1, block_m)).
 * Errors: as moe_route and moe_align (validated on the host before anything
 * is enqueued); n_shared outside {0, 1}, or E + n_shared > 1024, or
 * k + n_shared > 16: MOE_E_INVAL.  The workspace must hold
 * moe_route_align_workspace_size(T, H, E, k, n_shared) bytes.
 * ------------------------------------------------------------------------ */
moe_status moe_route_align(const void* x, const void* gate, int gate_is_fp32, const float* bias,
                           int T, int H, int E, int k, int n_shared,
                           int n_group, int topk_group,
                           int scoring, int renormalize, float routed_scale,
                           int block_m, int32_t* topk_ids, float* topk_weights,
                           int32_t* sorted_ids, int32_t* block_expert,
                           int32_t* num_post_padded,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);
size_t moe_route_align_workspace_size(int T, int H, int E, int k, int n_shared);

/* ------------------------------------------------------------------------
 * moe_expert_ffn - grouped expert GEMMs and combine ([Kernels] "The fused
 * expert GEMM" and "Combine"; [MoE] align-then-index path; [MegaMoE] §1.1,
 * §3.5).
 *
 *  x              bf16 [T, H]
 *  wformat, w13, w13_scale, w2, w2_scale    see moe_wformat
 *  topk_ids       int32 [T, k], topk_weights float32 [T, k] (the router's)
 *  sorted_ids, block_expert, num_post_padded  moe_align's outputs for the
 *                 same topk_ids and block_m
 *  swiglu_limit   L > 0: before SwiGLU the gate is capped at L and the up
 *                 value clipped to [-L, L] ([MegaMoE] §3.5, DeepSeek-V4);
 *                 +infinity: no clamp.  NaN or L <= 0: MOE_E_INVAL.
 *  y              bf16 [T, H] out:
 *                 y[t] = sum_j w[t,j] * W2_e (silu(g) * u), g = W1_e x_t and
 *                 u = W3_e x_t (clamped with a finite L), e = topk_ids[t,j],
 *                 summed over j in slot order in fp32 and rounded once;
 *                 slots whose id is outside [0, E) add nothing.
 * Each block of block_m rows multiplies by exactly one expert's weights;
 * rows are gathered through sorted_ids / k; blocks at or past the padded
 * length exit without work.  The SwiGLU output and the expert outputs are
 * bf16 in the workspace (fp8 with scales for the quantised formats).
 * Constraints: H and F multiples of 128 (bf16) or of 512 (fp8 formats,
 * else MOE_E_UNSUPPORTED); block_m in {16, 32, 64, 128}; k <= 16;
 * E <= 1024; x [T, H], the SwiGLU rows [max padded rows, F] and one
 * expert's w13 [2F, H] each below 4 GiB (the kernels address them with
 * 32-bit byte offsets), else MOE_E_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
moe_status moe_expert_ffn(const void* x, int wformat,
                          const void* w13, const void* w13_scale,
                          const void* w2, const void* w2_scale,
                          const int32_t* topk_ids, const float* topk_weights,
                          const int32_t* sorted_ids,
                          const int32_t* block_expert,
                          const int32_t* num_post_padded,
                          int T, int H, int E, int F, int k, int block_m,
                          float swiglu_limit,
                          void* y, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);
size_t moe_expert_ffn_workspace_size(int T, int H, int E, int F, int k,
                                     int block_m, int wformat);

/* Measurement hook: the same call as moe_expert_ffn, but only the stages in
 * `stages` (a bit mask of moe_ffn_stage) are enqueued, in pipeline order.  A
 * stage reads what the earlier stages left in the workspace, so running one
 * stage alone is meaningful only after a call that ran the stages before it
 * with the same arguments and workspace.  Lets a caller bracket a single
 * kernel with events.  Unknown bits return MOE_E_INVAL. */
typedef enum moe_ffn_stage {
  MOE_STAGE_QUANT = 1,    /* activation quantisation (fp8 formats); the   */
                          /* tile table of the paired GEMMs (bf16 and     */
                          /* MXFP4, block_m 64 or 128)                    */
  MOE_STAGE_GEMM1 = 2,    /* grouped GEMM1 + SwiGLU epilogue              */
  MOE_STAGE_GEMM2 = 4,    /* grouped GEMM2                                */
  MOE_STAGE_COMBINE = 8,  /* weighted slot-order combine into y           */
  MOE_STAGE_ALL = 15
} moe_ffn_stage;
moe_status moe_expert_ffn_stages(const void* x, int wformat,
                                 const void* w13, const void* w13_scale,
                                 const void* w2, const void* w2_scale,
                                 const int32_t* topk_ids,
                                 const float* topk_weights,
                                 const int32_t* sorted_ids,
                                 const int32_t* block_expert,
                                 const int32_t* num_post_padded,
                                 int T, int H, int E, int F, int k, int block_m,
                                 float swiglu_limit, void* y, void* workspace,
                                 size_t workspace_bytes, int stages,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_layer - the whole forward: moe_route -> moe_align -> moe_expert_ffn
 * on one stream with one workspace (arguments as above; the router and
 * the alignment run as moe_route_align).
 *  E, k           routed experts and routed slots per token.
 *  n_shared       0, or 1 for a shared expert (see moe_route_align): w13,
 *                 w2 and their scales then hold E + 1 experts, the shared
 *                 one last, and y adds its output with weight 1.
 *  block_m        0 lets the library choose from the tokens per expert
 *                 (moe_layer_block_m of T, E + n_shared, F, k + n_shared
 *                 and wformat);
 *                 otherwise 16, 32, 64 or 128.
 *  topk_ids_out, topk_weights_out   optional outputs (NULL allowed),
 *                 [T, k + n_shared].
 * ------------------------------------------------------------------------ */
moe_status moe_layer(const void* x, const void* gate, int gate_is_fp32, const float* bias,
                     int wformat, const void* w13, const void* w13_scale,
                     const void* w2, const void* w2_scale,
                     int T, int H, int E, int F, int k, int n_shared,
                     int n_group, int topk_group, int scoring,
                     int renormalize, float routed_scale, int block_m,
                     float swiglu_limit,
                     void* y, int32_t* topk_ids_out, float* topk_weights_out,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream);
size_t moe_layer_workspace_size(int T, int H, int E, int F, int k, int n_shared,
                                int block_m, int wformat);
/* ------------------------------------------------------------------------
 * moe_layer_noalloc - moe_layer without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, layouts, results and errors are those of moe_layer; the bits of
 * y (and of the optional routing outputs) equal moe_layer's for the same
 * arguments.  The workspace is a scratch array of MOE_NOALLOC_SCRATCH_BYTES
 * (128 MiB) that the library holds on each GPU it runs on, from the first
 * call on that GPU until the process ends.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).
 *  - A call whose moe_layer_workspace_size(T, H, E, F, k, n_shared, block_m,
 *    wformat) exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_E_WORKSPACE and
 *    enqueues nothing.  Every decode shape of the five layer configurations
 *    (T <= 512) fits; the prefill shapes (e.g. 2048 tokens at H 7168) do not.
 *  - The first call on a GPU looks up that GPU's scratch address (with the
 *    stream's device made current for the lookup) and clears the scratch's
 *    control block with one small kernel on `stream` before the layer.
 *  - Every call on one GPU uses that GPU's one scratch array, which keeps the
 *    last call's contents: calls that overlap in time on one GPU (two
 *    streams, two threads) RACE and give undefined results.  Serialise them.
 * ------------------------------------------------------------------------ */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status moe_layer_noalloc(const void* x, const void* gate, int gate_is_fp32, const float* bias,
                             int wformat, const void* w13, const void* w13_scale,
                             const void* w2, const void* w2_scale,
                             int T, int H, int E, int F, int k, int n_shared,
                             int n_group, int topk_group, int scoring,
                             int renormalize, float routed_scale, int block_m,
                             float swiglu_limit,
                             void* y, int32_t* topk_ids_out, float* topk_weights_out,
                             hipStream_t stream);

/* The block size moe_layer uses for block_m = 0, from the mean rows per
 * expert m = T*k/E: 32 if 2 <= m <= 24, then 64 while m <= 96 (m <= 44 for
 * MOE_W_FP8_BLOCK128), else 128.  Below
 * m = 2: 16 for MOE_W_FP8_BLOCK128; for bf16 and MXFP4, 32 once the
 * expected number of 32-row GEMM1 tiles, E (1 - (1 - k/E)^T) * 2F / 256,
 * reaches 400 (bf16) or 320 (MXFP4), else 16. */
int moe_layer_block_m(int T, int E, int F, int k, int wformat);

/* ------------------------------------------------------------------------
 * Diagnostics and measurement probes (not part of the layer).
 *
 * moe_debug_error: SYNCHRONISES `stream`, returns the sticky error bits that
 *   moe_align recorded in `workspace` (bit 0: an id outside [-1, E)) and
 *   clears them.  For tests only.
 * moe_probe_empty: enqueues one kernel that does nothing (launch floor,
 *   [Router] §3.3 "The Floor").
 * moe_probe_read: enqueues one kernel that reads `bytes` bytes at `p` once in
 *   16-byte loads and writes one float per workgroup to `sink`
 *   (sink: float32 [moe_probe_read_sink_len(bytes)]); the bare weight-read
 *   kernel of [Router] §3.3.  bytes must be a multiple of 16.
 * moe_probe_mfma: enqueues `grid` workgroups of 4 waves; each wave issues
 *   iters x accs matrix-core instructions on register constants, cycling
 *   through `accs` (4, 8 or 16) independent accumulators, and writes one
 *   float per thread to `sink` (float32 [moe_probe_mfma_sink_len(grid)]).
 *   kind: 0 bf16 16x16x32, 1 bf16 32x32x16 (accs 4 or 8), 2 e4m3 x e4m3,
 *   3 e4m3 x e2m1, 4 e2m1 x e2m1 (the last three 16x16x128 with e8m0
 *   scales).  FLOPs per instruction: 2 M N K.  The issue-rate ceiling of the
 *   instruction the grouped GEMMs use for each weight format.  Bad arguments:
 *   MOE_E_INVAL.
 * ------------------------------------------------------------------------ */
int32_t moe_debug_error(void* workspace, hipStream_t stream);
moe_status moe_probe_empty(hipStream_t stream);
moe_status moe_probe_read(const void* p, size_t bytes, float* sink,
                          hipStream_t stream);
size_t moe_probe_read_sink_len(size_t bytes);
moe_status moe_probe_mfma(int kind, int accs, int grid, int iters, float* sink,
                          hipStream_t stream);
size_t moe_probe_mfma_sink_len(int grid);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
