/*
 * moe.h -- C ABI of the MI355X (gfx950) fused Mixture-of-Experts layer.
 *
 * The layer (one batched GPU operation instead of a loop over experts):
 *   1. route:   logits = x . W_gate^T (fp32), the top_k experts per token
 *               (ties to the lower expert index), gates = softmax over the
 *               selected logits;
 *   2. align:   regroup the T*top_k routing slots by expert into blocks of
 *               block_m rows (padded, slots ascending inside an expert);
 *   3. W13:     per expert, h = SiLU(W1 x) * (W3 x) for the expert's tokens;
 *   4. W2:      y = gate * (W2 h) per routing slot;
 *   5. combine: out[t] = sum of the token's top_k slot outputs, in rank order.
 * Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal gyorsítja
 * a SageMaker AI-t", section "A fused MoE a számítási folyamat több lépését
 * egyesíti" (routing, data rearrangement and expert computation fused into
 * one batched GPU operation) and section "FP8 esetén a Triton backend
 * bizonyult gyorsabbnak" (FP8 scaling, matrix product and aggregation of the
 * experts' results in one pass); the French page "Ingénierie de kernels
 * Mixture-of-Experts sur Amazon SageMaker AI", first paragraph.  The pages do
 * not write out the router rule, the expert network or the FP8 format; the
 * readings above (softmax/top-k, SwiGLU with W13 = [W1; W3], OCP e4m3fn)
 * are the plain ones and are fixed by this ABI.
 *
 * Conventions for every entry point:
 *   - Tensors are caller-owned DEVICE buffers, contiguous, row-major, 16-byte
 *     aligned.  The library never allocates, frees or retains them (a
 *     moe_graph keeps their addresses, see moe_graph_create); inputs must
 *     stay alive and unmodified until the stream reaches the work.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns at once.  Outputs are valid once the stream has
 *     executed it.  Outputs are fully overwritten, never accumulated into.
 *   - Every argument is validated on the host before any HIP call; a bad
 *     argument returns a negative status and enqueues nothing.  No C++
 *     exception crosses the ABI.  MOE_ERR_HIP reports a failed launch.
 *   - T = 0 is valid: after the descriptor is validated the call returns
 *     MOE_OK, enqueues nothing and looks at no other argument.
 *   - Inputs are assumed finite.  A NaN logit ranks below every number.
 *   - Calls that share a workspace on one stream are ordered by the stream;
 *     concurrent calls on different streams need different workspaces.
 *
 * Shapes (row-major):
 *   x       [T, d]        act dtype (MOE_DTYPE_F32 or MOE_DTYPE_BF16)
 *   W_gate  [E, d]        fp32
 *   W13     [E, 2I, d]    weight dtype; rows 0..I-1 = W1 (gate projection),
 *                         rows I..2I-1 = W3 (up projection)
 *   W2      [E, d, I]     weight dtype
 *   out     [T, d]        act dtype (fp32 -> bf16 rounding is to nearest even)
 * Supported (act, weight) pairs: (F32, F32), (BF16, BF16), (BF16, E4M3FN).
 * E4M3FN weights are OCP e4m3fn bytes; value = decoded byte * fp32 scale, the
 * scale given per output channel (s13 [E, 2I], s2 [E, d]) or per expert
 * matrix (s13 [E], s2 [E]).  Activations stay bf16 (weight-only FP8) unless
 * desc->act_quant selects the W8A8 mode (MOE_ACT_MX_E4M3 below).
 * Limits: d and I multiples of 64 in [64, 2^19]; 1 <= E <= 1024;
 * 1 <= top_k <= min(E, 64);
 * T * top_k < 2^30; block_m in {0 (library default), 16, 32, 64, 128, 256};
 * 256 needs bf16 weights, d % 256 == 0, I % 128 == 0, 4*I*d < 2^31 and
 * 2*T*d < 2^31 (an expert's W13 and x addressed with 32-bit byte offsets).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

/* ---- status codes ---- */
#define MOE_OK 0
#define MOE_ERR_NULL_PTR (-1)      /* a required pointer is NULL            */
#define MOE_ERR_BAD_SHAPE (-2)     /* dimension out of range / not aligned  */
#define MOE_ERR_BAD_TOPK (-3)      /* top_k < 1, > E or > 64                */
#define MOE_ERR_BAD_DTYPE (-4)     /* unsupported dtype pair or scale mode  */
#define MOE_ERR_MISALIGNED (-5)    /* a pointer is not 16-byte aligned      */
#define MOE_ERR_WORKSPACE (-6)     /* workspace NULL or too small           */
#define MOE_ERR_HIP (-7)           /* a HIP call or kernel launch failed    */
#define MOE_ERR_BAD_BLOCK_M (-8)   /* block_m not allowed for the desc      */
#define MOE_ERR_BAD_ARG (-9)       /* any other invalid argument            */
#define MOE_ERR_NOALLOC_SIZE (-10) /* moe_forward_noalloc: workspace needed  */
                                   /* exceeds MOE_NOALLOC_WORKSPACE_BYTES    */

/* ---- dtypes and scale modes ---- */
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1
#define MOE_DTYPE_E4M3FN 2

/* Activations seen by the expert products.  MOE_ACT_MX_E4M3 (the W8A8 mode;
 * Hungarian page, section "FP8 esetén ...": FP8 scaling fused with the
 * matrix product) quantises x per token before W13 and h per routing slot
 * before W2 to e4m3fn in blocks of 32 consecutive values of a row, each block
 * with one power-of-two scale 2^(floor(log2 amax) - 8) (at least 2^-127; 1
 * for an all-zero block), values rounded to nearest even after clamping to
 * +-448.  Requires bf16 activations, e4m3fn weights, block_m 0 or 256 (0
 * means 256 here), d and I multiples of 256, 2*I*d and T*d under 2^31.  The
 * router still sees x as given. */
#define MOE_ACT_AS_IS 0
#define MOE_ACT_MX_E4M3 1

/* How the expert products hand their tiles to workgroups (Hungarian page,
 * section "FP8 esetén ...": dynamic scheduling layouts for token groups of
 * varying size; section "A fused MoE ...": one batched GPU operation).
 * With 128-token blocks (block_m 128), MOE_SCHED_STATIC and
 * MOE_SCHED_QUEUE select the token-tiled GEMM: MOE_SCHED_STATIC is one
 * workgroup per possible (row block, output-channel group) tile, in an
 * XCD-aware raster, those of row blocks past the realised ones exiting at
 * once; MOE_SCHED_QUEUE is as many workgroups as the GPU holds at once
 * taking only the realised tiles, from one work queue per XCD, helping drain
 * the other queues when their own is empty.  MOE_SCHED_AUTO takes the
 * register-token tile there instead (static raster; bf16 activations, bf16
 * weights with d and I multiples of 64 and at least 256, or e4m3fn weights
 * with d and I multiples of 128 and at least 384; I a multiple of 32), else
 * the 128-token tile with both operands through LDS (e4m3fn, d and I
 * multiples of 256; static raster), else the GEMM's queue.  In moe_forward
 * with bf16 weights and
 * activations on the decode path (blocks of 16 or 32 tokens, d and I
 * multiples of 256, T <= 64): MOE_SCHED_STATIC runs W13, W2 and the combine
 * as three launches; MOE_SCHED_QUEUE runs them as one persistent launch
 * whose workgroups take W13 tiles, then W2 tiles (each once the W13 tiles it
 * reads are done), from one ticket counter, and add up each token's slots as
 * soon as its last partial lands.  MOE_SCHED_AUTO (0) is, on the decode
 * path, the three launches, except that for at
 * most two row blocks of 16 (one token of a top-2 layer) W2 adds up each
 * token's slots itself (two launches: the last W2 workgroup to finish a
 * token's channel group sums its partials).  The persistent kernel is
 * slower there (its W2 tiles wait for the W13 tiles they read, and read
 * those h rows at device scope, past their own XCD's L2).  The static and queue
 * schedules give bit-identical outputs, and on the decode path so does the
 * automatic one; with 128-token blocks its tiles sum over K in another
 * order (equal within rounding).  Other paths ignore the field. */
#define MOE_SCHED_AUTO 0
#define MOE_SCHED_STATIC 1
#define MOE_SCHED_QUEUE 2

#define MOE_SCALE_NONE 0         /* F32 / BF16 weights                       */
#define MOE_SCALE_PER_TENSOR 1   /* one fp32 scale per expert matrix: [E]    */
#define MOE_SCALE_PER_CHANNEL 2  /* one per output row: [E,2I] and [E,d]     */

/* Problem description.  block_m is the row-block size of the regrouped
 * layout (align); 0 lets the library choose from the shape. */
typedef struct moe_desc {
  int64_t num_tokens;    /* T >= 0                   */
  int64_t hidden;        /* d                        */
  int64_t num_experts;   /* E                        */
  int64_t intermediate;  /* I                        */
  int32_t act_dtype;     /* MOE_DTYPE_F32 / _BF16    */
  int32_t weight_dtype;  /* MOE_DTYPE_F32/_BF16/_E4M3FN */
  int32_t block_m;       /* 0 or 16/32/64/128/256    */
  int32_t act_quant;     /* MOE_ACT_AS_IS or MOE_ACT_MX_E4M3 */
  int32_t schedule;      /* MOE_SCHED_*              */
  int32_t reserved;      /* must be 0                */
} moe_desc;

/* FP8 weight scales (device pointers, fp32).  Pass NULL (or mode
 * MOE_SCALE_NONE) for F32 / BF16 weights. */
typedef struct moe_scales {
  int32_t mode;          /* MOE_SCALE_*              */
  int32_t reserved;      /* must be 0                */
  const float* w13;      /* [E, 2I] or [E]           */
  const float* w2;       /* [E, d]  or [E]           */
} moe_scales;

/* ---- sizing ---- */

/* The block size the library uses for `desc` (desc->block_m, or the default
 * it picks when that is 0) and the capacity of the regrouped layout:
 * capacity = roundup(A + min(E, A) * (block_m - 1), block_m) rows, A = T*top_k
 * (each expert that receives a slot pads at most block_m - 1 rows).
 * sorted_ids needs `capacity` int32 entries, block_expert capacity/block_m. */
MOE_API int moe_align_capacity(const moe_desc* desc, int top_k, int32_t* block_m,
                               int64_t* capacity);

/* Bytes of device workspace moe_forward (with_routing = 1) or
 * moe_expert_ffn (with_routing = 0) needs for `desc`. */
MOE_API int moe_workspace_bytes(const moe_desc* desc, int top_k, int with_routing,
                                size_t* bytes);

/* ---- the fused layer ---- */

/* out = MoE(x).  Runs route, align, W13+SiLU*mul, W2+gate scale and combine
 * on `stream` with no host synchronisation.  `workspace` is a device buffer
 * of at least moe_workspace_bytes(desc, top_k, 1) bytes, 256-byte aligned;
 * its contents on entry do not matter.  `scales` may be NULL unless the
 * weights are E4M3FN.  (Hungarian page, section "A fused MoE ...": routing,
 * rearrangement and expert compute as one batched operation.) */
MOE_API int moe_forward(const moe_desc* desc, const void* x, const float* w_gate,
                        const void* w13, const void* w2, int top_k,
                        const moe_scales* scales, void* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same layer, checks and results, bit for bit, with no workspace
 * argument.  Its workspace is a static device array of
 * MOE_NOALLOC_WORKSPACE_BYTES bytes inside the library, one per GPU, which
 * exists from the library's load until the process ends; the call allocates
 * and frees nothing (no hipMalloc, no allocating library routine).
 *   - Size limit: returns MOE_ERR_NOALLOC_SIZE, enqueuing nothing, when
 *     moe_workspace_bytes(desc, top_k, 1) exceeds the array (it holds every
 *     decode batch up to 64 tokens at d = 4096, I = 14336, E = 8, top-2, and
 *     64 tokens at d = 7168, I = 2048, E = 256, top-8; larger batches need
 *     moe_forward and a caller workspace).
 *   - Sharing: every call on one GPU uses that GPU's one array, which keeps
 *     whatever the last call left in it (nothing reads it before writing).
 *     Calls ordered on one stream are safe; calls that may overlap on one
 *     GPU (different streams, or threads without ordering) race on the
 *     array and give wrong results.
 *   - The device is the stream's (the current device for the null stream);
 *     the first call on a device looks up the array's address there (a HIP
 *     call, MOE_ERR_HIP if it fails).
 * Other arguments, ownership and errors as moe_forward; asynchronous on
 * `stream`. */
#define MOE_NOALLOC_WORKSPACE_BYTES (64u << 20)
MOE_API int moe_forward_noalloc(const moe_desc* desc, const void* x, const float* w_gate,
                                const void* w13, const void* w2, int top_k,
                                const moe_scales* scales, void* out, void* stream);

/* ---- stage entry points (the same kernels moe_forward runs) ---- */

/* Routing.  Writes logits_out [T, E] fp32 (x . W_gate^T, fp32 products and
 * sums), topk_ids [T, top_k] int32 in rank order (descending logit, ties to
 * the lower index) and topk_w [T, top_k] fp32 gates (softmax over the
 * selected logits; they sum to 1 per token).  All three are required.
 * (Hungarian page, section "A fused MoE ...": token routing.) */
MOE_API int moe_route(const moe_desc* desc, const void* x, const float* w_gate, int top_k,
                      float* logits_out, int32_t* topk_ids, float* topk_w, void* stream);

/* Top-k selection and gates from given logits [T, E] fp32 (the second half
 * of moe_route, same kernel): the token routing of the Hungarian page,
 * section "A fused MoE ..." (which names the step, not its rule; the rule is
 * the reading at the top of this header: the top_k largest logits, ties to
 * the lower expert index, gates = softmax over the selected logits).  Lets a
 * caller check routing against any logits.  logits, topk_ids [T, top_k]
 * int32 and topk_w [T, top_k] fp32 are caller-owned device buffers; same
 * outputs, rules and errors as moe_route; asynchronous on `stream`. */
MOE_API int moe_route_logits(const moe_desc* desc, const float* logits, int top_k,
                             int32_t* topk_ids, float* topk_w, void* stream);

/* Regrouping by expert (the pages' "data rearrangement"; Hungarian page,
 * section "A fused MoE ..."; French page, first paragraph).  From topk_ids
 * [T, top_k] writes:
 *   counts      [E]          slots routed to each expert;
 *   sorted_ids  [capacity]   expert e's group starts at
 *                            sum_{e'<e} roundup(counts[e'], block_m) and
 *                            lists its flat slot ids f = t*top_k + j in
 *                            ascending order, padded with the sentinel
 *                            A = T*top_k; entries past the padded total = A;
 *   block_expert[capacity/block_m]  owner expert of each block, -1 past the
 *                            padded total;
 *   num_padded  [1]          the padded total (a multiple of block_m).
 * Ids outside [0, E) are ignored (their slot is dropped).  Deterministic. */
MOE_API int moe_align(const moe_desc* desc, const int32_t* topk_ids, int top_k,
                      int32_t* counts, int32_t* sorted_ids, int32_t* block_expert,
                      int32_t* num_padded, void* stream);

/* Routing and regrouping in one call: the outputs of moe_route (logits
 * [T, E], topk_ids [T, top_k], topk_w [T, top_k]) followed by those of
 * moe_align (counts, sorted_ids, block_expert, num_padded, laid out and
 * sized as moe_align documents for the same desc), with the same rules,
 * bit for bit.  The pages fuse the routing and the data rearrangement with
 * the expert computation into one GPU operation (Hungarian page, section
 * "A fused MoE ..."); here, for bf16 activations with T <= 16 and E <= 16,
 * the workgroup that selects the experts also regroups the slots, so the
 * two steps are a single kernel launch (otherwise the two steps' kernels run
 * back to back).  moe_forward takes the same path.  All pointers are device
 * buffers owned by the caller; outputs are overwritten; errors as moe_route.
 * Asynchronous on `stream`. */
MOE_API int moe_route_align(const moe_desc* desc, const void* x, const float* w_gate, int top_k,
                            float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                            int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                            void* stream);

/* Expert computation and combine for an existing routing: W13 grouped
 * product with SiLU(gate)*up, W2 grouped product scaled by the slot's gate,
 * sum of each token's slots into out [T, d].  topk_w [T, top_k] fp32 and
 * sorted_ids / block_expert / num_padded as written by moe_align with the
 * same desc (same block_m).  `workspace`: moe_workspace_bytes(desc, top_k, 0)
 * bytes.  (Hungarian page, sections "A fused MoE ..." and "FP8 esetén ...":
 * expert computation, FP8 scaling and aggregation of the experts' results.) */
MOE_API int moe_expert_ffn(const moe_desc* desc, const void* x, const void* w13,
                           const void* w2, int top_k, const moe_scales* scales,
                           const float* topk_w, const int32_t* sorted_ids,
                           const int32_t* block_expert, const int32_t* num_padded,
                           void* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Activation quantisation of the W8A8 mode: the step moe_forward and
 * moe_expert_ffn run on x before W13 when desc->act_quant is
 * MOE_ACT_MX_E4M3 (Hungarian page, section "FP8 esetén ...": the FP8
 * scaling of the activations).  From x [T, d] bf16 writes codes [T, d]
 * (e4m3fn bytes) and exps [T, d/32] (E8M0 bytes: block j of row t is scaled
 * by 2^(exps[t, j] - 127)) by the rule stated at MOE_ACT_MX_E4M3; a value
 * is codes * 2^(exps - 127).  desc must be a valid descriptor with
 * act_quant = MOE_ACT_MX_E4M3 (else MOE_ERR_BAD_ARG); its E, I and weight
 * dtype are only validated.  Caller-owned device buffers, asynchronous on
 * `stream`. */
MOE_API int moe_quantize_act(const moe_desc* desc, const void* x, uint8_t* codes,
                             uint8_t* exps, void* stream);

/* A captured forward: moe_forward's launch sequence for one desc and one
 * set of buffers, recorded once into a HIP graph and replayed with a single
 * launch per step.  The pages' fused operation replaces a sequence of
 * separate operations by one batched GPU operation (Hungarian page, section
 * "A fused MoE ..."); at decode sizes the gaps between the layer's kernels
 * are a visible share of a step, and a graph replay submits the whole
 * layer at once.  A decode loop writes the next tokens into the same x and
 * replays.
 *   moe_graph_create: same arguments and checks as moe_forward, plus the
 *     handle out-parameter.  It records, it does not run: nothing is
 *     enqueued on any caller stream.  The graph keeps the addresses given
 *     here (x, w_gate, W13, W2, the scales, out, the workspace): they must
 *     stay allocated, at the same addresses, until moe_graph_destroy.  Each
 *     replay reads what those buffers hold when the stream reaches it.
 *     *graph is NULL on error.  MOE_ERR_HIP if capture or instantiation
 *     fails.  Kernel timing (moe_timing_enable) does not see replays.
 *   moe_graph_launch: enqueue one replay on `stream`; asynchronous.
 *     Replays of one graph share its workspace: replays on different
 *     streams must be ordered by the caller.
 *   moe_graph_destroy: release the graph (NULL is accepted); the stream
 *     work already enqueued completes normally. */
typedef struct moe_graph moe_graph;
MOE_API int moe_graph_create(const moe_desc* desc, const void* x, const float* w_gate,
                             const void* w13, const void* w2, int top_k,
                             const moe_scales* scales, void* out, void* workspace,
                             size_t workspace_bytes, moe_graph** graph);
MOE_API int moe_graph_launch(moe_graph* graph, void* stream);
MOE_API int moe_graph_destroy(moe_graph* graph);

/* ---- diagnostics ---- */

/* Static text for a status code (never NULL). */

MOE_API const char* moe_strerror(int status);

/* Kernel timing.  Kernels of the kinds set in the mask given to
 * moe_timing_enable (bit MOE_KERNEL_x) are each bracketed by two HIP events
 * recorded on the stream they are launched on (a small cost per launch);
 * moe_timing_collect waits for the recorded events and adds their durations
 * into per-kind totals.  Mask 0 (the initial state) times nothing.  Kernel
 * kinds index the arrays. */
#define MOE_KERNEL_ROUTE_LOGITS 0
#define MOE_KERNEL_ROUTE_TOPK 1
#define MOE_KERNEL_ALIGN 2
#define MOE_KERNEL_FFN13 3
#define MOE_KERNEL_FFN2 4
#define MOE_KERNEL_COMBINE 5
#define MOE_KERNEL_QUANT_X 6  /* W8A8 mode: x to block-scaled e4m3fn */
#define MOE_KERNEL_FFN_FUSED 7  /* decode: W13, W2 and combine in one launch */
#define MOE_KERNEL_COUNT 8

MOE_API int moe_timing_enable(int kind_mask);  /* MOE_ERR_BAD_ARG if out of range */
#define MOE_TIMING_ALL ((1 << MOE_KERNEL_COUNT) - 1)
/* total_ms[MOE_KERNEL_COUNT], launches[MOE_KERNEL_COUNT]; reset != 0 clears
 * the totals after reading.  Blocks until the recorded events complete. */
MOE_API int moe_timing_collect(double* total_ms, int64_t* launches, int reset);
/* Name of a kernel kind ("ffn13", ...), or "" if out of range. */
MOE_API const char* moe_kernel_name(int kind);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
