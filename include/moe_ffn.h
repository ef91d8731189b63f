/*
 * moe_ffn.h - C ABI of the MI355X (gfx950) routed-expert MoE FFN layer.
 *
 * One Qwen3-MoE decoder layer's routed-expert FFN: for every token a router
 * matvec, a softmax over all experts, top-k selection and renormalisation of
 * the k weights, then each chosen expert's SwiGLU FFN on Q4_K weights, and the
 * router-weighted sum of the expert outputs.
 *
 * Passages that define the operation (docs.rs source pages of the
 * aprender-serve crate):
 *   - forward_qwen3_moe.rs, step 2h of the single-token forward (MoE FFN): the
 *     layer maps one position to a hidden_dim vector; each chosen expert runs a
 *     SwiGLU of its gate and up projections and a down projection, and the
 *     expert results are summed with the softmax-then-renormalised top-k
 *     router weights. The module doc: each chosen expert's matvecs dequantise
 *     its Q4_K bytes in flight.
 *   - forward_qwen3_moe.rs, step 2g of the full-sequence forward: positions are
 *     sent through the layer one by one (tokens are independent).
 *   - forward_qwen3_moe_cuda_traced.rs, doc of ..._traced_with_plan: the
 *     MoeRouter stage is a token's k post-softmax, renormalised router weights
 *     and MoeFfnOut its hidden_dim output; moe_ffn_forward mirrors both with
 *     router_out and out.
 *   - qwen3_moe_dispatch.rs, qwen3_moe_shape: the layer shape is the triple
 *     expert count, experts used per token and expert FFN width (read from
 *     model metadata), plus the model's hidden size.
 *   - forward_qwen3_moe.rs / forward_qwen3_moe_cuda_traced.rs argument checks:
 *     an empty token list, a zero expert count, zero experts per token, a zero
 *     expert width, and more experts per token than experts are shape errors.
 *
 * Conventions
 *   - Every data pointer is a DEVICE pointer (memory from hipMalloc, e.g. a
 *     torch tensor on the GPU) unless marked "host". Host memory passed where
 *     device memory is required is rejected with MOE_ERR_INVALID_ARG.
 *   - stream is a hipStream_t (NULL = the legacy default stream).
 *   - All calls are C ABI, return moe_status, and on failure record a reason
 *     readable with moe_ffn_last_error() (per calling thread).
 *   - Arguments are validated on the host before anything is enqueued; a call
 *     that fails validation enqueues nothing and changes nothing.
 *   - A handle may be used by one host thread and one stream at a time.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: adds moe_ffn_set_norm, moe_ffn_forward_block, moe_ffn_debug_stats and moe_ffn_forward_q8.
 * 3: adds moe_ffn_forward_noalloc. */
#define MOE_FFN_ABI_VERSION 3

typedef struct moe_ffn_s *moe_ffn_t;

/* Layer shape. hidden_dim and moe_intermediate must be multiples of 256 (Q4_K
 * super-blocks run along the reduction dimension of every matrix);
 * 1 <= num_experts_per_tok <= num_experts <= 1024 and num_experts_per_tok <= 64. */
typedef struct moe_ffn_shape {
    int32_t hidden_dim;          /* H */
    int32_t num_experts;         /* E */
    int32_t num_experts_per_tok; /* k */
    int32_t moe_intermediate;    /* I */
} moe_ffn_shape;

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_SHAPE = 1, /* shape or token count outside the rules above */
    MOE_ERR_INVALID_ARG = 2,   /* null / host / aliased pointer, bad handle     */
    MOE_ERR_BLOB_SIZE = 3,     /* a byte count differs from the shape's         */
    MOE_ERR_DEVICE = 4,        /* a HIP call or kernel launch failed            */
    MOE_ERR_OOM = 5            /* device allocation failed                      */
} moe_status;

/* Build a layer from its weights.
 *   shape       host pointer to the layer shape.
 *   gate_q4k    [E][I][H/256] Q4_K blocks of 144 bytes (expert-major, row-major,
 *               blocks along H), gate_bytes = E*I*(H/256)*144.
 *   up_q4k      same layout and size as gate.
 *   down_q4k    [E][H][I/256] blocks, down_bytes = E*H*(I/256)*144.
 *               Block format: public GGUF Q4_K (fp16 d, fp16 dmin, 12 bytes of
 *               6-bit sub-block scales and mins, 128 bytes of 4-bit quants).
 *   router_w    [E][H] fp32, row e scores expert e.
 *   router_bias [E] fp32 added to the logits, or NULL for none.
 *   stream      the weights are copied and repacked on this stream; the call
 *               synchronises it before returning, so the caller may free or
 *               reuse all of its buffers afterwards (the handle owns copies).
 *   out         host pointer; receives the handle.
 * Errors: INVALID_SHAPE, BLOB_SIZE, INVALID_ARG (null/host pointers), OOM,
 * DEVICE. */
moe_status moe_ffn_create(const moe_ffn_shape *shape, const void *gate_q4k, size_t gate_bytes,
                          const void *up_q4k, size_t up_bytes, const void *down_q4k, size_t down_bytes,
                          const float *router_w, const float *router_bias, void *stream, moe_ffn_t *out);

/* Pre-size the per-call workspace for up to max_tokens tokens so that later
 * forwards of at most that many tokens allocate nothing. Synchronises stream.
 * Errors: INVALID_ARG (bad handle), INVALID_SHAPE (max_tokens < 1), OOM. */
moe_status moe_ffn_reserve(moe_ffn_t h, int32_t max_tokens, void *stream);

/* The layer on T tokens (the MoE FFN step of the pages, generalised from one
 * position per call to T).
 *   x          [T][H] fp32 activations (input of the pre-FFN norm's output).
 *   out        [T][H] fp32, the router-weighted sum of the chosen experts'
 *              SwiGLU FFN outputs (MoeFfnOut per token). Must not overlap x.
 *   router_out [T][k] fp32 renormalised router weights, largest logit first
 *              (MoeRouter per token), or NULL.
 *   router_idx [T][k] int32 chosen experts in the same order, or NULL.
 * Expert choice: the k largest logits; equal logits go to the lower expert
 * index. Results are bitwise reproducible from call to call (no floating-point
 * atomics; every sum has a fixed order).
 * Paths: T <= 4 with num_experts <= 256, hidden_dim <= 4096 and
 * num_experts_per_tok * moe_intermediate / 256 <= 384 take the decode path
 * (three launches: router, gate/up per pair, down and combine); other calls
 * the bucketed path (router, top-k, bucketing, grouped GEMMs, combine).
 * Asynchronous on stream: nothing waits on the host, except that a T above
 * the reserved capacity first grows the workspace (a device synchronisation).
 * Non-finite inputs give unspecified routing and outputs.
 * Errors: INVALID_SHAPE (T < 1, or T so large that T*4*hidden_dim or
 * T*k*4*moe_intermediate reaches 2^32), INVALID_ARG (null/host pointers, out
 * overlapping x, bad handle), OOM, DEVICE. */
moe_status moe_ffn_forward(moe_ffn_t h, int32_t T, const float *x, float *out, float *router_out,
                           int32_t *router_idx, void *stream);

/* moe_ffn_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, outputs, results (bit for bit) and errors as
 * moe_ffn_forward, but the per-call workspace is a fixed scratch array of 64
 * MiB that the library holds on each device from its load until the process
 * ends, instead of the handle's own workspace: the call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine) and never grows
 * anything. Its limit is the token count whose workspace fits 64 MiB (about
 * 490 tokens at hidden 2048, 128 experts, top-8, intermediate 768); a larger
 * T returns INVALID_SHAPE naming the limit, before anything is enqueued. Every
 * call on one device shares that device's scratch and leaves its contents
 * there: calls that overlap on one device (several streams, or several host
 * threads, whatever the handle) race, so the caller orders them, e.g. on one
 * stream. moe_ffn_debug_routing and moe_ffn_debug_stats after this call read
 * the shared scratch, valid until the next no-alloc call on the device. The
 * current device must be the handle's (else INVALID_ARG). */
moe_status moe_ffn_forward_noalloc(moe_ffn_t h, int32_t T, const float *x, float *out, float *router_out,
                                   int32_t *router_idx, void *stream);

/* The layer with Q8_K-style int8 activations for the routed experts (the
 * activation format of the production CPU path in qwen3_moe_dispatch.rs, doc
 * of cpu_reference, whose logits differ measurably from the fp32-activation
 * forward's): each token's x row and each expert's h
 * enter the expert matvecs as codes q and a scale d per 256 values, amax =
 * max |v|, q = rint(v * (127 / amax)) in [-127, 127], d = amax / 127, all in
 * fp32; the router runs on the fp32 x. Arguments, outputs, token counts and
 * errors as moe_ffn_forward (the same paths: the decode path and the
 * bucketed grouped GEMMs, there in one MFMA pass on the codes, each output in
 * units of the row's d per super-block). Non-finite inputs give unspecified
 * outputs. */
moe_status moe_ffn_forward_q8(moe_ffn_t h, int32_t T, const float *x, float *out, float *router_out,
                              int32_t *router_idx, void *stream);

/* Set the pre-FFN norm of the block around the layer: the RMSNorm weight and
 * eps that moe_ffn_forward_block applies (forward_qwen3_moe.rs, prefill step
 * 2f and decode step 2g, "Pre-FFN norm": the residual stream is normalised
 * with the layer's ffn norm weight and the model's eps before the MoE layer).
 *   norm_w  [H] fp32, host or device pointer; copied (the caller keeps it).
 *   eps     finite, >= 0 (Qwen3-MoE models use 1e-6).
 * Synchronises stream. May be called again to replace the weight.
 * Errors: INVALID_ARG (bad handle, NULL norm_w, eps negative or not finite),
 * OOM, DEVICE. */
moe_status moe_ffn_set_norm(moe_ffn_t h, const float *norm_w, float eps, void *stream);

/* The layer inside its block on T tokens of the residual stream:
 *   out[t] = hidden[t] + layer(rms_norm(hidden[t]))
 * with rms_norm(x)[i] = x[i] * norm_w[i] / sqrt(mean_c x[c]^2 + eps) (the
 * standard RMSNorm; the pages name the op without its formula), rounded to
 * fp32 as the layer's input, and the residual add of the block after the MoE
 * FFN (forward_qwen3_moe.rs: the "Residual" step after prefill step 2g,
 * decode step 2i). On the decode path (see moe_ffn_forward) the norm is
 * fused into the router launch; on the bucketed path with T > 4 into the
 * router and top-k launches when num_experts <= 256 and hidden_dim <= 4096;
 * otherwise it is a launch of its own ahead of the layer. The residual add
 * happens in the kernel that writes out.
 *   hidden      [T][H] fp32 residual stream.
 *   out         [T][H] fp32 block output. Must not overlap hidden.
 *   router_out, router_idx, stream: as for moe_ffn_forward (routing of the
 *               normalised rows).
 * Errors: as moe_ffn_forward, and INVALID_ARG if moe_ffn_set_norm has not been
 * called on this handle. */
moe_status moe_ffn_forward_block(moe_ffn_t h, int32_t T, const float *hidden, float *out, float *router_out,
                                 int32_t *router_idx, void *stream);

/* Copy the routing state of the most recent forward on this handle (for tests):
 *   logits  [T][E] fp64 router logits (bias included), or NULL;
 *   counts  [E] int32 tokens per expert, or NULL;
 *   offsets [E+1] int32 exclusive prefix sum of counts, or NULL;
 *   entries [T*k] int32, entries[offsets[e] + r] = t*k + j for the r-th
 *           (token, slot) pair, in token order, that chose expert e; or NULL.
 * T is the token count of that forward. Enqueued on stream after it.
 * Errors: INVALID_ARG (bad handle, host pointers, no forward yet). */
moe_status moe_ffn_debug_routing(moe_ffn_t h, double *logits, int32_t *counts, int32_t *offsets,
                                 int32_t *entries, void *stream);

/* Per-stage statistics of one token of the most recent forward on this handle
 * (moe_ffn_forward or moe_ffn_forward_block): the traced forward's summary
 * (forward_qwen3_moe_cuda_traced.rs, doc of forward_qwen3_moe_cuda_traced:
 * per-layer activation statistics of the last token, with its MoeRouter and
 * MoeFfnOut stages, used to find the first stage where a NaN or Inf enters).
 *   token       0 <= token < T of that forward (the pages' traced path takes
 *               the last).
 *   out         the [T][H] output buffer that forward wrote.
 *   router_out  the router_out that forward was given (NULL if it was NULL).
 *   stats       [4][7] fp64 device array. Stages: 0 router logits (E values,
 *               bias included), 1 router weights (k, MoeRouter), 2 SwiGLU
 *               output h of the token's k slots (k * moe_intermediate values,
 *               slot order), 3 the output row (hidden_dim values: MoeFfnOut,
 *               or the block output). Fields: number of values, NaN count,
 *               +-Inf count, then over the finite values min, max, mean and
 *               root mean square (each 0 when no value is finite). The page
 *               names the statistics type without its fields; these are the
 *               reading taken.
 * Enqueued on stream after the forward; reads the workspace, so no other
 * forward may run on the handle in between.
 * Errors: INVALID_ARG (bad handle, no forward yet, token out of range, host
 * pointers), DEVICE. */
moe_status moe_ffn_debug_stats(moe_ffn_t h, int32_t token, const float *out, const float *router_out,
                               double *stats, void *stream);

/* Per-stage GPU timing for benchmarks. Stages of one forward, in launch order:
 * 0 router (logits, and for at most 4 tokens also the top-k), 1 topk (which
 * also stages x when num_experts <= 256), 2 bucket (the per-chunk expert
 * histogram; 13 bucket_scatter places the pairs), 3 stage_x (when the top-k
 * launch does not stage x), 4 gate_up (16-row tiles of buckets of at most 16 entries, or the
 * per-pair decode kernel), 5 gate_up_big (tiles of up to 64 rows for larger
 * buckets), 6 stage_h, 7 down (16-row tiles, or the fused decode down +
 * combine), 8 down_big, 9 combine, 10 gate_up_tail and 11 down_tail (the
 * 64-row GEMMs' last-round tiles as half-width units), 12 norm (the RMSNorm of
 * moe_ffn_forward_block, where it is a launch of its own), 13 bucket_scatter;
 * a stage a forward does not run has no
 * launches (moe_ffn_stage_name gives the name, moe_ffn_stage_count the number).
 * moe_ffn_profile sets a bit mask of stages; while it is non-zero, each forward
 * records a HIP event on its stream right before and right after every
 * selected stage's kernel. moe_ffn_profile_read waits for those events, adds
 * stage s's elapsed milliseconds to ms[s] and its launch count to launches[s]
 * (host arrays of moe_ffn_stage_count() entries), and forgets them.
 * Errors: INVALID_ARG (bad handle, NULL arrays), DEVICE. */
moe_status moe_ffn_profile(moe_ffn_t h, uint32_t stage_mask);
moe_status moe_ffn_profile_read(moe_ffn_t h, double *ms, int32_t *launches);
int32_t moe_ffn_stage_count(void);
const char *moe_ffn_stage_name(int32_t stage); /* NULL outside 0..count-1 */

/* Release the handle and all device memory it owns. Synchronises the device
 * first. NULL is accepted and ignored. */
moe_status moe_ffn_destroy(moe_ffn_t h);

/* Reason for the calling thread's most recent failure ("" if none). The
 * string stays valid until that thread's next call into this library. */
const char *moe_ffn_last_error(void);

/* MOE_FFN_ABI_VERSION of the built library. */
int32_t moe_ffn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
