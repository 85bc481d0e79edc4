/*
 * moe_route.h -- C ABI of the MI355X (gfx950) fused MoE top-k routing library.
 *
 * Operations, each one asynchronous launch sequence on the caller's HIP
 * stream:
 *
 *   moe_route            router logits [T, E] -> top-k ids and weights
 *                        (+ optional full-E scores and per-expert counts)
 *   moe_route_permute    moe_route + the tile-padded dispatch bookkeeping
 *   moe_aux_loss         load-balancing loss, forward and/or backward
 *   rmsnorm_gate_route   RMSNorm -> router projection (MFMA) -> top-k on the
 *                        raw logits -> activation of the chosen experts
 *   moe_route_backward   gradient of the weights / scores w.r.t. the logits
 *   moe_topk_to_dense    dense [T, E] probs and routing map from the top-k
 *   moe_dispatch         token rows into permuted (expert) order
 *   moe_combine          weighted expert rows back into token order
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * Pointers: every data pointer is a DEVICE pointer, allocated and owned by the
 *   caller.  The library never allocates, frees, synchronises, or copies device
 *   memory to the host.  Scratch memory comes from the caller's `workspace`
 *   (device memory, 256-byte aligned, at least the size the matching
 *   *_workspace_size() helper returns).  The ROUTING workspace (moe_route
 *   with expert_counts, moe_route_permute) starts with a counting region (the
 *   first moe_route_count_region_bytes() bytes), the FRONT-END workspace
 *   (rmsnorm_gate_route) with a synchronisation region (the first
 *   rmsnorm_gate_route_sync_region_bytes() bytes), and the AUX-LOSS workspace
 *   (moe_aux_loss with loss) with one of moe_aux_loss_sync_region_bytes()
 *   bytes; the rest of every workspace is ignored on entry.  That region must be
 *   zero-filled before the workspace's first use; every call leaves it
 *   zero-filled again when its work completes (apart from the front end's
 *   failure count, see rmsnorm_gate_route), so one workspace serves any
 *   sequence of calls of any sizes on one stream.  After an MOE_EHIP failure
 *   mid-call, zero it again.  A region that is not clean never moves an access
 *   outside the workspace and the caller's arrays; what it does to the results
 *   is stated at each entry point (routing: see moe_route_permute).  All
 *   arrays are dense and row-major.
 * Streams: all work is enqueued on `stream` (0 = the null stream); outputs are
 *   valid once that work completes.  Calls on different streams that share a
 *   workspace race.  Calls are otherwise re-entrant and thread-safe.
 * Errors: arguments are validated on the host before anything is enqueued; on
 *   any error nothing is written and nothing is launched.  MOE_EINVAL: a size,
 *   flag or pointer is invalid; MOE_EUNSUPPORTED: valid per the method but
 *   outside what the kernels implement (the message names the limit);
 *   MOE_EWORKSPACE: workspace too small; MOE_EHIP: a HIP launch failed
 *   (moe_last_hip_error() returns the hipError_t).  No exception crosses the
 *   ABI.  moe_status_string() and moe_last_error_message() describe a status.
 * Outputs: every output element a call owns is written by the device,
 *   including -1 padding; nothing is left for the caller to pre-fill.
 *
 * Method sources (page title, section):
 *   [TE]   Implementation:NVIDIA TransformerEngine Fused Router -- Description,
 *          Code Reference / Signature, I/O Contract.
 *   [FI]   flashinfer.fused_moe.trtllm_gen_routing -- Parameters, Returns, Notes.
 *   [NKI]  RMSNorm Router Top-K A2AV Kernel API Reference -- Background,
 *          Parameters, Returns, Notes.
 *   [LMD]  Implementation:InternLM Lmdeploy Gemm MoeUtils -- Description,
 *          Code Reference / Signature, I/O Contract.
 *   [MAX]  max.nn.moe.SigmoidTopKRouter -- routing steps 1-4, Parameters.
 */
#ifndef MOE_ROUTE_H_
#define MOE_ROUTE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EWORKSPACE = 3,
  MOE_EHIP = 4
} moe_status;

/* Element types.  F16 is accepted by rmsnorm_gate_route only ([NKI] Parameters
 * allow bf16/fp16 hidden states). */
typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype;

/* Score function: [TE] I/O Contract (score_function "softmax" or "sigmoid");
 * [NKI] Parameters (router_act_fn SOFTMAX or SIGMOID). */
typedef enum moe_score_fn { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score_fn;

/* The routing method of one call.  Field names follow [TE] and [FI].
 *
 * num_tokens        T >= 0 (T = 0 is valid: counts are zeroed, nothing else
 *                   is written).
 * num_experts       E, 1 <= E <= 2048.
 * top_k             k, 1 <= k <= min(E, 64); with grouping also
 *                   k <= topk_group * E / n_group.
 * score_fn          moe_score_fn.
 * use_pre_softmax   softmax only: 1 = softmax over all E experts, then top-k;
 *                   0 = top-k on the logits, then softmax over the k chosen
 *                   ([TE] Description: pre- and post-softmax ordering).
 *                   Ignored for sigmoid.
 * n_group, topk_group
 *                   group-limited routing ([FI] Parameters: n_group /
 *                   topk_group, 0 disables; [TE] num_groups / group_topk):
 *                   the E experts form n_group contiguous groups of E/n_group;
 *                   only the topk_group best groups stay eligible.  Grouping
 *                   is off when n_group <= 1, topk_group == 0 or
 *                   topk_group == n_group.  E % n_group must be 0.
 * group_score_topn  a group's score is the sum of its group_score_topn largest
 *                   selection keys (2 for DeepSeek-V3-style routing);
 *                   1 <= group_score_topn <= E / n_group when grouping is on.
 *                   Implemented (else MOE_EUNSUPPORTED): group_score_topn
 *                   <= 2, and a group size E / n_group equal to w times a
 *                   power of two for some w in {4, 8, 16, 32} with
 *                   E <= 64 w (a group spans whole kernel lanes of w experts).
 * renormalize       1 = divide the chosen weights by their sum
 *                   ([FI] norm_topk_prob; [MAX] norm_topk_prob; [LMD]
 *                   norm_topk).  No effect for post-softmax, whose weights
 *                   already sum to one.
 * routed_scaling_factor
 *                   multiplies every weight last ([FI], [MAX]; [TE]
 *                   scaling_factor).
 * logits_dtype      MOE_F32 or MOE_BF16 ([FI] Parameters: routing_logits).
 * bias_dtype        MOE_F32 or MOE_BF16; the type of the optional bias.
 * weights_dtype     MOE_F32 (default) or MOE_BF16 ([FI] Notes: bfloat16
 *                   weights).
 *
 * Selection key per expert e of a token with logits x:
 *   sigmoid:       s_e = 1/(1+exp(-x_e)) in float32 ([MAX] step 2),
 *                  key_e = s_e + bias_e ([MAX] step 3).
 *   softmax pre:   p_e = softmax(x)_e, key_e = p_e + bias_e.
 *   softmax post:  key_e = x_e + bias_e.
 * The bias only ever enters the key ([MAX] step 4: weights use the unbiased
 * score).  Top-k takes the k largest keys; equal keys go to the lower expert
 * index; ids are listed by descending key.  Weights: sigmoid s_e, pre-softmax
 * p_e, post-softmax the softmax over the k chosen logits; then renormalised
 * (if asked) and multiplied by routed_scaling_factor. */
typedef struct moe_route_args {
  int32_t num_tokens;
  int32_t num_experts;
  int32_t top_k;
  int32_t score_fn;
  int32_t use_pre_softmax;
  int32_t n_group;
  int32_t topk_group;
  int32_t group_score_topn;
  int32_t renormalize;
  float routed_scaling_factor;
  int32_t logits_dtype;
  int32_t bias_dtype;
  int32_t weights_dtype;
} moe_route_args;

/* Expert selection ([TE] FusedTopkScoreFunction and
 * FusedComputeScoresForMoEAuxLoss; [FI] topk_ids / topk_weights; [MAX] steps
 * 2-4; [LMD] invokeMoeGate_V2 scales).
 *
 * logits         [T, E] of logits_dtype.
 * bias           nullable [E] of bias_dtype: the expert / correction bias.
 * topk_ids       out [T, k] int32.
 * topk_weights   out [T, k] of weights_dtype.
 * scores         nullable out [T, E] float32: full-E scores for the aux loss
 *                (softmax over E; for sigmoid s_e / sum_e s_e).
 * expert_counts  nullable out [E] int32: tokens that chose each expert.
 * workspace      >= moe_route_workspace_size(args, 1, E) bytes when
 *                expert_counts is given, else may be NULL. */
moe_status moe_route(const moe_route_args* args, const void* logits, const void* bias,
                     int32_t* topk_ids, void* topk_weights, float* scores,
                     int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Expert selection plus the permutation a grouped GEMM consumes ([FI]
 * trtllm_gen_routing: Parameters, Returns, Notes; [LMD] per-expert offsets).
 *
 * tile_tokens_dim     power of two, 1 <= tile <= 1024: each expert's segment
 *                     is padded to a multiple of it ([FI] Parameters).
 * local_expert_offset, local_num_experts
 *                     the experts this call permutes: [off, off + E_loc) with
 *                     0 <= off, 1 <= E_loc, off + E_loc <= E ([FI] Parameters).
 *                     Ids outside that range are still returned in topk_ids
 *                     but map to -1 in expanded_idx_to_permuted_idx.
 * expert_counts       out [E_loc] int32: tokens per local expert.
 * padded_offsets      out [E_loc + 1] int32: exclusive prefix sums of the
 *                     tile-padded counts; segment e is
 *                     [padded_offsets[e], padded_offsets[e + 1]).
 * total_num_padded_tokens  out [1] int32 = padded_offsets[E_loc].
 * num_non_exiting_ctas     out [1] int32 = total / tile (the number of tiles).
 * expanded_idx_to_permuted_idx  out [T * k] int32: for the j-th id of token t
 *                     (expanded index t * k + j) its slot in permuted space,
 *                     or -1 for a non-local expert.  Inside a segment tokens
 *                     are in ascending order.
 * permuted_idx_to_token_idx  out [moe_max_padded_tokens(T, k, E_loc, tile)]
 *                     int32: the token in each slot, -1 for padding slots.
 *                     Slots at or beyond total are not written.
 * cta_idx_xy_to_batch_idx  out [moe_max_tiles(...)] int32: the local expert of
 *                     each tile; slot p's expert is
 *                     cta_idx_xy_to_batch_idx[p / tile] + local_expert_offset
 *                     ([FI] Notes).  Entries at or beyond the tile count are
 *                     not written.
 * cta_idx_xy_to_mn_limit   out [moe_max_tiles(...)] int32: exclusive end of the
 *                     tile's valid rows in permuted space,
 *                     min((c + 1) * tile, segment start + count).
 * workspace           >= moe_route_workspace_size(args, tile, E_loc) bytes.
 * The other arguments are as for moe_route (scores nullable).
 *
 * A counting region that is not clean on entry (never zeroed, or left by an
 * MOE_EHIP mid-call) leaves topk_ids / topk_weights / scores exact and moves
 * no write outside the output arrays.  The bookkeeping detects it when the
 * region's header is out of range, a count falls outside [0, T k] or the
 * padded offsets overflow: then total_num_padded_tokens,
 * num_non_exiting_ctas and every expert_counts entry are -1, the other
 * bookkeeping outputs are not valid, and the region is clean again for the
 * next call.  Garbage that looks like counts (small non-negative values
 * under a valid header) goes undetected: the bookkeeping of a call whose
 * counting rows hold it is off by it (still in bounds), and the call after
 * that call clears those rows.  moe_route with
 * expert_counts reports a detected dirty region as -1 in every count (a
 * count outside [0, T k] as -1 in that count) and leaves the region clean. */
moe_status moe_route_permute(const moe_route_args* args, int32_t tile_tokens_dim,
                             int32_t local_expert_offset, int32_t local_num_experts,
                             const void* logits, const void* bias, int32_t* topk_ids,
                             void* topk_weights, float* scores, int32_t* expert_counts,
                             int32_t* padded_offsets, int32_t* total_num_padded_tokens,
                             int32_t* num_non_exiting_ctas,
                             int32_t* expanded_idx_to_permuted_idx,
                             int32_t* permuted_idx_to_token_idx,
                             int32_t* cta_idx_xy_to_batch_idx,
                             int32_t* cta_idx_xy_to_mn_limit, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* moe_route_permute without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, outputs and results are those of
 * moe_route_permute; the scratch (counting region and per-block counts) is a
 * library-owned device array of moe_route_permute_noalloc_max_scratch_bytes()
 * bytes (8 MiB), one per device, held until the process ends.  A call whose
 * moe_route_workspace_size() exceeds it (more than about 1.96 million pairs
 * of a 64-token block and a local expert: T = 262144 with 256 local experts
 * fits, twice that does not) fails with MOE_EUNSUPPORTED before anything is
 * enqueued.  The call allocates nothing: no hipMalloc, no host or
 * device allocation of any kind.  The first call on a device (and the first
 * after a call on it returned MOE_EHIP) enqueues a zero-fill kernel of the
 * counting region ahead of its work; every completed call leaves that region
 * zero.  All calls on one device share the array: calls that overlap on one
 * device (different streams, or different host threads) race and must be
 * ordered by the caller. */
moe_status moe_route_permute_noalloc(const moe_route_args* args, int32_t tile_tokens_dim,
                                     int32_t local_expert_offset, int32_t local_num_experts,
                                     const void* logits, const void* bias, int32_t* topk_ids,
                                     void* topk_weights, float* scores, int32_t* expert_counts,
                                     int32_t* padded_offsets, int32_t* total_num_padded_tokens,
                                     int32_t* num_non_exiting_ctas,
                                     int32_t* expanded_idx_to_permuted_idx,
                                     int32_t* permuted_idx_to_token_idx,
                                     int32_t* cta_idx_xy_to_batch_idx,
                                     int32_t* cta_idx_xy_to_mn_limit, hipStream_t stream);
size_t moe_route_permute_noalloc_max_scratch_bytes(void);

/* Load-balancing aux loss ([TE] FusedAuxLoss, forward and backward, with the
 * arguments of fused_moe_aux_loss):
 *
 *   loss = coeff * E / (top_k * total_num_tokens^2)
 *          * sum_e (sum_t probs[t, e]) * tokens_per_expert[e]
 *   grad_probs[t, e] = grad_loss * coeff * E / (top_k * total_num_tokens^2)
 *                      * tokens_per_expert[e]
 *
 * probs              [rows, E] float32 (nullable when only the backward runs).
 * tokens_per_expert  [E] int32, >= 0.
 * rows               rows of probs held here, >= 0; total_num_tokens >= 1 is
 *                    the global token count (probs may be a shard of it).
 * loss               nullable out [1] float32: runs the forward.
 * grad_loss          nullable [1] float32 device scalar; NULL means 1.
 * grad_probs         nullable out [rows, E] float32: runs the backward.
 * At least one of loss / grad_probs must be given.
 * workspace          >= moe_aux_loss_workspace_size(rows, E) bytes, used by the
 *                    forward only (NULL is fine for a backward-only call); its
 *                    first moe_aux_loss_sync_region_bytes() bytes (the whole
 *                    of it) are zero on entry and again when the call's work
 *                    completes (see the conventions above).
 * The forward is one launch and deterministic: the same inputs give the same
 * bits on every call.  Its blocks hand their partial sums to the last block
 * through the workspace; that block's wait is bounded, and one that runs out
 * (no block that was dispatched before it finished within seconds: not seen
 * in practice) writes *loss as the float32 NaN with bits 0x7FC0A0A0 and leaves
 * the workspace dirty: zero it again before the next forward.  (The
 * environment variable MOE_ROUTE_AUX_SPIN_LIMIT, an integer no larger than the
 * default, lowers the limit on each call; 0 forces the give-up, for tests.)  A dirty slot
 * (non-zero on entry) is taken for a published partial: the forward that
 * reads it gives a wrong loss.  Its summing block then need not wait for the
 * other blocks, so a block that publishes after that block has cleared the
 * slots leaves its slot set: zero the region again after a forward that ran
 * on a dirty region.  No access leaves the region either way. */
moe_status moe_aux_loss(const float* probs, const int32_t* tokens_per_expert, int64_t rows,
                        int64_t total_num_tokens, int32_t num_experts, int32_t top_k,
                        float coeff, float* loss, const float* grad_loss, float* grad_probs,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward of moe_route's outputs with respect to the logits ([TE]
 * Description: fused_topk_with_score_function and
 * fused_compute_score_for_moe_aux_loss each have a backward).  The pages
 * print no formula; this is the derivative of the forward with the chosen
 * experts held fixed (the top-k choice passes no gradient; the bias, which
 * only enters the choice, receives none):
 *
 *   grad_logits = d/dlogits ( sum_j grad_weights[t, j] * topk_weights[t, j]
 *                             + sum_e grad_scores[t, e] * scores[t, e] )
 *
 * through the score function of args (sigmoid; softmax before or after top-k),
 * the renormalisation (args->renormalize) and args->routed_scaling_factor.
 *
 * args           the forward's arguments: num_tokens, num_experts (<= 2048),
 *                top_k, score_fn, use_pre_softmax, renormalize,
 *                routed_scaling_factor, logits_dtype are used; the grouping
 *                and bias fields are not (the choice is given by topk_ids).
 * logits         [T, E], logits_dtype (the forward's input).
 * topk_ids       [T, k] int32, the forward's ids (required with grad_weights);
 *                ids outside [0, E) contribute nothing; a token's ids are
 *                expected to be distinct, as moe_route writes them.
 * grad_weights   nullable [T, k] float32, the gradient of topk_weights.
 * grad_scores    nullable [T, E] float32, the gradient of the full-E scores.
 * grad_logits    out [T, E] float32, every element written.
 * At least one of grad_weights / grad_scores must be given.  No workspace. */
moe_status moe_route_backward(const moe_route_args* args, const void* logits,
                              const int32_t* topk_ids, const float* grad_weights,
                              const float* grad_scores, float* grad_logits, hipStream_t stream);

/* Dense form of moe_route's top-k outputs ([TE] I/O Contract: the probs and
 * routing_map outputs of fused_topk_with_score_function, each [T, E]):
 *
 *   probs[t, e]       = topk_weights[t, j] where topk_ids[t, j] == e, else 0
 *   routing_map[t, e] = 1 where token t chose expert e, else 0
 *
 * Values are copied, not recomputed (bf16 weights are widened exactly).
 * topk_ids [T, k] int32 (ids outside [0, E) are ignored), topk_weights [T, k]
 * in weights_dtype (MOE_F32 or MOE_BF16); probs: nullable out [T, E] float32;
 * routing_map: nullable out [T, E] uint8 (bool); at least one is given.
 * E <= 2048, k in [1, 64].  No workspace. */
moe_status moe_topk_to_dense(int32_t T, int32_t E, int32_t top_k, const int32_t* topk_ids,
                             const void* topk_weights, int32_t weights_dtype, float* probs,
                             uint8_t* routing_map, hipStream_t stream);

/* Token dispatch and combine either side of the grouped expert GEMM ([LMD]
 * Description: dispatch sends tokens to expert buffers by the routing
 * decision, combine returns expert outputs to token order with the routing
 * scales).  The pages give names and signatures only; the plainest reading in
 * moe_route_permute's own maps ([FI] Returns):
 *
 *   moe_dispatch:  permuted_hidden[p, :] = hidden[permuted_idx_to_token_idx[p], :]
 *                  for p < *total_num_padded_tokens (a bit copy), a zero row
 *                  where the slot is padding (-1); rows past the total are not
 *                  written.
 *   moe_combine:   out[t, :] = sum_j topk_weights[t, j]
 *                              * expert_out[expanded_idx_to_permuted_idx[t*k + j], :]
 *                  summed in choice order in float32 and rounded once to dtype
 *                  (bfloat16: nearest even); a choice whose index is -1 (an
 *                  expert outside the local range) adds nothing.
 *
 * dtype            MOE_F32 or MOE_BF16 for hidden / permuted_hidden /
 *                  expert_out / out; topk_weights are weights_dtype (MOE_F32 or
 *                  MOE_BF16), as moe_route_permute wrote them.
 * T, H             tokens and hidden size (H >= 1); top_k in [1, 64].
 * permuted_idx_to_token_idx, total_num_padded_tokens: device outputs of
 *                  moe_route_permute; max_padded_tokens = the rows of
 *                  permuted_hidden (moe_max_padded_tokens()).
 * No workspace.  Rows move with 16-byte accesses when rows and pointers are
 * 16-byte aligned, element by element otherwise. */
moe_status moe_dispatch(const void* hidden, int32_t dtype, int32_t T, int32_t H,
                        const int32_t* permuted_idx_to_token_idx,
                        const int32_t* total_num_padded_tokens, int64_t max_padded_tokens,
                        void* permuted_hidden, hipStream_t stream);
moe_status moe_combine(const void* expert_out, int32_t dtype, int32_t T, int32_t H, int32_t top_k,
                       const int32_t* expanded_idx_to_permuted_idx, const void* topk_weights,
                       int32_t weights_dtype, void* out, hipStream_t stream);

/* Fused decode front end ([NKI] rmsnorm_router_topk_a2av: Background,
 * Parameters, Returns, Notes):
 *
 *   r_t        = (mean_h hidden[t,h]^2 + eps)^(-1/2)           (float32)
 *   normed     = round_to_dtype((hidden * gamma) * r_t)        out [T, H]
 *   z          = normed @ router_weights (+ router_bias)       (MFMA, float32
 *                accumulation; consumes exactly the stored normed values)
 *   topk_ids   = the k largest z per token, lower index on ties   out [T, k]
 *   affinities = act(z) on the chosen experts, 0 elsewhere     out [T, E] bf16
 *                (sigmoid: sigma(z_e); softmax: softmax over the k chosen z)
 *
 * dtype        MOE_BF16 or MOE_F16 for hidden, gamma, router_weights,
 *              router_bias and normed.
 * T            1 <= T <= 128 ([NKI] Notes); H % 128 == 0 ([NKI] Notes),
 *              128 <= H <= 16384; 1 <= E <= 512 with E % 16 == 0;
 *              1 <= top_k <= min(E, 64).
 * router_bias  nullable [E].
 * workspace    >= rmsnorm_gate_route_workspace_size(T, H, E) bytes, starting
 *              with the zero-filled synchronisation region (conventions above).
 *
 * Two launches: normalisation and projection in one, whose projection blocks
 * wait in-kernel (polling the synchronisation region) for the normalisation
 * scale of their tokens; then the selection.  Should a wait ever exceed its
 * spin limit (it cannot while blocks are dispatched in index order), the call
 * still completes, writes -1 into every topk_ids entry and adds one to the
 * uint32 failure count at byte offset 4 of the workspace, which the library
 * never clears (read it with a device-to-host copy when -1 ids need an
 * explanation; a caller may reset it); the region is clean again for the next
 * call.  A region that was not zero on entry: a dirty failure word (byte
 * offset 0) makes that call report a give-up (-1 ids, counted) and is cleared;
 * the word is never cleared before the projection has run, so that a real
 * give-up cannot be lost.  A dirty normalisation-scale slot of a token t < T
 * gives that call wrong ids and affinities, and the call returns the slot to
 * zero.  (The environment variable MOE_ROUTE_FRONT_END_SPIN_LIMIT,
 * an integer no larger than the default, lowers the limit on each call; 0
 * forces the give-up, for tests.) */
moe_status rmsnorm_gate_route(const void* hidden, const void* gamma, const void* router_weights,
                              const void* router_bias, int32_t dtype, int32_t T, int32_t H,
                              int32_t E, float eps, int32_t top_k, int32_t act_fn, void* normed,
                              int32_t* topk_ids, void* affinities, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Workspace sizes in bytes (0 = none needed).  Pure host functions.
 * moe_route_workspace_size() covers both routing entry points; its first
 * moe_route_count_region_bytes() bytes are the counting region described in
 * the conventions above; rmsnorm_gate_route_sync_region_bytes() and
 * moe_aux_loss_sync_region_bytes() are the synchronisation regions of the
 * front end and of the aux-loss forward (all three constants, independent of
 * the sizes). */
size_t moe_route_workspace_size(const moe_route_args* args, int32_t tile_tokens_dim,
                                int32_t local_num_experts);
size_t moe_route_count_region_bytes(void);
size_t moe_aux_loss_workspace_size(int64_t rows, int32_t num_experts);
size_t moe_aux_loss_sync_region_bytes(void);
size_t rmsnorm_gate_route_workspace_size(int32_t T, int32_t H, int32_t E);
size_t rmsnorm_gate_route_sync_region_bytes(void);

/* Depth of the float32 accumulation chain of rmsnorm_gate_route's projection
 * at hidden size H (MFMA steps of one k-chunk + number of chunks + the 32
 * products one MFMA sums + 1): each logit errs by at most depth * 2^-24 *
 * sum_h |normed * W| from the exact product, the bound by which near-tie
 * tokens of the front end are classified.  -1 for an invalid H. */
int32_t rmsnorm_gate_route_sum_depth(int32_t H);

/* Output-size helpers for moe_route_permute ([FI] Returns): an upper bound on
 * total_num_padded_tokens, T*k + E_loc*(tile-1), and on the tile count,
 * that bound / tile.  Return -1 for invalid arguments. */
int64_t moe_max_padded_tokens(int32_t T, int32_t k, int32_t local_num_experts, int32_t tile);
int64_t moe_max_tiles(int32_t T, int32_t k, int32_t local_num_experts, int32_t tile);

/* Profiling aid for benchmarks.  Between moe_profile_begin() and
 * moe_profile_end() every kernel the library launches is timed by two HIP
 * events on the caller's stream (the stream the kernel runs on): a kind that
 * is one kernel is launched through hipExtLaunchKernel, which stamps the
 * events with the kernel's own start and end; a kind of several kernels
 * (AUX_FWD, FRONT_END) is bracketed by event records.  moe_profile_read() waits for the recorded events of one kernel kind and
 * returns their summed elapsed time and launch count since
 * moe_profile_begin().  Kernel kinds: MOE_KERNEL_*.  The profiling state is
 * process-wide (one switch and one set of totals, guarded by a mutex, so the
 * calls are thread-safe; launches from every thread are counted).  Not for
 * use while capturing a HIP graph. */
typedef enum moe_kernel_kind {
  MOE_KERNEL_ROUTE = 0,
  MOE_KERNEL_COUNTS = 1,
  MOE_KERNEL_SCATTER = 2,
  MOE_KERNEL_AUX_FWD = 3,
  MOE_KERNEL_AUX_BWD = 4,
  MOE_KERNEL_FRONT_END = 5,
  MOE_KERNEL_ROUTE_BWD = 6,
  MOE_KERNEL_DISPATCH = 7,
  MOE_KERNEL_COMBINE = 8,
  MOE_KERNEL_DENSE = 9,
  MOE_KERNEL_KINDS = 10
} moe_kernel_kind;
moe_status moe_profile_begin(void);
moe_status moe_profile_end(void);
moe_status moe_profile_read(int32_t kernel_kind, double* total_ms, int64_t* launches);

const char* moe_status_string(moe_status status);
/* Message of the last failed call on this host thread ("" if none). */
const char* moe_last_error_message(void);
/* hipError_t of the last MOE_EHIP on this host thread (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H_ */
