/*
 * moe.h — C ABI of the token-choice Mixture-of-Experts layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (as the "专家组合 (MoE)" lesson of AI Engineering from Scratch
 * states it in its Concept section): a linear router scores every token
 * against E experts, each token picks its k best experts, each chosen expert
 * is an independent SwiGLU FFN, and the layer output is the gate-weighted sum
 * of the chosen experts' outputs, plus the output of shared experts that every
 * token passes through (Shared experts section).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked HOST.  The caller owns and
 *     allocates every buffer, including workspaces (size them with
 *     moe_workspace_size); the library allocates nothing per call and keeps no
 *     pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work and return without synchronising; device-side
 *     faults surface at the caller's next synchronisation.
 *   - Matrices are row-major with the last index contiguous.  Weights use the
 *     nn.Linear layout [out, in].  bf16 tensors are raw 16-bit bf16 values.
 *   - Indices and counts are int32; sizes are int64 where they can pass 2^31.
 *   - Arguments are checked before anything is enqueued: MOE_EINVAL for a
 *     NULL required pointer, a non-positive size or k outside [1, E];
 *     MOE_EWORKSPACE for a NULL workspace or one smaller than
 *     moe_workspace_size asks for; MOE_ENOTSUP for shapes outside the
 *     supported set (stated per call).  A call that fails these checks
 *     enqueues nothing.  MOE_EHIP: a kernel launch (or setting a kernel's
 *     LDS limit) failed; kernels the call enqueued before it may still run.
 *   - Values that must agree between calls (offsets[G] == rows, the expert
 *     indices being in [0, E)) live on the device and are not checked.
 *   - NaN or Inf inputs give undefined expert selection.
 *   - Calls on different streams (or host threads) with disjoint buffers may
 *     run concurrently.  The only global state is a per-device cache (the
 *     compute-unit count, the kernels' LDS limits), filled once per device
 *     under atomics.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int moe_status;
enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,     /* bad argument */
  MOE_ENOTSUP = 2,    /* shape or option outside what the library supports */
  MOE_EWORKSPACE = 3, /* workspace missing or too small */
  MOE_EHIP = 4        /* a HIP runtime call or kernel launch failed */
};

/* storage type of activations and expert weights */
enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

/* Router score function and gate rule.  The AREX article on The Ultimate MoE
 * Training Handbook (router-precision paragraph) names the three score
 * functions; the lesson's Build-it step 1 fixes the softmax-over-chosen gate.
 *   MOE_SOFTMAX_CHOSEN:     score = logit; gates = softmax of the chosen
 *                           experts' raw logits.
 *   MOE_SIGMOID_NORM:       score = 1/(1+e^-logit); gates = chosen scores
 *                           divided by their sum.
 *   MOE_SQRT_SOFTPLUS_NORM: score = sqrt(ln(1+e^logit)); gates as above.
 *   MOE_UNIFORM_GATES:      no learned router (moe_route_hash): gates are the
 *                           constant 1/k; only moe_backward takes it (no
 *                           logit or router-weight gradient exists). */
enum moe_score { MOE_SOFTMAX_CHOSEN = 0, MOE_SIGMOID_NORM = 1, MOE_SQRT_SOFTPLUS_NORM = 2, MOE_UNIFORM_GATES = 3 };

/* which call a workspace is sized for */
enum moe_call { MOE_CALL_ROUTE = 0, MOE_CALL_PERMUTE = 1, MOE_CALL_GROUPED_FFN = 2, MOE_CALL_BACKWARD = 3,
                MOE_CALL_AUX_LOSS = 4, MOE_CALL_BACKWARD_SHARED = 5 };

/* Largest supported expert count and top-k (the handbook article's router
 * table has a model choosing 16 of 896 experts, the largest on the pages). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

/*
 * moe_route — router GEMM, scoring, top-k selection and gates.
 * Lesson "专家组合 (MoE)", Concept (scores = router(x), top-k) and Build it
 * step 1 (bias added for the ranking only; gates from the unbiased values);
 * Load balancing item 3 (the DeepSeek-V3 auxiliary-loss-free bias).
 *
 *   x            [T, d]  activations, x_dtype (MOE_F32 or MOE_BF16)
 *   w_router     [E, d]  f32 router weight
 *   logit_offset [E]     f32 or NULL: added to every token's logit for expert
 *                        e (a fixed router bias term; it is part of the raw
 *                        logit, so it moves both selection and gates)
 *   sel_bias     [E]     f32 or NULL: the loss-free balancing bias; added to
 *                        the score for selection only, never to a gate
 *   E, k, score_fn       experts, experts per token, enum moe_score
 *   topk_idx     [T, k]  int32 out: chosen experts, best first (key
 *                        descending, equal keys to the lower expert index)
 *   topk_gate    [T, k]  f32 out: gate of each chosen expert
 *   logits_out   [T, E]  f32 out: router logits (offset included), kept for
 *                        the backward
 * Logits are computed in fp32 from x (bf16 widened exactly) and W_r, with
 * blocked accumulation (partial sums of at most 64 products).
 * ENOTSUP: E > MOE_MAX_EXPERTS, k > MOE_MAX_TOPK, d not a multiple of 8,
 * d >= 2^24, T >= 2^31.
 */
moe_status moe_route(const void* x, int x_dtype, int64_t T, int64_t d,
                     const float* w_router, const float* logit_offset, const float* sel_bias,
                     int E, int k, int score_fn,
                     int32_t* topk_idx, float* topk_gate, float* logits_out, void* stream);

/*
 * moe_route_replay — gates and logits of a GIVEN expert choice.
 * Lesson, Exercises item 3 (routing replay: record the experts fired at
 * inference and force the same routing when computing gradients).  The
 * logits are computed as in moe_route; topk_idx is an input, and the gates
 * follow score_fn over exactly those experts.  Passing moe_route's own
 * choice reproduces its gates.
 * Precondition: a replayed choice is one a router made, so each row holds k
 * distinct ids in [0, E).  The library does not check this on the device.
 * For a row that breaks it the gates, the expert rows and the gradients of
 * that token are unspecified; the kernels never use such an id as an index,
 * so every call stays inside its buffers, and the outputs and input
 * gradients of the other tokens are unaffected.
 *   topk_idx [T, k] int32 in;  topk_gate [T, k] f32 out;  logits_out [T, E] out
 * Errors as moe_route.
 */
moe_status moe_route_replay(const void* x, int x_dtype, int64_t T, int64_t d,
                            const float* w_router, const float* logit_offset,
                            int E, int k, int score_fn, const int32_t* topk_idx,
                            float* topk_gate, float* logits_out, void* stream);

/*
 * moe_route_hash — a deterministic router with nothing learned.
 * Lesson, Exercises item 2 (replace the learned router by a hash-based
 * one).  For token id (token_ids[t], e.g. its vocabulary id) and expert e,
 * the key is the SplitMix64 output for state id*2^32 + e advanced salt+1
 * times (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014):
 *   z = id*2^32 + e + (salt+1) * 0x9E3779B97F4A7C15   (mod 2^64)
 *   z = (z ^ z>>30) * 0xBF58476D1CE4E5B9
 *   z = (z ^ z>>27) * 0x94D049BB133111EB
 *   key = z ^ z>>31
 * The token takes the k experts with the smallest keys, in ascending key
 * order, each with gate 1/k (f32).  Use salt to give layers different maps.
 *   token_ids [T] int32 in;  topk_idx [T, k] int32 out;  topk_gate [T, k] out
 * ENOTSUP: E > MOE_MAX_EXPERTS, k > MOE_MAX_TOPK, T >= 2^31.
 */
moe_status moe_route_hash(const int32_t* token_ids, int64_t T, int E, int k, uint32_t salt,
                          int32_t* topk_idx, float* topk_gate, void* stream);

/*
 * moe_permute — group the T*k (token, expert) assignments by expert.
 * The expert GEMMs need each expert's tokens contiguous: this is the
 * "permute" step whose fusion the AREX article's paragraph on hiding
 * all-to-all reports (permute/copy kernels 11.45% -> 7.14% of step time).
 * Stable counting sort: experts ascending, and inside an expert the tokens
 * ascending, so the result is unique and reproducible bit for bit.  No
 * atomics are used.
 *
 *   topk_idx [T, k]     int32 expert per assignment (from moe_route)
 *   x        [T, d]     rows to copy, x_dtype
 *   counts   [E]        int32 out: assignments per expert
 *   offsets  [E+1]      int32 out: exclusive prefix sum of counts
 *   row_of   [T, k]     int32 out: row of assignment (t, j) in x_perm
 *                       (INT32_MIN for an expert id outside [0, E): that
 *                       assignment has no row and is skipped downstream)
 *   token_of [T*k]      int32 out: token of each x_perm row
 *   x_perm   [T*k, d]   out: x_perm[r] = x[token_of[r]] (bit copy), or NULL:
 *                       indices only, no copy (for moe_grouped_ffn_gather,
 *                       which reads x through token_of); x may then be NULL
 *   workspace           moe_workspace_size(MOE_CALL_PERMUTE, T, k, E, d, 0)
 * ENOTSUP: E > MOE_MAX_EXPERTS, k > MOE_MAX_TOPK, T*k >= 2^31, d*elem not a
 * multiple of 16 bytes.
 */
moe_status moe_permute(const int32_t* topk_idx, int64_t T, int k, int E,
                       const void* x, int x_dtype, int64_t d,
                       int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of,
                       void* x_perm, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_permute_capacity — moe_permute with an expert capacity.
 * Lesson, Load balancing item 2 (expert capacity + token dropping): each
 * expert processes at most a fixed number of tokens (C x N / E for a
 * capacity factor C) and the overflow skips the layer.  With top-k routing
 * the cap counts assignments; the caller passes it in rows, usually
 * ceil(C * T * k / E).  An expert keeps its first `capacity` assignments in
 * token order and drops the rest.
 *   capacity  rows per expert; < 0 (or >= T*k) keeps everything, which is
 *             exactly moe_permute
 *   counts    [E]   every assignment per expert, dropped ones included (the
 *                   router's demand: what moe_bias_update balances)
 *   offsets   [E+1] exclusive prefix sum of the KEPT counts
 *                   min(counts, capacity): expert e runs on rows
 *                   offsets[e] .. offsets[e+1]-1, A_kept = offsets[E]
 *   row_of    [T,k] r >= 0 for a kept assignment; ~r (< 0, not INT32_MIN)
 *                   for a dropped one, whose row r lies in [A_kept, T*k)
 *   token_of, x_perm  all T*k rows: the kept rows grouped by expert, then
 *                   the dropped rows grouped by expert (experts ascending,
 *                   tokens ascending inside each); dropped rows are still
 *                   copied because the router weight gradient uses them
 * A dropped slot contributes nothing to moe_combine's sum (the token skips
 * the layer for that slot; gates are not renormalised), gets no expert
 * gradient in moe_backward, and still passes the gate-normalisation gradient
 * to its logit.  Workspace and errors as moe_permute.
 */
moe_status moe_permute_capacity(const int32_t* topk_idx, int64_t T, int k, int E, int64_t capacity,
                                const void* x, int x_dtype, int64_t d,
                                int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of,
                                void* x_perm, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch behind moe_permute_noalloc. */
#define MOE_PERMUTE_NOALLOC_SCRATCH (4u << 20)

/*
 * moe_permute_noalloc — moe_permute with no workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It calls no allocator:
 * its scratch (the per-chunk expert histogram) is a static device array of
 * MOE_PERMUTE_NOALLOC_SCRATCH bytes, one per GPU, held until the process
 * ends.  Arguments, results and errors as moe_permute (no capacity), plus
 * ENOTSUP when the histogram, ceil(T*k/256) * E * 4 bytes, exceeds that
 * size (T*k = 2^20 assignments fit with E up to 256, 2^18 with E up to
 * 1024); EHIP when the scratch address cannot be looked up.  Every call on one GPU uses that
 * GPU's one scratch array: calls that may overlap on one GPU (different
 * streams, host threads) race and give wrong results; order them on one
 * stream.  Nothing in the scratch has to start at zero.
 */
moe_status moe_permute_noalloc(const int32_t* topk_idx, int64_t T, int k, int E,
                               const void* x, int x_dtype, int64_t d,
                               int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of,
                               void* x_perm, void* stream);

/*
 * moe_grouped_ffn — G independent SwiGLU experts over row segments.
 * Lesson, Concept: each expert is an independent FFN, usually SwiGLU.
 * Expert g runs on rows offsets[g] .. offsets[g+1]-1 of x_rows (rows at or
 * past offsets[G], e.g. those dropped by an expert capacity, are neither read
 * nor written):
 *   G = X W_gate^T, U = X W_up^T, H = silu(G) * U, Y = H W_down^T,
 *   silu(z) = z / (1 + e^-z).
 * The shared expert of the lesson's Shared-experts section is the same call
 * with G = 1 and offsets = {0, T} over the layer input.
 *
 *   x_rows     [rows, d]     dtype
 *   offsets    [G+1]         int32 device, nondecreasing, offsets[0] = 0,
 *                            offsets[G] <= rows (device values, not checked:
 *                            offsets outside that range read and write out of
 *                            bounds)
 *   w_gate_up  [G, 2f, d]    dtype: f gate rows, then f up rows per expert
 *   w_down     [G, d, f]     dtype
 *   gu_saved   [rows, 2f]    dtype out or NULL: G (cols 0..f-1) and U
 *                            (cols f..2f-1), kept for the backward
 *   h          [rows, f]     dtype out: SwiGLU output (from the unrounded
 *                            fp32 G and U)
 *   y          [rows, d]     f32 out
 *   workspace                moe_workspace_size(MOE_CALL_GROUPED_FFN, rows, 1, G, d, f)
 * bf16 uses MFMA with fp32 accumulation; f32 uses fp32 FMA.
 * ENOTSUP: G > MOE_MAX_EXPERTS, rows >= 2^31; bf16 needs d and f to be
 * multiples of 64 (the GEMM loops run over pairs of 32-deep slabs and the
 * SwiGLU tiles pair 64-column gate and up blocks; there is no tail path
 * along d or f) and one expert's gate/up weight under 2 GiB
 * (2f*d*2 < 2^31 bytes: it is addressed through one buffer resource); f32
 * needs d a multiple of 4.
 */
moe_status moe_grouped_ffn(const void* x_rows, int64_t rows, int64_t d, int dtype,
                           const int32_t* offsets, int G, int64_t f,
                           const void* w_gate_up, const void* w_down,
                           void* gu_saved, void* h, float* y,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_grouped_ffn_gather — moe_grouped_ffn on the unpermuted input: GEMM
 * row r reads row token_of[r] of x (the permute fused into the expert GEMM's
 * operand loads).  The AREX article on The Ultimate MoE Training Handbook, in
 * its paragraph on the handbook's section 3.7, reports that fusing the
 * permute cut the permute/copy kernels' share of the step; with this call
 * (and moe_backward with x_perm = NULL) a forward or training step runs
 * moe_permute with x_perm = NULL and never writes X_perm.
 *   x          [T, d]        dtype, the layer input
 *   token_of   [rows]        int32 device, from moe_permute (values in
 *                            [0, T); an index outside reads as a zero row)
 *   rows, offsets, w_gate_up, w_down, gu_saved, h, y, workspace: as
 *                            moe_grouped_ffn (h, y, gu_saved in permuted
 *                            row order)
 * Errors as moe_grouped_ffn; EINVAL for a NULL token_of; ENOTSUP (bf16) when
 * T*d*2 >= 2^31 (x is addressed through one buffer resource).
 */
moe_status moe_grouped_ffn_gather(const void* x, int64_t T, const int32_t* token_of, int64_t rows, int64_t d,
                                  int dtype, const int32_t* offsets, int G, int64_t f,
                                  const void* w_gate_up, const void* w_down, void* gu_saved, void* h, float* y,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Expert weights packed in the order the bf16 GEMM tiles stream them.
 * The expert GEMM's slab loads fetch, per 32-deep step, 64 bytes from each
 * of 256 weight rows; at the 256-expert shape the expert weights are read
 * from HBM about once per forward, and that strided pattern streams at
 * about two thirds of what the same bytes read in order do.  A serving
 * caller whose weights do not change between calls packs them once
 * (moe_pack_expert_weights) and runs moe_grouped_ffn_packed, which reads
 * each slab as one contiguous 16 KB block and gives bit for bit the
 * results of moe_grouped_ffn / moe_grouped_ffn_gather on the unpacked
 * weights.  The Lesson's Concept section defines the expert FFN computed;
 * the packing is a storage order only.
 *
 * moe_packed_weight_bytes: bytes of the packed copy of w_gate_up (which =
 * 0: G*2f*d*2) or of w_down (which = 1: G*ceil(d/256)*256*f*2, rows past d
 * zero); 0 for other arguments.
 *
 * moe_pack_expert_weights: w_gate_up [G, 2f, d] and w_down [G, d, f], bf16,
 * as moe_grouped_ffn takes them, into packed_gate_up / packed_down (device
 * buffers of moe_packed_weight_bytes, caller-owned; the layout is private
 * to this library).  ENOTSUP unless d is a multiple of 64 and f of 128 (the
 * 256 x 256 tile), G <= MOE_MAX_EXPERTS.
 *
 * moe_grouped_ffn_packed: moe_grouped_ffn_gather (token_of set: GEMM row r
 * reads row token_of[r] of x, which has T rows) or moe_grouped_ffn
 * (token_of NULL: x holds the `rows` rows; T is ignored) on packed weights,
 * bf16 only.  Other arguments, outputs and errors as those calls; ENOTSUP
 * when f is not a multiple of 128.
 */
size_t moe_packed_weight_bytes(int which, int64_t G, int64_t d, int64_t f);
moe_status moe_pack_expert_weights(const void* w_gate_up, const void* w_down, int64_t G, int64_t d, int64_t f,
                                   void* packed_gate_up, void* packed_down, void* stream);
moe_status moe_grouped_ffn_packed(const void* x, int64_t T, const int32_t* token_of, int64_t rows, int64_t d,
                                  const int32_t* offsets, int G, int64_t f, const void* packed_gate_up,
                                  const void* packed_down, void* gu_saved, void* h, float* y,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_ffn_stage_events — per-GEMM timing of one grouped FFN call.  The next
 * moe_grouped_ffn, moe_grouped_ffn_gather or moe_grouped_ffn_packed call
 * made from the calling host thread records events[MOE_FFN_STAGE_UP] on
 * its stream after the up-projection (with its tile schedule) and
 * events[MOE_FFN_STAGE_DOWN] after the down-projection, so a caller that
 * records one event before the call can time both GEMMs with
 * hipEventElapsedTime (the two expert GEMMs of the Lesson's Concept section
 * and its Cost profile).  The setting is taken by that one call, whatever
 * it returns, and then cleared.
 *   events   NULL (no timing), or a HOST array of MOE_FFN_STAGES hipEvent_t
 *            (as void*, NULL entries skipped) owned by the caller; the array
 *            must stay valid until the call that takes it returns.
 * Returns MOE_OK.  A failed event record makes the grouped FFN call return
 * MOE_EHIP at that point (what it enqueued before stays enqueued).
 */
enum moe_ffn_stage {
  MOE_FFN_STAGE_UP = 0,     /* tile schedule; x W_gate_up with the SwiGLU epilogue */
  MOE_FFN_STAGE_DOWN = 1,   /* H W_down */
  MOE_FFN_STAGES = 2
};
moe_status moe_ffn_stage_events(void* const* events);

/*
 * moe_combine — gate-weighted sum of each token's expert outputs.
 * Lesson, Concept: the layer adds, over the chosen experts, gate times the
 * expert's output; shared experts add their output unweighted.  The residual
 * add of the transformer block is outside this call.
 *   out[t] = shared_y[t] + sum_j topk_gate[t,j] * y_perm[row_of[t,j]]
 * summed in fp32, j ascending.  A slot with row_of[t,j] < 0 (dropped by an
 * expert capacity, or an invalid expert id) adds nothing; its y_perm row is
 * never read into the sum, so it may hold any bits.
 *   y_perm   [T*k, d] f32;  row_of [T, k] int32;  topk_gate [T, k] f32
 *   shared_y [T, d]   f32 or NULL
 *   out      [T, d]   out_dtype (MOE_F32, or MOE_BF16 rounded to nearest even)
 * ENOTSUP: k > MOE_MAX_TOPK, d not a multiple of 4.
 */
moe_status moe_combine(const float* y_perm, const int32_t* row_of, const float* topk_gate,
                       const float* shared_y, int64_t T, int k, int64_t d,
                       void* out, int out_dtype, void* stream);

/*
 * moe_bias_update — the loss-free balancing controller.
 * Lesson, Load balancing item 3 and Build it step 2: after each step an
 * expert used more than the uniform target moves its bias down by gamma, one
 * used less moves it up.  Here: E*counts[e] > T*k -> bias[e] -= gamma;
 * E*counts[e] < T*k -> bias[e] += gamma; equal -> unchanged (integer
 * comparison, one fp32 add).
 *   sel_bias [E] f32 in/out;  counts [E] int32 (from moe_permute)
 */
moe_status moe_bias_update(float* sel_bias, const int32_t* counts, int E, int64_t T, int k,
                           float gamma, void* stream);

/*
 * moe_aux_loss — auxiliary load-balancing loss (the alternative to the
 * loss-free bias).  Lesson, Load balancing item 1 and Key terms: an extra
 * loss term that penalises uneven expert usage, with its own weight and
 * gradient.  The pages give no formula; this is the Switch/GShard form
 *   L_aux = alpha * E / (T*k) * sum_e counts[e] * P[e],
 *   P[e]  = (1/T) sum_t p[t, e],
 * p the router probabilities over ALL E experts: softmax of the logits for
 * MOE_SOFTMAX_CHOSEN, each score over the sum of all E scores for the
 * normalised score functions.  Balanced counts and uniform p give alpha.
 * Reductions run in a fixed order (bit-reproducible).
 *   logits [T, E] f32 (moe_route's logits_out);  counts [E] int32 (moe_permute)
 *   loss_out [1] f32 device out;  p_mean_out [E] f32 out or NULL
 *   workspace  moe_workspace_size(MOE_CALL_AUX_LOSS, T, k, E, 0, 0)
 * Its gradient is added by moe_backward when moe_bwd_args.aux_alpha != 0.
 * ENOTSUP: E > MOE_MAX_EXPERTS, T >= 2^31.
 */
moe_status moe_aux_loss(const float* logits, const int32_t* counts, int64_t T, int E, int k, int score_fn,
                        float alpha, float* loss_out, float* p_mean_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_backward — gradients of the routed layer (training).
 * The pages give no backward formulas; this is the chain rule through the
 * forward above.  The selection bias and the logit offset get no gradient
 * (lesson, Key terms: the loss-free bias adds no gradient signal), and the
 * discrete top-k choice is held fixed.
 *   combine:  dg[t,j] = <dy[t], y_perm[row_of[t,j]]>, computed as
 *             <dy[t] W_down[e], H[row]> (the same sum, y_perm = H W_down^T,
 *             so y_perm is not read), dY_perm[row_of[t,j]] = bf16(gate[t,j] * dy[t])
 *   gates:    softmax: dl_j = g_j (dg_j - D), D = sum_i g_i dg_i;
 *             normalised scores: dl_j = (dg_j - D) / S * s'(l_j), S = sum s
 *   router:   dW_r = dL^T x, dx_r = dL W_r (dL = dl at the chosen experts)
 *   experts:  dH = gate * (dy W_down) (fp32); dG = bf16(dH U silu'(G));
 *             dU = bf16(dH silu(G)) from the saved bf16 G, U;
 *             dW_down = dY_perm^T H; dW_gate = dG^T X; dW_up = dU^T X;
 *             dX_perm = dG W_gate + dU W_up
 *   unpermute: dx[t] = sum_j dX_perm[row_of[t,j]] + dx_r[t]
 * All pointers are device pointers held in a HOST struct.  bf16 layers only.
 * An expert id outside [0, E) (which moe_route_replay's precondition rules
 * out) gives that token unspecified gradients and stays in bounds.
 * score_fn MOE_UNIFORM_GATES (hash routing): dl = 0, there is no router term
 * in dx, w_router / logits may be NULL, and dw_router (if not NULL) is
 * set to zero.
 */
typedef struct moe_bwd_args {
  size_t struct_size;          /* sizeof(moe_bwd_args): the ABI version */
  int64_t T, d, f;
  int E, k, score_fn;
  /* inputs */
  const void* dy;              /* [T, d] bf16: gradient of the layer output */
  const void* x;               /* [T, d] bf16 */
  const float* w_router;       /* [E, d] */
  const float* logits;         /* [T, E] from moe_route */
  const int32_t* topk_idx;     /* [T, k] */
  const float* topk_gate;      /* [T, k] */
  const int32_t* row_of;       /* [T, k] */
  const int32_t* token_of;     /* [T*k] */
  const int32_t* offsets;      /* [E+1] */
  const void* x_perm;          /* [T*k, d] bf16, or NULL: the weight gradient
                                  of W_gate_up then reads row token_of[r] of x
                                  for row r (no X_perm buffer needed) */
  const void* gu_saved;        /* [T*k, 2f] bf16 */
  const void* h;               /* [T*k, f] bf16 */
  const float* y_perm;         /* not read, may be NULL (kept for the struct
                                  layout): dg is formed from dy W_down and H */
  const void* w_gate_up;       /* [E, 2f, d] bf16 */
  const void* w_down;          /* [E, d, f] bf16 */
  /* outputs (f32) */
  float* dx;                   /* [T, d] */
  float* dw_router;            /* [E, d] */
  float* dw_gate_up;           /* [E, 2f, d] */
  float* dw_down;              /* [E, d, f] */
  float* dgate;                /* [T, k] or NULL: dg, exposed for checking */
  float* dlogit;               /* [T, k] or NULL: dl at the chosen experts */
  void* workspace;
  size_t workspace_bytes;      /* moe_workspace_size(MOE_CALL_BACKWARD, T, k, E, d, f) */
  /* appended; a struct_size that ends before it means NULL */
  const int32_t* counts;       /* [E] from moe_permute_capacity, or NULL when
                                  nothing was dropped (then x_perm holds the
                                  kept rows only); required with aux_alpha */
  float aux_alpha;             /* weight of the auxiliary load-balancing loss
                                  (moe_aux_loss) whose gradient is added; 0: none */
  /* appended: the shared expert (lesson, Shared experts section: an expert
     every token passes through, its output added with weight 1).  NULL
     w_gate_up_shared: the layer has none and the other shared fields are
     ignored.  Its backward is the expert chain rule above with dY_perm = dy
     and X = x over all T rows; its input gradient is added to dx. */
  int64_t f_shared;            /* shared expert FFN width (a multiple of 64) */
  const void* w_gate_up_shared;   /* [2fs, d] bf16 */
  const void* w_down_shared;      /* [d, fs] bf16 */
  const void* gu_shared;       /* [T, 2fs] bf16: G|U saved by the forward
                                  (moe_grouped_ffn's gu_saved) */
  const void* h_shared;        /* [T, fs] bf16: the forward's H */
  float* dw_gate_up_shared;    /* [2fs, d] out */
  float* dw_down_shared;       /* [d, fs] out */
  void* workspace_shared;      /* moe_workspace_size(MOE_CALL_BACKWARD_SHARED,
                                  T, 1, 1, d, f_shared) bytes */
  size_t workspace_shared_bytes;
  /* appended: per-stage timing.  NULL, or a HOST array of MOE_BWD_STAGES
     hipEvent_t (as void*): event s is recorded on the stream after stage s
     (enum moe_bwd_stage), so a caller that records one event before the call
     can time every stage with hipEventElapsedTime.  Stages the call does not
     run (e.g. the shared expert's without one) still record their event. */
  void* const* stage_events;
} moe_bwd_args;

/* Stages of moe_backward, in stream order (for moe_bwd_args.stage_events). */
enum moe_bwd_stage {
  MOE_BWD_COMBINE = 0,      /* combine backward: dY_perm = bf16(g dy) per expert row */
  MOE_BWD_DGRAD_DOWN = 1,   /* tile schedule; dH' = dy W_down, dg partials <dH', H>,
                               dH = g dH', SwiGLU backward -> dG|dU */
  MOE_BWD_ROUTER = 2,       /* gate backward (dg, dl) and the router weight gradient */
  MOE_BWD_WGRAD_DOWN = 3,   /* dW_down = dY_perm^T H */
  MOE_BWD_WGRAD_UP = 4,     /* dW_gate_up = [dG|dU]^T X */
  MOE_BWD_DGRAD_UP = 5,     /* dX_perm = [dG|dU] W_gate_up */
  MOE_BWD_SHARED = 6,       /* the shared expert's four GEMMs */
  MOE_BWD_UNPERMUTE = 7,    /* dx = sum_j dX_perm rows + router and shared terms */
  MOE_BWD_STAGES = 8
};

/* With aux_alpha != 0 the gradient of moe_aux_loss (same alpha, counts
 * and logits) is added: it reaches every logit, so dW_r = dL^T x and
 * dx_r = dL W_r use the dense [T, E] logit gradient dL (the chosen experts'
 * dl plus the aux part); `dlogit` still reports the main-loss dl of the
 * chosen experts.  Needs a learned router and `counts`.
 * With an expert capacity (row_of < 0 for dropped slots, `counts` set): a
 * dropped slot gets dg = 0 and no dY_perm / dX_perm row; its dl (through the
 * gate normalisation) still reaches dW_r over its dropped x_perm row and
 * dx_r.  Expert GEMMs run on the kept rows offsets[0] .. offsets[E]-1.
 * ENOTSUP: non-bf16 use, d, f or f_shared not a multiple of 64,
 * E > MOE_MAX_EXPERTS, k > MOE_MAX_TOPK, T*k >= 2^31, and buffers the GEMMs
 * address through one buffer resource reaching 2 GiB: T*k*max(d, 2f)*2 >=
 * 2^31 or 2f*d*2 >= 2^31 bytes (for the shared expert T*max(d, 2fs)*2 and
 * 2fs*d*2).  The multiples of 64: the GEMM loops run over pairs of
 * 32-deep slabs and the SwiGLU tiles pair 64-column gate and up blocks,
 * with no tail path along d or f.  EINVAL also
 * for a struct_size other than sizeof(moe_bwd_args) or the offset of one of
 * the appended fields counts, aux_alpha, f_shared or stage_events (older
 * callers: the missing fields read as NULL / 0); EWORKSPACE for a missing
 * or small workspace_shared when a shared expert is given. */
moe_status moe_backward(const moe_bwd_args* args, void* stream);

/* Workspace bytes a call needs (0 if it needs none).  `which` is enum
 * moe_call; arguments a call does not use are ignored.  For
 * MOE_CALL_GROUPED_FFN pass T = rows, k = 1, E = G. */
size_t moe_workspace_size(int which, int64_t T, int k, int E, int64_t d, int64_t f);

/* Static description of a status code. */
const char* moe_status_str(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
