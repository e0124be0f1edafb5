/*
 * moe.h - C ABI of libmoe.so, the MI355X (gfx950) MoE feed-forward layer.
 *
 * The layer, per token x_t (width D), as the Laguna pages define it:
 *   logits   z_t = W_r x_t + b                          ("Laguna M.1/XS.2 Technical
 *            Report", Key claims: sigmoid router, token-choice top-8 of 256,
 *            post-top-k normalization, routed output modulated by 2.5 before
 *            the shared expert is added; report section 3.1)
 *   select   the k experts first under (z descending, expert index ascending)
 *   weights  w_j = sigmoid(z_{e_j}) / sum_i sigmoid(z_{e_i})
 *   experts  y = W_d (silu(W_g x) * (W_u x)), no biases ("Laguna-M.1-base",
 *            Feed-forward: SwiGLU, FFN bias = no)
 *   output   out_t = ysh_t + alpha * sum_j w_j y_{t,j}, ysh = the shared expert
 *
 * The pages' training system sends tokens to expert owners over NVLink inside a
 * fused grouped GEMM ("Laguna M.1/XS.2 Technical Report", Key claims: dispatch
 * and combine fused into the grouped GEMM, report section 3.1.2, Fig. 2).  On
 * one GPU that exchange becomes an on-device permutation into expert order.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the
 *     caller, 16-byte aligned, row-major and densely packed.  The library never
 *     allocates or frees device memory and keeps no device state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue kernels on it and never synchronise; results are ready when the
 *     stream has reached that point.  Asynchronous faults surface at the
 *     caller's next synchronisation.
 *   - "elem" is 4 bytes (fp32) for MOE_F32 and 2 bytes (bf16 bit patterns)
 *     for MOE_BF16.  Accumulation is fp32 in both cases.
 *   - Return value: a moe_status.  Arguments are checked on the host before
 *     anything is launched; a rejected call enqueues nothing.  The reason of
 *     the last failure on the calling thread is in moe_last_error().
 *   - T == 0 is a valid empty batch: the call does nothing and returns MOE_OK.
 *   - Calls that share output buffers on one stream are ordered by the stream;
 *     calls on different streams that write the same buffers race.
 *
 * Shape limits (else MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED):
 *   1 <= E <= 256, 1 <= k <= min(E, 16), T >= 0, T * k < 2^31.
 *   MOE_BF16: D % 256 == 0, F % 256 == 0, Fs % 256 == 0 (Fs == 0 = no shared expert),
 *             T * D < 2^31, T * Fs < 2^31.
 *   MOE_F32:  D % 32 == 0, F % 16 == 0, Fs % 16 == 0, D, F, Fs <= 8192.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* bad shape, null or misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2,   /* valid layer, but outside this library's limits */
  MOE_ERR_WORKSPACE = 3,     /* workspace missing or smaller than moe_workspace_bytes */
  MOE_ERR_HIP = 4            /* a kernel launch failed (hipGetLastError) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer shape.  T tokens, model width D, E routed experts, k experts per token,
 * routed SwiGLU width F, shared SwiGLU width Fs (0 = none), routed scale alpha
 * (2.5 for XS.2, 1 for M.1: "Laguna M.1/XS.2 Technical Report", Key claims;
 * "Laguna-M.1-base", Mixture of experts: Routed scaling factor), dtype. */
typedef struct moe_shape {
  int32_t T, D, E, k, F, Fs;
  float alpha;
  int32_t dtype; /* moe_dtype */
} moe_shape;

/* Library ABI version (this header: 1). */
int moe_version(void);

/* Static description of a status code.  Never NULL. */
const char* moe_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if none).
 * The string is thread-local and valid until the next call on that thread. */
const char* moe_last_error(void);

/* Bytes of device workspace moe_permute needs for this shape (0 on a bad shape).
 * A multiple of 256. */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Router: logits, top-k selection and renormalised weights.
 * Defined by the sigmoid token-choice top-k router with post-top-k
 * normalisation ("Laguna M.1/XS.2 Technical Report", Key claims; report
 * section 3.1) -- selection on the fp32 logit, ties to the lower expert index
 * (-0.0 equals +0.0).
 *   x         [T, D] elem      layer input (after the pre-norm)
 *   w_router  [E, D] elem      router weight
 *   bias      [E] fp32 or NULL additive logit bias (affects selection and weight)
 *   logits    [T, E] fp32      out: z = x W_r^T + b, the values selection used
 *   topk_idx  [T, k] int32     out: slot j = j-th expert under the order above
 *   topk_w    [T, k] fp32      out: sigmoid(z)/sum over the k slots (sums to 1;
 *                              alpha is NOT applied here)
 * Non-finite logits are outside the contract: the result is unspecified (still
 * k distinct in-range experts per token) and nothing faults. */
int moe_route(const moe_shape* shape, const void* x, const void* w_router, const float* bias,
              float* logits, int32_t* topk_idx, float* topk_w, void* stream);

/* moe_route with a padding mask: padding tokens are neither routed nor load
 * balanced ("Laguna M.1/XS.2 Technical Report", thread on the report: padding
 * tokens always went to one expert and could not learn, so they were left out
 * of routing and load balancing).
 *   mask      [T] uint8 or NULL (= every token routed); 0 marks padding
 * A padding token's logits are still written; its topk_idx row is -1 and its
 * topk_w row 0.  moe_permute and moe_combine then skip it: its output is the
 * shared expert's alone. */
int moe_route_masked(const moe_shape* shape, const void* x, const void* w_router, const float* bias,
                     const uint8_t* mask, float* logits, int32_t* topk_idx, float* topk_w,
                     void* stream);

/* Expert-order permutation: the on-device form of the dispatch all-to-all
 * (tokens copied "in expert order": "Laguna M.1/XS.2 Technical Report", Key
 * claims, fused dispatch/grouped GEMM, report section 3.1.2, Fig. 2).
 *   topk_idx     [T, k] int32   in: from moe_route (values in [0, E)) or
 *                               moe_route_masked (-1: a slot not routed)
 *   x            [T, D] elem    in: layer input
 *   counts       [E] int32      out: tokens routed to each expert
 *   offsets      [E+1] int32    out: exclusive scan of counts; offsets[E] = the
 *                               routed slots (k*T without padding)
 *   sorted_token [k*T] int32    out: expert by expert, the tokens in ascending
 *                               token order (the first offsets[E] entries)
 *   slot_of      [T, k] int32   out: position of (t, j) in that order; -1 for a
 *                               slot not routed
 *   x_perm       [k*T, D] elem  out: x_perm[p] = x[sorted_token[p]]; may be NULL
 *                               to skip the copy
 *   workspace    >= moe_workspace_bytes(shape) bytes, caller-owned scratch
 * The result is deterministic (no order depends on timing). */
int moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* counts,
                int32_t* offsets, int32_t* sorted_token, int32_t* slot_of, void* x_perm,
                void* workspace, size_t workspace_bytes, void* stream);

/* moe_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and outputs, with the per-block histograms in a
 * device-resident array of the library instead of a caller workspace.
 *   - the array holds 1 MiB per GPU (kept until the process ends), enough for
 *     moe_workspace_bytes(shape) <= 1 MiB, i.e. ceil(T / 256) * E * 4 bytes
 *     (T <= 262144 tokens at E = 256); larger shapes return
 *     MOE_ERR_UNSUPPORTED before anything is launched;
 *   - nothing is allocated or freed; the array's address on the current device
 *     is looked up once per device (MOE_ERR_HIP if that fails);
 *   - every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (other streams, other threads) race and must be ordered by the caller;
 *     no part of the array needs to start at zero (each call writes what it
 *     reads).
 * Arguments as moe_permute, without workspace and workspace_bytes. */
int moe_permute_static(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_token, int32_t* slot_of, void* x_perm,
                       void* stream);

/* Repack weight matrices into MFMA fragment order, the layout every weight
 * argument of moe_grouped_gate_up / moe_grouped_down / moe_grouped_ffn takes
 * (a one-time pass when weights are loaded; the pages' experts are the
 * SwiGLU projections of "Laguna-M.1-base", Feed-forward).
 *   w         [count, rows, cols] elem, row-major (e.g. w_gate_up as [E, 2F, D])
 *   w_packed  moe_packed_bytes(count, rows, cols, dtype) bytes, out; must not
 *             overlap w
 *   rows % 32 == 0, cols % 16 == 0 (else MOE_ERR_INVALID_ARG)
 * Layout: matrix i starts at element i * rows * cols; in it, element (r, c)
 * goes to
 *   ((r / 32) * (cols / 16) + c / 16) * 512 + ((r % 32) + 32 * ((c % 16) / 8)) * 8 + c % 8,
 * i.e. 32 x 16 blocks, row-block major, in which 16-byte (bf16) lane chunks
 * are the operand of one wave for one 32x32x16 MFMA step. */
int moe_pack_weights(const void* w, void* w_packed, int64_t count, int32_t rows, int32_t cols,
                     int32_t dtype, void* stream);

/* Size in bytes of `count` packed [rows, cols] matrices of type dtype (the
 * same as unpacked: count * rows * cols * element size); 0 for sizes
 * moe_pack_weights rejects. */
size_t moe_packed_bytes(int64_t count, int32_t rows, int32_t cols, int32_t dtype);

/* First grouped GEMM of the experts with the SwiGLU fused in its epilogue
 * ("Laguna-M.1-base", Feed-forward: SwiGLU, no bias; the grouped GEMM over
 * expert-ordered tokens of "Laguna M.1/XS.2 Technical Report", Key claims,
 * report section 3.1.2).  For each expert e and each of its rows p in
 * [offsets[e], offsets[e+1]):  h[p] = silu(Wg_e a_p) * (Wu_e a_p)  where a_p is
 * x_perm[p], or x[sorted_token[p]] when x_perm is NULL.  The shared expert
 * does the same for every token t:  hs[t] = silu(Wsg x_t) * (Wsu x_t).
 *   x_perm       [k*T, D] elem or NULL (then sorted_token is read)
 *   sorted_token [k*T] int32 (read only when x_perm is NULL)
 *   x            [T, D] elem
 *   offsets      [E+1] int32 from moe_permute
 *   w_gate_up    E matrices [2F, D] elem, packed (moe_pack_weights, count E):
 *                rows 0..F-1 = gate projection, F..2F-1 = up projection
 *   ws_gate_up   one matrix [2Fs, D] elem, packed, same split; ignored (may be
 *                NULL) when Fs == 0.  bf16: NULL with Fs > 0 computes the routed
 *                experts only and leaves the shared rows of h untouched (the
 *                shared expert then runs through moe_shared_ffn)
 *   h            [k*T*F + T*Fs] elem out: routed rows [k*T, F], then shared rows [T, Fs]
 * The h values are rounded once to elem (bf16 round-to-nearest-even). */
int moe_grouped_gate_up(const moe_shape* shape, const void* x_perm, const int32_t* sorted_token,
                        const void* x, const int32_t* offsets, const void* w_gate_up,
                        const void* ws_gate_up, void* h, void* stream);

/* Second grouped GEMM: y_perm[p] = Wd_e h[p] for the rows of each expert e, and
 * y_shared[t] = Wsd hs[t] ("Laguna-M.1-base", Feed-forward: down projection).
 *   h         as written by moe_grouped_gate_up
 *   offsets   [E+1] int32
 *   w_down    E matrices [D, F] elem, packed (moe_pack_weights, count E)
 *   ws_down   one matrix [D, Fs] elem, packed (ignored, may be NULL, when Fs == 0;
 *             bf16: NULL with Fs > 0 computes the routed experts only)
 *   y_perm    [k*T, D] elem out
 *   y_shared  [T, D] elem out (untouched when Fs == 0 or ws_down is NULL; may
 *             then be NULL) */
int moe_grouped_down(const moe_shape* shape, const void* h, const int32_t* offsets,
                     const void* w_down, const void* ws_down, void* y_perm, void* y_shared,
                     void* stream);

/* The shared expert alone ("Laguna M.1/XS.2 Technical Report", Key claims: one
 * always-on shared expert; "Laguna-M.1-base", Feed-forward: SwiGLU), bf16 only:
 *   hs[t] = silu(Wsg x_t) * (Wsu x_t),  y_shared[t] = Wsd hs[t]  for all T tokens.
 * It reads no routing result, so it can run on a second stream while the
 * router and the permutation run, beside moe_grouped_gate_up and
 * moe_grouped_down called with NULL shared weights (routed experts only).
 *   x           [T, D] bf16
 *   ws_gate_up  [2Fs, D] bf16 packed; ws_down [D, Fs] bf16 packed
 *   h_shared    [T, Fs] bf16 out (h + k*T*F in the layout of moe_grouped_gate_up)
 *   y_shared    [T, D] bf16 out
 * Results equal those of the shared rows of moe_grouped_gate_up and
 * moe_grouped_down bit for bit.  MOE_ERR_UNSUPPORTED for fp32, MOE_ERR_INVALID_ARG
 * when Fs == 0. */
int moe_shared_ffn(const moe_shape* shape, const void* x, const void* ws_gate_up,
                   const void* ws_down, void* h_shared, void* y_shared, void* stream);

/* moe_grouped_gate_up followed by moe_grouped_down on the same stream.
 * The expert weights this takes are NOT row-major [E, 2F, D] / [E, D, F]: they
 * are the output of moe_pack_weights (the same bytes permuted into MFMA operand
 * order, a one-time step when weights are loaded, into a buffer the caller owns
 * and reuses for every call).  Row-major weights have the same size and cannot
 * be told apart here: passing them gives wrong results, not an error.  The
 * grouped GEMMs read every 32-row x 16-column operand block of a weight matrix
 * as one contiguous 1 KB load; packing per call would add a full read and
 * write of the expert weights (1.6-6.4 GB at the configured widths) to every
 * pass.  They need no workspace (the tile table is built on the device from
 * offsets), and with x_perm NULL they read x through sorted_token instead of a
 * materialised copy.  bf16 widths D, F, Fs must be multiples of 256 (whole
 * weight-prefetch rounds of the reduction, 128- and 256-wide output tiles):
 * other widths return MOE_ERR_UNSUPPORTED. */
int moe_grouped_ffn(const moe_shape* shape, const void* x_perm, const int32_t* sorted_token,
                    const void* x, const int32_t* offsets, const void* w_gate_up,
                    const void* w_down, const void* ws_gate_up, const void* ws_down, void* h,
                    void* y_perm, void* y_shared, void* stream);

/* ---- FP8 expert weights --------------------------------------------------
 * The XS.2 release ships FP8 recipes for its MoE layers ("Laguna M.1/XS.2
 * Technical Report", Key claims: FP8, INT4 and NVFP4 quantisation of the MoE
 * layers) without encoding details; this library's reading:
 *   - element format OCP FP8 E4M3 (bias 7, largest finite 448, subnormals,
 *     no infinities; gfx950's native FP8);
 *   - one fp32 scale per output row of every weight matrix:
 *     s_r = max_c |w[r,c]| / 448 in fp32 (1 for an all-zero row);
 *   - code[r,c] = E4M3 nearest to w[r,c] / s_r (fp32 quotient), ties to the
 *     even code, magnitudes past 448 saturating to 448;
 *   - the layer runs with the weights code * s_r.  The GEMMs widen the codes
 *     to bf16 (exact), multiply by the bf16 activations with fp32
 *     accumulation, and apply s_r to the accumulated row before the SwiGLU /
 *     the rounding, which equals the product with code * s_r in exact
 *     arithmetic.
 * Activations stay bf16 (shape dtype MOE_BF16; anything else returns
 * MOE_ERR_UNSUPPORTED).  Weights must be finite (non-finite inputs give
 * unspecified codes). */

/* Bytes of `count` FP8 [rows, cols] matrices (count * rows * cols); 0 unless
 * rows and cols are multiples of 32. */
size_t moe_fp8_packed_bytes(int64_t count, int32_t rows, int32_t cols);

/* Quantise bf16 weights to FP8 and pack them for moe_grouped_gate_up_fp8 /
 * moe_grouped_down_fp8 (a one-time pass when weights are loaded).
 *   w       [count, rows, cols] bf16, row-major, rows = output rows (e.g.
 *           w_gate_up as [E, 2F, D], w_down as [E, D, F])
 *   w_fp8   moe_fp8_packed_bytes(count, rows, cols) bytes, out
 *   scales  [count, rows] fp32, out: s_r per matrix row
 *   rows % 32 == 0, cols % 32 == 0 (else MOE_ERR_INVALID_ARG); the three buffers
 *   must not overlap.
 * Layout: matrix i starts at byte i * rows * cols; in it, the code of (r, c)
 * sits at byte
 *   ((r / 32) * (cols / 32) + c / 32) * 1024 + ((r % 32) + 32 * ((c % 16) / 8)) * 16
 *     + ((c % 32) / 16) * 8 + c % 8,
 * i.e. 32 x 32 blocks of 1 KB in which lane l's 16 bytes are its 8 codes of two
 * consecutive 16-wide K steps of a 32x32x16 MFMA operand. */
int moe_quantize_weights_fp8(const void* w, void* w_fp8, float* scales, int64_t count, int32_t rows,
                             int32_t cols, void* stream);

/* moe_grouped_gate_up with FP8 weights: the same computation and buffers, with
 * w_gate_up / ws_gate_up replaced by moe_quantize_weights_fp8's codes and
 * scales (w_gate_up_scale [E, 2F], ws_gate_up_scale [2Fs]; the shared pair is
 * ignored, may be NULL, when Fs == 0). */
int moe_grouped_gate_up_fp8(const moe_shape* shape, const void* x_perm, const int32_t* sorted_token,
                            const void* x, const int32_t* offsets, const void* w_gate_up,
                            const float* w_gate_up_scale, const void* ws_gate_up,
                            const float* ws_gate_up_scale, void* h, void* stream);

/* moe_grouped_down with FP8 weights (w_down_scale [E, D], ws_down_scale [D]). */
int moe_grouped_down_fp8(const moe_shape* shape, const void* h, const int32_t* offsets,
                         const void* w_down, const float* w_down_scale, const void* ws_down,
                         const float* ws_down_scale, void* y_perm, void* y_shared, void* stream);

/* Combine: out[t] = y_shared[t] + sum_{j=0..k-1} (alpha * topk_w[t,j]) * y_perm[slot_of[t,j]],
 * accumulated in fp32 in slot order and rounded once to elem ("Laguna M.1/XS.2
 * Technical Report", Key claims: routed output modulated by alpha before
 * combining with the shared expert).
 *   y_perm    [k*T, D] elem;  y_shared [T, D] elem or NULL (no shared expert)
 *   slot_of   [T, k] int32 (slots < 0 are skipped);   topk_w [T, k] fp32
 *   out       [T, D] elem out */
int moe_combine(const moe_shape* shape, const void* y_perm, const void* y_shared,
                const int32_t* slot_of, const float* topk_w, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Training pass (MOE_BF16 only, and T * 2 Fs < 2^31; MOE_ERR_UNSUPPORTED otherwise).
 *
 * Forward: moe_route_masked, moe_permute, moe_load_stats,
 * moe_grouped_gate_up_train, moe_grouped_down, moe_combine.  Backward of
 *   J = <dout, out> + L_aux
 * with the top-k selection held fixed: moe_combine_backward,
 * moe_grouped_backward_h, moe_grouped_backward_x, moe_weight_grads, moe_bias_grad.
 * Readings (the pages state none of these formulas):
 *   - load balancing is the global-batch auxiliary loss of Qiu et al. ("Laguna
 *     M.1/XS.2 Technical Report", Key claims, XS.2 routing item): over the N
 *     routed tokens of this batch, f_e = counts_e / sum counts (counts of the
 *     GLOBAL batch: the caller's sum over micro-batches and ranks, or this
 *     batch's), p_e = mean of sigmoid(z_te) / sum_e' sigmoid(z_te'),
 *     L_aux = beta * E * sum_e f_e p_e; the gradient flows through p only;
 *   - weight gradients are bf16 for the experts (bf16 mixed precision: report,
 *     Key claims, report section 3.1.1), fp32 for the router and its bias.
 * Packed transposed weights (moe_pack_weights_transposed) serve the backward
 * products: w_down_t = W_d^T [E, F, D] (k_padded = D), w_gate_up_t =
 * [W_g; W_u]^T [E, D, 2F] (k_padded = 2F), the shared ones alike, and
 * w_router_t = W_r^T [D, 256] (k_padded = 256: rows of W_r past E are zero).
 * Buffers below: S = k*T; "routed + shared" buffers hold the S routed rows in
 * expert order, then the T shared rows.
 * ------------------------------------------------------------------------- */

/* Bytes of workspace moe_load_stats and moe_bias_grad need. */
size_t moe_train_workspace_bytes(const moe_shape* shape);

/* Bytes of moe_pack_weights_transposed's output: count * cols * k_padded * 2,
 * or 0 for a shape it rejects. */
size_t moe_packed_transposed_bytes(int64_t count, int32_t rows, int32_t cols, int32_t k_padded);

/* Transposed packing: matrix i of w [count, rows, cols] bf16 becomes its
 * transpose [cols, k_padded], packed like moe_pack_weights, with columns
 * k >= rows of the transpose zero.  cols % 32 == 0, k_padded % 16 == 0,
 * k_padded >= rows (else MOE_ERR_INVALID_ARG); w_packed must not overlap w. */
int moe_pack_weights_transposed(const void* w, void* w_packed, int64_t count, int32_t rows, int32_t cols,
                                int32_t k_padded, void* stream);

/* Load statistics and auxiliary loss.
 *   logits, topk_idx   from moe_route_masked (topk_idx[t, 0] < 0: padding)
 *   counts [E] int32   this batch's counts (moe_permute); N = sum counts / k
 *                      (not read when T == 0: an empty batch has N = 0, p = 0)
 *   counts_global [E] int32 or NULL: the global batch's counts (NULL = counts)
 *   beta               auxiliary-loss coefficient (not disclosed by the pages)
 *   f, p [E] fp32 out; aux_loss [1] fp32 out;
 *   aux_coef [E] fp32 out: beta * E * f / N, the input of moe_combine_backward
 *   workspace >= moe_train_workspace_bytes
 * Sums run in a fixed order: the results are bit-reproducible. */
int moe_load_stats(const moe_shape* shape, const float* logits, const int32_t* topk_idx,
                   const int32_t* counts, const int32_t* counts_global, float beta, float* f, float* p,
                   float* aux_loss, float* aux_coef, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Forward gate/up for training: the pre-activations and the SwiGLU output.
 *   arguments as moe_grouped_gate_up (w_gate_up packed by moe_pack_weights)
 *   gu  [S, 2F] + [T, 2Fs] bf16 out: [g | u] of each routed row, then of the
 *       shared expert (rounded to bf16)
 *   h   [S, F] + [T, Fs] bf16 out: silu(g) * u from those bf16 values */
int moe_grouped_gate_up_train(const moe_shape* shape, const void* x_perm, const int32_t* sorted_token,
                              const void* x, const int32_t* offsets, const void* w_gate_up,
                              const void* ws_gate_up, void* gu, void* h, void* stream);

/* Backward of the combine, the renormalisation, the sigmoid and L_aux.
 *   dout [T, D] bf16; y_perm, slot_of, topk_idx, topk_w, logits from the forward
 *   aux_coef [E] fp32 from moe_load_stats, or NULL (no auxiliary loss)
 *   dy_perm [S, D] bf16 out: alpha * w_{t,j} * dout_t at row slot_of[t, j]
 *   dz [T, E] fp32 out: dJ/dz (zero rows for padding)
 *   dz_bf16 [T, 256] bf16 out: the same, rounded, zero past column E */
int moe_combine_backward(const moe_shape* shape, const void* dout, const void* y_perm,
                         const int32_t* slot_of, const int32_t* topk_idx, const float* topk_w,
                         const float* logits, const float* aux_coef, void* dy_perm, float* dz,
                         void* dz_bf16, void* stream);

/* dh = dy W_d per expert (the shared expert's dy is dout), then the SwiGLU
 * backward dg = dh u silu'(g), du = dh silu(g).
 *   w_down_t [E, F, D], ws_down_t [Fs, D]: packed transposed down weights
 *   gu from moe_grouped_gate_up_train
 *   dh [S, F] + [T, Fs] bf16 out (intermediate); dgu [S, 2F] + [T, 2Fs] bf16 out */
int moe_grouped_backward_h(const moe_shape* shape, const void* dy_perm, const void* dout,
                           const int32_t* offsets, const void* w_down_t, const void* ws_down_t,
                           const void* gu, void* dh, void* dgu, void* stream);

/* Input gradient: dx_perm = [dg | du] [W_g; W_u] per routed row, dx_shared the
 * same for the shared expert, dx_router = dz W_r, then
 *   dx_t = dx_shared_t + dx_router_t + sum over t's routed slots of dx_perm rows.
 *   w_gate_up_t [E, D, 2F], ws_gate_up_t [D, 2Fs], w_router_t [D, 256]: packed
 *   transposed; dx_perm [S, D], dx_shared [T, D] (unused when Fs == 0),
 *   dx_router [T, D], dx [T, D]: bf16 out */
int moe_grouped_backward_x(const moe_shape* shape, const void* dgu, const int32_t* offsets,
                           const void* w_gate_up_t, const void* ws_gate_up_t, const void* dz_bf16,
                           const void* w_router_t, const int32_t* slot_of, void* dx_perm, void* dx_shared,
                           void* dx_router, void* dx, void* stream);

/* Weight gradients, each a sum over the group's token rows (zero for an expert
 * without rows; T == 0 writes zeros and reads no input):
 *   dw_gate_up [E, 2F, D] bf16 = [dg | du]^T x of the expert's rows
 *   dw_down    [E, D, F]  bf16 = dy^T h
 *   dws_gate_up [2Fs, D], dws_down [D, Fs] bf16: the shared expert over all T
 *              rows (dy = dout); unused when Fs == 0
 *   dw_router  [E, D] fp32 = dz^T x (from dz_bf16), or NULL to skip
 *   x_perm may be NULL (rows then come from x through sorted_token). */
int moe_weight_grads(const moe_shape* shape, const void* x, const int32_t* sorted_token,
                     const void* x_perm, const int32_t* offsets, const void* dgu, const void* dy_perm,
                     const void* dout, const void* h, const void* dz_bf16, void* dw_gate_up, void* dw_down,
                     void* dws_gate_up, void* dws_down, float* dw_router, void* stream);

/* Router bias gradient: dbias [E] fp32 = sum over tokens of dz [T, E] (fp32,
 * from moe_combine_backward), summed in a fixed order.
 *   workspace >= moe_train_workspace_bytes */
int moe_bias_grad(const moe_shape* shape, const float* dz, float* dbias, void* workspace,
                  size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
