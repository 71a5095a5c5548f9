/*
 * libmoe -- the forward and backward pass of one Mixture-of-Experts (MoE) layer on AMD
 * MI355X (gfx950).
 *
 * Each token's hidden state is gated to its top-k experts (or routed by replayed
 * expert IDs), the (token, slot) pairs are counting-sorted into contiguous
 * per-expert segments, every segment runs through its expert's SwiGLU FFN as one
 * grouped GEMM, and the k expert outputs of each token are combined by a
 * fixed-order weighted sum.  Every reduction in the library has one fixed order and
 * no floating-point atomics, so results are bitwise reproducible and do not depend
 * on which other tokens share the batch or on the order of the tokens.
 *
 * Sources of the operations (page title, then section):
 *   - gate picks 8 of 384 experts per token and layer; a tiny hidden-state
 *     difference can flip the choice: Training Data podcast page "How Cursor Trained
 *     Composer on Fireworks" (Chinese rewrite), section on floating point and MoE;
 *     same facts on the page "Cursor 訓練 Composer 2 的五大工程挑戰", section
 *     "浮點數的陷阱".  Both pages also describe fixed-order (batch-invariant)
 *     kernels as the cure for train/inference mismatch.
 *   - router replay (IDs from inference override the router; gate scores are still
 *     computed): Composer 2 Technical Report, section 6.2, paragraph on inference
 *     and weight sync.
 *   - grouped-GEMM MoE flow: Composer 2 Technical Report, section 6.1 "Kernels",
 *     Figure 10; token dispatch/combine with MXFP8 tokens before dispatch and a BF16
 *     combine: section 6.1 "Parallelism".
 *   - MXFP8 = E4M3 elements with one E8M0 scale per 32-element block: section 6.1
 *     "Kernels" (backward-pass format), OCP Microscaling Formats v1.0.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers to row-major arrays owned by the
 *     caller; the library never allocates, frees or synchronises, except in
 *     moe_check.  Every call enqueues its kernels asynchronously on `stream`
 *     (a hipStream_t; NULL = the default stream) and returns.
 *   - Host-side argument validation happens before any launch; on any status other
 *     than MOE_OK nothing was enqueued by that call (MOE_ERR_HIP: a launch failed).
 *   - Device-detected errors (bad replayed IDs, non-finite logits) are OR-ed into a
 *     flag in the workspace header and reported by moe_check.  Results of a call
 *     are defined only if moe_check reports MOE_OK afterwards.
 *   - Calls that share one workspace must be ordered on one stream: calls that
 *     overlap on the same workspace race.
 *   - dtype (moe_dtype) names the storage of activations and expert weights:
 *       MOE_F32   : fp32 x, fp32 weights, fp32 intermediate, fp32 outputs.
 *       MOE_BF16  : bf16 x, bf16 weights, fp32 accumulation, bf16 intermediate
 *                   h = silu(x W1) * (x W3) and bf16 expert outputs and y.
 *       MOE_MXFP8 : OCP MXFP8 x and weights (uint8 E4M3 codes plus one uint8 E8M0
 *                   scale per 32 consecutive elements of the contiguous dimension),
 *                   fp32 accumulation, bf16 expert outputs and y.
 *       MOE_NVFP4 : the NVFP4 forward (Composer 2 Technical Report, section 6.1
 *                   "Kernels"): bf16 x and y, NVFP4 expert weights; the expert FFN
 *                   quantizes x per token and h per row to NVFP4 (E2M1 values, one
 *                   E4M3 scale per 16 elements, one fp32 scale per row).  Only the
 *                   expert-FFN calls take MOE_NVFP4; routing, dispatch and combine of
 *                   such a layer take MOE_BF16 (their tensors are bf16).
 *   - Expert weight layout (per expert, output-major, reduction dimension
 *     contiguous): w1, w3 [I][d] and w2 [d][I]; i.e. the mathematical W1 [d x I]
 *     is stored transposed.  A bank of n experts is n such matrices back to back.
 *   - The gate weight is fp32 [d][E] (expert index contiguous), the optional
 *     per-expert logit bias fp32 [E].
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer, bad dtype */
  MOE_ERR_UNSUPPORTED = 2, /* valid request this build does not implement (shape/dtype) */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes is smaller than moe_workspace_size() requires */
  MOE_ERR_BAD_IDS = 4,     /* (moe_check) an expert id was out of range or repeated in a row */
  MOE_ERR_NONFINITE = 5,   /* (moe_check) a gate logit was NaN or infinite */
  MOE_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2, MOE_NVFP4 = 3 } moe_dtype;

/* One bank of SwiGLU experts (n experts stored back to back; see layout above).
 * The *_scale pointers are the E8M0 scales for MOE_MXFP8 ([n][I][d/32] for w1/w3,
 * [n][d][I/32] for w2), the E4M3 block scales for MOE_NVFP4, and must be NULL for the
 * other dtypes.  MOE_NVFP4 weights are E2M1 codes two per byte (element 2i in the low
 * nibble) with one E4M3 scale per 16 elements of a row and one fp32 scale per row in
 * *_rscale ([n][I], [n][I], [n][d]); codes and block scales are K-blocked, as
 * moe_nvfp4_pack_weights writes them from the row-major form (codes [R][K/2], scales
 * [R][K/16] per matrix of R rows: I rows of d for w1/w3, d rows of I for w2). */
typedef struct {
  const void* w1;
  const void* w3;
  const void* w2;
  const uint8_t* w1_scale;
  const uint8_t* w3_scale;
  const uint8_t* w2_scale;
  const float* w1_rscale;   /* MOE_NVFP4 only (else NULL): fp32 scale per weight row */
  const float* w3_rscale;
  const float* w2_rscale;
} moe_expert_bank;

/* Size in bytes of the workspace that every call below accepts for a layer with
 * T tokens, hidden size d, E routed experts, top-k, expert intermediate size
 * `inter` and storage dtype.  One workspace serves every call of the layer.
 * Returns MOE_ERR_INVALID_ARG for out-of-range sizes (T < 0, d < 1, E outside
 * [1, 1024], k outside [1, min(E, 32)], inter < 1) or a null `bytes`. */
moe_status moe_workspace_size(int T, int d, int E, int k, int inter, int dtype, size_t* bytes);

/* Clears the workspace header (the device error flag).  Call once after
 * allocating a workspace, before its first use. */
moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Learned routing: gate GEMM, softmax over the E experts, top-k, renormalise.
 * Defined by: a gating layer picks 8 of 384 experts for each token in each MoE layer,
 * and a hidden-state difference in the fifth decimal can change the pick (Training
 * Data podcast page "How Cursor Trained Composer on Fireworks", section on floating
 * point and MoE; page "Cursor 訓練 Composer 2 的五大工程挑戰", section "浮點數的陷阱").
 * The pages name neither the gating function nor a tie rule: softmax, top-k with ties
 * to the lower index, and renormalisation are this library's reading.
 *   x       [T][d] activations in `dtype` (x_scale [T][d/32] E8M0 for MOE_MXFP8,
 *           else NULL; the gate reads the exact dequantised values).
 *   w_gate  fp32 [d][E], 16-byte aligned when E % 4 == 0 (else 4-byte aligned);
 *           bias fp32 [E] or NULL (added to the logits used for both the selection
 *           and the weights).
 *   ids     out int32 [T][k]: the k experts with the largest logits, ordered by
 *           (logit descending, expert index ascending).  The selection equals the
 *           one made on the exactly rounded logits.  A first pass with a rigorous
 *           per-logit error bound (the fp64 gate GEMM for fp32 activations and small
 *           batches; for large bf16 / MXFP8 batches a bf16 matrix-core screen over an
 *           exact three-way bf16 split of w_gate, followed by fp64 logits of the
 *           experts the screen cannot exclude) decides every token it can certify;
 *           the other tokens are recomputed with exact (error-free) summation on the
 *           device.
 *   weights out fp32 [T][k]: softmax probabilities of the chosen experts
 *           renormalised to sum to one (computed in fp64 from the fp64 logits,
 *           rounded once), in the same column order as ids.
 * Every logit is summed in one fixed order that depends on d only (not on T or on
 * the other tokens), so a token's ids and weights are the same in every batch.
 * Sets MOE_ERR_NONFINITE in the device flag if any logit of a token is not finite.
 * MOE_ERR_INVALID_ARG: misaligned x or w_gate.  MOE_ERR_UNSUPPORTED: d % 16 != 0.
 * T == 0 is a valid no-op. */
moe_status moe_route(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                     const float* w_gate, const float* bias, int E, int k,
                     int32_t* ids, float* weights,
                     void* ws, size_t ws_bytes, void* stream);

/* Router replay: the caller's expert IDs override the router's choice.  The gate
 * logits are still computed (as in moe_route).
 *   ids_in      int32 [T][k]: replayed expert IDs; each must lie in [0, E) and be
 *               distinct within its row, else the device flag gets MOE_ERR_BAD_IDS.
 *               Column order is the combine's rank order.
 *   weights_in  fp32 [T][k] used verbatim, or NULL: then the weights are the gate's
 *               softmax probabilities at ids_in renormalised to sum to one, with
 *               exactly the arithmetic moe_route uses, so replaying moe_route's own
 *               ids reproduces its weights bit for bit.
 *   weights_out fp32 [T][k]. */
moe_status moe_route_replay(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                            const float* w_gate, const float* bias, int E, int k,
                            const int32_t* ids_in, const float* weights_in, float* weights_out,
                            void* ws, size_t ws_bytes, void* stream);

/* Router replay with the plausibility filter (Composer 2 Technical Report, section
 * 6.2, paragraph on inference and weight sync: replayed experts whose gate score
 * falls below a threshold derived from the router's own top-k are dropped and
 * replaced with the router's candidates).  The page fixes neither the score nor the
 * threshold; here the score is the gate's softmax probability p_e and the threshold
 * tau * p_(k), p_(k) being the probability of the router's own k-th choice.  The
 * test runs in logit form on the exactly rounded logits:
 *     replayed column j keeps its expert e  iff  fl(l_e - l_(k)) >= log_tau
 * (l = the correctly rounded fp64 logits, the difference rounded once), decided on
 * the device by an fp64 bound and, where that bound cannot separate the two sides,
 * by exact summation, so the kept set equals the one made on exact logits.
 *   ids_in      int32 [T][k]: replayed expert IDs, in [0, E) and distinct within a
 *               row, else the device flag gets MOE_ERR_BAD_IDS (that row's output is
 *               then the router's own choice).  Must not overlap ids_out.
 *   log_tau     ln tau, not NaN.  -INFINITY keeps every replayed id (plain replay);
 *               +INFINITY drops them all (learned routing); 0 keeps exactly the
 *               replayed experts at least as likely as the router's k-th choice.
 *   ids_out     out int32 [T][k]: kept columns hold the replayed id; dropped
 *               columns, in column order, get the router's top-k ids in rank order
 *               (as moe_route orders them) that no kept column holds.
 *   weights_out out fp32 [T][k]: the gate's softmax probabilities at ids_out
 *               renormalised, with exactly moe_route_replay's arithmetic (so
 *               log_tau = -INFINITY reproduces moe_route_replay bit for bit, and
 *               +INFINITY reproduces moe_route).
 * Runs moe_route first (same workspace).  MOE_ERR_INVALID_ARG: NaN log_tau,
 * overlapping ids_in / ids_out, or as moe_route. */
moe_status moe_route_replay_filtered(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                     const float* w_gate, const float* bias, int E, int k,
                                     const int32_t* ids_in, double log_tau, int32_t* ids_out,
                                     float* weights_out, void* ws, size_t ws_bytes, void* stream);

/* Counting sort of the T*k (token, slot) pairs by (expert ascending, token
 * ascending), the grouped GEMM's input order.  Positions come from deterministic
 * histograms and prefix sums, never from atomic position counters.
 * Defined by: tokens are dispatched to their experts and the expert outputs combined
 * back (Composer 2 Technical Report, section 6.1 "Parallelism", DeepEP dispatch and
 * combine), and each expert's tokens form one group of the grouped GEMM (section 6.1
 * "Kernels", Figure 10).  Here the dispatch is local to one GPU.
 *   ids     int32 [T][k] (from moe_route or replayed).  An id outside [0, E) sets
 *           MOE_ERR_BAD_IDS and is treated as expert 0 so every output stays a
 *           valid permutation.
 *   offsets out int32 [E+1]: segment e is sorted rows offsets[e] .. offsets[e+1]-1.
 *   perm    out int32 [T*k]: perm[j] = t*k + r of sorted row j.
 *   row_of  out int32 [T*k]: row_of[t*k + r] = j (inverse of perm). */
moe_status moe_dispatch(const int32_t* ids, int T, int E, int k,
                        int32_t* offsets, int32_t* perm, int32_t* row_of,
                        void* ws, size_t ws_bytes, void* stream);

/* moe_dispatch for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * the same results, with the scratch (per-block histograms, expert totals and the error
 * flag) in a library-owned static device array of 4 MiB instead of a caller workspace.
 * The array exists once per GPU and is held until the process ends; the call itself
 * allocates nothing.  Arguments as moe_dispatch, plus
 *   status_out  device int32 or NULL: receives MOE_OK, or MOE_ERR_BAD_IDS when an id
 *               was outside [0, E) (treated as expert 0, as moe_dispatch does), once the
 *               call's kernels have run (no host synchronisation).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, two threads) race, and must be ordered by the caller.  The caller's device
 * must be current (hipSetDevice) and own `stream`.
 * MOE_ERR_UNSUPPORTED when the scratch would exceed 4 MiB: it takes 256 bytes plus
 * (ceil(T / 64) + 1) * E * 4 bytes, each part rounded up to 256 bytes (up to 174,656
 * tokens at E = 384, 65,408 at E = 1024); MOE_ERR_HIP when the array's device address
 * cannot be obtained.  Other argument checks as moe_dispatch. */
moe_status moe_dispatch_noalloc(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                                int32_t* perm, int32_t* row_of, int32_t* status_out, void* stream);

/* Grouped SwiGLU expert FFN over the dispatched segments (one grouped GEMM for
 * W1 and W3 with the SwiGLU epilogue, one for W2).
 * Defined by: the MoE layer runs its experts as grouped GEMMs, with MXFP8 (E4M3
 * values, one E8M0 scale per 32) or NVFP4 operands (Composer 2 Technical Report,
 * section 6.1 "Kernels", Figure 10).  The expert's form (SwiGLU) and the shared expert
 * are not on the pages; they are this library's workload.
 *   x        [T][d] activations in `dtype` (x_scale as in moe_route); rows are
 *            gathered through perm inside the GEMM (no separate permuted copy).
 *   routed   bank of E experts; shared: bank of 1 always-on expert, or NULL.
 *   offsets, perm from moe_dispatch.
 *   out      [T*k + (shared ? T : 0)][d]: row j < T*k is expert(j)'s output for the
 *            pair perm[j]; row T*k + t is the shared expert's output for token t.
 *            fp32 for MOE_F32, bf16 otherwise.
 * Per output element the reduction order is fixed (same instruction sequence for
 * every row of every segment), so a token's output row does not depend on which
 * other tokens share its expert.
 * For MOE_MXFP8 the intermediate h is requantised to MXFP8 per row (one E8M0
 * scale per 32 columns: the smallest power of two that maps the block's largest
 * magnitude to at most 448, so no element saturates; E4M3 elements rounded to
 * nearest even) before the W2 GEMM, so it is consumed by the same block-scaled MFMA.
 * For MOE_NVFP4, x is quantized per token and h per row to NVFP4 (the quantizer of
 * moe_nvfp4_quantize) before their GEMMs; both GEMMs run on the decoded values (E2M1
 * times E4M3, exact in fp16) with fp32 accumulation, and the two operands' fp32 row
 * scales multiply the accumulator.
 * MOE_ERR_UNSUPPORTED: MOE_BF16 needs d % 128 == 0 and inter % 64 == 0;
 * MOE_MXFP8 needs d % 128 == 0 and inter % 128 == 0; MOE_NVFP4 needs d % 256 == 0 and
 * inter % 128 == 0.
 * MOE_ERR_INVALID_ARG: x or a weight pointer not 16-byte aligned (bf16, MXFP8,
 * NVFP4), or an MXFP8 or NVFP4 scale pointer not 4-byte aligned. */
moe_status moe_expert_ffn(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                          int E, int k, int inter,
                          const moe_expert_bank* routed, const moe_expert_bank* shared,
                          const int32_t* offsets, const int32_t* perm, void* out,
                          void* ws, size_t ws_bytes, void* stream);

/* The two halves of moe_expert_ffn, for callers that schedule or time them apart
 * (same kernels, same results).  moe_expert_ffn_gate_up builds the segment table and
 * runs the W1/W3 grouped GEMM with the SwiGLU epilogue, leaving h in the workspace;
 * moe_expert_ffn_down runs the W2 grouped GEMM on that h and table and writes `out`.
 * The down call must follow a gate_up call with the same shape arguments and banks
 * on the same workspace and stream, with no other call on that workspace between. */
moe_status moe_expert_ffn_gate_up(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                  int E, int k, int inter,
                                  const moe_expert_bank* routed, const moe_expert_bank* shared,
                                  const int32_t* offsets, const int32_t* perm,
                                  void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_ffn_down(int dtype, int T, int d, int E, int k, int inter,
                               const moe_expert_bank* routed, const moe_expert_bank* shared,
                               void* out, void* ws, size_t ws_bytes, void* stream);

/* Defined by: the combine of the expert outputs is kept in BF16 (Composer 2 Technical
 * Report, section 6.1 "Parallelism"), and batch-invariant kernels sum in one fixed
 * order so inference and training agree bit for bit (both podcast pages, sections on
 * floating point and MoE).
 * Fixed-order combine: y[t] = round( (...((w[t,0]*O0 + w[t,1]*O1) + ...) + w[t,k-1]*O_{k-1})
 * + S[t] ) with O_r = out[row_of[t*k + r]] and S[t] = out[T*k + t] when has_shared;
 * fp32 fused multiply-adds in rank order r = 0..k-1, shared output last, one final
 * rounding to the output dtype.  No atomics.
 *   out      expert outputs from moe_expert_ffn (fp32 for MOE_F32, else bf16).
 *   weights  fp32 [T][k]; y out [T][d] (fp32 for MOE_F32, else bf16).
 * Requires d % 8 == 0. */
moe_status moe_combine(const void* out, int dtype, const int32_t* row_of, const float* weights,
                       int T, int d, int k, int has_shared, void* y, void* stream);

/* ------------------------------------------------------------------------------
 * Backward pass.  The MoE layer is trained as one grouped-GEMM flow forward and
 * backward (Composer 2 Technical Report, section 6.1 "Kernels", Figure 10), and under
 * router replay the router still computes gate scores so that gradients can flow
 * through them (section 6.2, paragraph on inference and weight sync).  Given dL/dy,
 * the four calls below give dL/dx, the expert weights' gradients and the gate's:
 *   moe_combine_backward -> moe_expert_ffn_backward -> moe_route_backward.
 * The expert selection is piecewise constant, so no gradient flows through the ids.
 * Every reduction has one fixed order (no atomics): results are bitwise reproducible.
 * ------------------------------------------------------------------------------ */

/* moe_expert_ffn_gate_up that also keeps the pre-activations for the backward pass:
 * pre out fp32 [T*k (+T)][2*inter], row j = (x W1, x W3) of dispatched row j, exactly the
 * values the SwiGLU epilogue uses (bf16, MXFP8 and NVFP4 layers, for NVFP4 with both row
 * scales applied; MOE_ERR_UNSUPPORTED for fp32).
 * Same results as moe_expert_ffn_gate_up; pass `pre` to moe_expert_ffn_backward (bf16) or
 * moe_expert_ffn_backward_mxfp8. */
moe_status moe_expert_ffn_gate_up_save(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                       int E, int k, int inter, const moe_expert_bank* routed,
                                       const moe_expert_bank* shared, const int32_t* offsets,
                                       const int32_t* perm, float* pre, void* ws, size_t ws_bytes,
                                       void* stream);

/* NVFP4 quantization of the rows of a bf16 matrix [rows][K] (K % 16 == 0): per row
 * s = amax / 2688, per block of 16 S = E4M3_RNE((bamax / s) / 6), per element
 * E2M1_RNE(v / (S s)), each step one IEEE fp32 operation rounded to nearest even,
 * saturating (a zero row has s = 0 and zero codes).  codes out [rows][K/2] (two per
 * byte, element 2i in the low nibble, 8-byte aligned), block_scales out [rows][K/16]
 * (E4M3 codes), row_scales out fp32 [rows].  src 16-byte aligned. */
moe_status moe_nvfp4_quantize(const void* src, int rows, int K, uint8_t* codes,
                              uint8_t* block_scales, float* row_scales, void* stream);

/* K-blocking of n NVFP4 weight matrices of R rows x K columns (R % 32 == 0,
 * K % 64 == 0), the layout moe_expert_bank takes for MOE_NVFP4: from row-major codes
 * [n][R][K/2] and block scales [n][R][K/16] to packed_codes [n][R/32][K/64][32][32]
 * (tile of rows 32 g .. 32 g + 31 and columns 64 s .. 64 s + 63: row r's 32 code bytes,
 * unchanged, at 32 r) and packed_scales [n][R/32][K/64][32][4] (row r's 4 block scales
 * at 4 r).  A pure permutation of bytes; same sizes as the inputs.  codes and
 * packed_codes 16-byte aligned, the scales 4-byte aligned, outputs must not overlap the
 * inputs or each other (MOE_ERR_INVALID_ARG). */
moe_status moe_nvfp4_pack_weights(const uint8_t* codes, const uint8_t* block_scales, int n, int R, int K,
                                  uint8_t* packed_codes, uint8_t* packed_scales, void* stream);

/* Gradients of one expert bank, fp32, in the bank's layout: dw1, dw3 [n][I][d],
 * dw2 [n][d][I]; 16-byte aligned. */
typedef struct {
  float* dw1;
  float* dw3;
  float* dw2;
} moe_grad_bank;

/* Workspace bytes for the forward calls and the backward calls of one layer shape
 * (at least moe_workspace_size).  Same argument checks as moe_workspace_size. */
moe_status moe_backward_workspace_size(int T, int d, int E, int k, int inter, int dtype, size_t* bytes);

/* Backward of moe_combine for y_t = sum_r w_tr out[row_of[t,r]] (+ out[T k + t]).
 *   dy        [T][d] dL/dy in the layer's output type (bf16; fp32 for MOE_F32).
 *   out       the expert outputs moe_expert_ffn produced, [T*k (+T)][d].
 *   d_out     out [T*k (+T)][d], same type: d_out[row_of[t,r]] = w_tr * dy_t (fp32
 *             product, rounded once); with has_shared, d_out[T*k + t] = dy_t.
 *   d_weights out fp32 [T][k]: dL/dw_tr = <dy_t, out[row_of[t,r]]>, an fp32 sum in one
 *             fixed order that depends on d only.
 * MOE_ERR_UNSUPPORTED: d % 8 != 0.  Pointers to 16-byte aligned rows. */
moe_status moe_combine_backward(const void* dy, int dtype, const void* out, const int32_t* row_of,
                                const float* weights, int T, int d, int k, int has_shared,
                                void* d_out, float* d_weights, void* stream);

/* Backward of moe_expert_ffn (bf16 layers; MOE_ERR_UNSUPPORTED for other dtypes and
 * unless d % 128 == 0 and inter % 128 == 0).  Arguments x .. perm as moe_expert_ffn.
 *   pre       the pre-activations moe_expert_ffn_gate_up_save kept, or NULL: then they
 *             are recomputed (same values, bit for bit; one more pass over W1 and W3).
 *   d_out     bf16 [T*k (+T)][d] from moe_combine_backward.
 *   dx_rows   out fp32 [T*k (+T)][d]: each dispatched row's dL/dx, da W1 + dg W3 with
 *             a = x W1, g = x W3 recomputed as the forward computes them, dh = d_out W2,
 *             da = dh g silu'(a), dg = dh silu(a) (fp32, rounded to bf16 for the GEMMs).
 *   routed_grads, shared_grads  out (moe_grad_bank): dW1 = da^T x, dW3 = dg^T x,
 *             dW2 = d_out^T h per expert over its rows (h = the forward's bf16 h), every
 *             expert written (zero when it got no rows).  shared_grads is NULL iff
 *             shared is NULL.
 *   ws        sized by moe_backward_workspace_size. */
moe_status moe_expert_ffn_backward(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                   int E, int k, int inter, const moe_expert_bank* routed,
                                   const moe_expert_bank* shared, const int32_t* offsets,
                                   const int32_t* perm, const float* pre, const void* d_out,
                                   float* dx_rows,
                                   const moe_grad_bank* routed_grads,
                                   const moe_grad_bank* shared_grads, void* ws, size_t ws_bytes,
                                   void* stream);

/* The two halves of moe_expert_ffn_backward, for callers that overlap or time them
 * apart (same arguments, same results).  The data half computes dx_rows and leaves
 * da | dg, h and the segment table in the workspace; the weights half then writes
 * the weight gradients from them (call it next on the same workspace and stream). */
moe_status moe_expert_ffn_backward_data(const void* x, const uint8_t* x_scale, int dtype, int T,
                                        int d, int E, int k, int inter,
                                        const moe_expert_bank* routed, const moe_expert_bank* shared,
                                        const int32_t* offsets, const int32_t* perm, const float* pre,
                                        const void* d_out, float* dx_rows, void* ws, size_t ws_bytes,
                                        void* stream);
moe_status moe_expert_ffn_backward_weights(const void* x, int dtype, int T, int d, int E, int k,
                                           int inter, const moe_expert_bank* routed,
                                           const moe_expert_bank* shared, const int32_t* perm,
                                           const void* d_out, const moe_grad_bank* routed_grads,
                                           const moe_grad_bank* shared_grads, void* ws,
                                           size_t ws_bytes, void* stream);

/* The expert weights of an MXFP8 layer requantised for the backward's data-gradient
 * GEMMs, whose reductions run along the other axis of each weight (Composer 2
 * Technical Report, section 6.1 "Kernels": the MoE backward in MXFP8, one E8M0 scale
 * per 32 elements of the reduction):
 *   w2t  [n][I][d] E4M3 codes, w2t_scale [n][I][d/32]: row c of expert e is column c of
 *        W2[e] (over d), quantised along d;
 *   w13t [n][d][2I] codes, w13t_scale [n][d][2I/32]: row i of expert e is column i of
 *        W1[e] (over I), then column i of W3[e], quantised along I.
 * Scales are the smallest power of two that maps a block's largest magnitude to at most
 * 448; elements round to the nearest E4M3 value, ties to even.  Codes 16-byte aligned,
 * scales 4-byte aligned. */
typedef struct {
  uint8_t* w2t;
  uint8_t* w2t_scale;
  uint8_t* w13t;
  uint8_t* w13t_scale;
} moe_mxfp8_tbank;

/* Writes the requantised weights of an MXFP8 bank of n experts (w1, w3 [n][I][d] and w2
 * [n][d][I] with their E8M0 scales, as moe_expert_bank holds them) into `out`; call once
 * per weight version.  Requires d % 128 == 0 and inter % 128 == 0 (else
 * MOE_ERR_UNSUPPORTED); MOE_ERR_INVALID_ARG for missing or misaligned pointers. */
moe_status moe_mxfp8_transpose_weights(const moe_expert_bank* bank, int n, int d, int inter,
                                       const moe_mxfp8_tbank* out, void* stream);

/* Backward of moe_expert_ffn for MXFP8 layers, with every backward GEMM on the
 * block-scaled matrix cores and both of its operands in MXFP8 blocked along its own
 * reduction dimension (Composer 2 Technical Report, section 6.1 "Kernels", Figure 10):
 *   dh = MX_row(d_out) . MX_d(W2)^T, da = dh g silu'(a), dg = dh silu(a),
 *   dx_rows = MX_row(da | dg) . MX_I(W1 | W3)^T        (row-local: a token's dx rows do
 *                                                     not depend on the other tokens),
 *   dW2 = MX_rows(d_out)^T MX_rows(hq), dW1 | dW3 = MX_rows(da | dg)^T MX_rows(x)
 * where MX_row quantises each row, MX_rows quantises along the expert's rows in blocks
 * of 32 from its first row (zero-padded), and hq is the forward's MXFP8 h (recomputed
 * from the pre-activations with the forward's arithmetic).
 *   x, x_scale   the layer's MXFP8 activations [T][d] and scales [T][d/32].
 *   routed, shared, offsets, perm  as moe_expert_ffn; routed_t, shared_t: the banks'
 *                requantised weights (moe_mxfp8_transpose_weights); shared_t NULL iff
 *                shared is NULL.
 *   pre          fp32 [T*k (+T)][2*inter] from moe_expert_ffn_gate_up_save, or NULL:
 *                then recomputed with the forward's GEMM (one more pass over W1, W3).
 *   d_out        bf16 [T*k (+T)][d] from moe_combine_backward.
 *   dx_rows      out fp32 [T*k (+T)][d]; routed_grads, shared_grads out fp32, as
 *                moe_expert_ffn_backward (every expert written, zero without rows).
 *   ws           sized by moe_backward_workspace_size(..., MOE_MXFP8).
 * MOE_ERR_UNSUPPORTED unless d % 128 == 0 and inter % 128 == 0. */
moe_status moe_expert_ffn_backward_mxfp8(const void* x, const uint8_t* x_scale, int T, int d, int E,
                                         int k, int inter, const moe_expert_bank* routed,
                                         const moe_expert_bank* shared,
                                         const moe_mxfp8_tbank* routed_t,
                                         const moe_mxfp8_tbank* shared_t, const int32_t* offsets,
                                         const int32_t* perm, const float* pre, const void* d_out,
                                         float* dx_rows, const moe_grad_bank* routed_grads,
                                         const moe_grad_bank* shared_grads, void* ws,
                                         size_t ws_bytes, void* stream);

/* The MXFP8 backward (moe_expert_ffn_backward_mxfp8) of a layer whose forward ran in
 * NVFP4 (Composer 2 Technical Report, section 6.1 "Kernels": an NVFP4 forward paired with
 * an MXFP8 backward).  The backward GEMMs take the forward's operands as the forward
 * quantized them: the weights' NVFP4 values, x quantized per token and h per row to
 * NVFP4 (recomputed from `pre` with the forward's arithmetic), each requantised to MXFP8
 * along the backward GEMM's reduction.
 *   x          the layer's bf16 activations [T][d]; routed, shared: the K-blocked NVFP4
 *              banks the forward took; routed_t, shared_t: moe_nvfp4_transpose_weights.
 *   pre        required: fp32 [T*k (+T)][2*inter] from moe_expert_ffn_gate_up_save with
 *              MOE_NVFP4 (x W1, x W3 with both row scales applied).
 * Other arguments and results as moe_expert_ffn_backward_mxfp8; ws sized by
 * moe_backward_workspace_size(..., MOE_NVFP4).  MOE_ERR_UNSUPPORTED unless
 * d % 256 == 0 and inter % 128 == 0. */
moe_status moe_expert_ffn_backward_nvfp4(const void* x, int T, int d, int E, int k, int inter,
                                         const moe_expert_bank* routed, const moe_expert_bank* shared,
                                         const moe_mxfp8_tbank* routed_t,
                                         const moe_mxfp8_tbank* shared_t, const int32_t* offsets,
                                         const int32_t* perm, const float* pre, const void* d_out,
                                         float* dx_rows, const moe_grad_bank* routed_grads,
                                         const moe_grad_bank* shared_grads, void* ws,
                                         size_t ws_bytes, void* stream);

/* moe_mxfp8_transpose_weights for a K-blocked NVFP4 bank (moe_nvfp4_pack_weights):
 * w2t and w13t as there, requantised to MXFP8 from the exact NVFP4 values (E2M1 x E4M3 x
 * row scale).  Requires d % 256 == 0 and inter % 128 == 0. */
moe_status moe_nvfp4_transpose_weights(const moe_expert_bank* bank, int n, int d, int inter,
                                       const moe_mxfp8_tbank* out, void* stream);

/* Backward of the routing and of the token gather.
 *   dx        out fp32 [T][d]: sum_r dx_rows[row_of[t,r]] (r ascending), plus
 *             dx_rows[T*k + t] when has_shared, plus the gate term below.
 *   d_w_gate  out fp32 [d][E], or NULL when the routing weights did not come from the
 *             gate (replay with caller weights): then the gate gets no gradient and dx
 *             no gate term.  With the gate's weights w = softmax over the chosen ids,
 *             renormalised: dl_tr = w_tr (d_weights_tr - sum_s w_ts d_weights_ts),
 *             d_w_gate[:, e] = sum over expert e's rows of dl x_t (token ascending),
 *             dx_t += sum_r dl_tr w_gate[:, ids_tr].
 *   d_bias    out fp32 [E] (sum of dl per expert) or NULL; requires d_w_gate.
 *   ids, weights, d_weights [T][k]; offsets, perm, row_of from moe_dispatch;
 *   x as moe_route (read only for d_w_gate; MOE_ERR_INVALID_ARG if it is not 16-byte
 *   aligned then).  ws: moe_backward_workspace_size.  MOE_ERR_UNSUPPORTED: d % 4. */
moe_status moe_route_backward(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                              const float* w_gate, int E, int k, const int32_t* ids,
                              const float* weights, const float* d_weights, const int32_t* offsets,
                              const int32_t* perm, const int32_t* row_of, const float* dx_rows,
                              int has_shared, float* dx, float* d_w_gate, float* d_bias, void* ws,
                              size_t ws_bytes, void* stream);

/* Synchronises `stream`, reads and clears the workspace's device error flag and
 * returns MOE_ERR_BAD_IDS, MOE_ERR_NONFINITE or MOE_OK. */
moe_status moe_check(void* ws, size_t ws_bytes, void* stream);

/* Static string naming a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_MOE_H */
