/*
 * moe.h -- C ABI of the MI355X (gfx950) token-choice top-k Mixture-of-Experts
 * FFN layer: routing, token permutation, grouped SwiGLU expert GEMMs, weighted
 * combine, and the backward pass.
 *
 * What the layer computes (sources are the pages this library follows):
 *   - "Beam" blog (hncyxsy.com), sections 2.2 and 5.3: the MoE layer replaces a
 *     transformer FFN; a router (d_model x N matrix, nn.Linear without bias)
 *     scores every expert, the top-k experts of each token run, and the output
 *     is the gate-weighted sum of their outputs; the gates are a softmax over
 *     the k selected logits.
 *   - "Trinity Large" commentary (ai-stack.site), code examples 1-3: top-k then
 *     softmax; per-expert counts; dispatch to per-expert buffers and combine.
 *   - Olmo-core 3 article (pwwt.cn), "three splits" section: tokens are written
 *     straight into contiguous per-expert input buffers, routing stays resident
 *     on the GPU (the host never waits for routing metadata), the expert GEMMs
 *     are grouped, and MXFP8 is a precision switch for them.
 *   - SonicMoE article (techwalker.com), section 1: the router-score gradient is
 *     dS = <dA', A> (not <dO, Y>), so expert outputs Y are never stored;
 *     section 3: token rounding of per-expert counts to the GEMM tile.
 *
 * Expert e is a SwiGLU FFN without biases: h = W1_e x (W1_e = [W_gate; W_up],
 * [2f, d], gate rows first), a = silu(h_gate) * h_up, y = W2_e a (W2_e [d, f]).
 *
 * Conventions (all entry points):
 *   - Every data pointer is a DEVICE pointer owned by the caller, row-major,
 *     16-byte aligned.  The library never allocates or frees device memory and
 *     keeps no global mutable state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it and return; there is no device-to-host copy
 *     or synchronisation anywhere.  Routing-dependent sizes stay in device
 *     memory (plan.offsets etc.); kernels read them there.
 *   - Validation happens on the host before anything is enqueued: on any error
 *     nothing is launched.  MOE_EHIP reports a failed kernel launch; faults that
 *     happen asynchronously on the device surface at the caller's next sync.
 *   - Results are bitwise reproducible run to run (no floating-point atomics).
 *   - Concurrent calls on different streams need separate plan and workspace
 *     buffers.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,     /* null/misaligned pointer, non-positive size, k > E, bad dtype mix */
  MOE_ENOTSUP = 2,    /* shape outside what the kernels support (see moe_shape) */
  MOE_EWORKSPACE = 3, /* workspace or plan blob smaller than the *_bytes() query */
  MOE_EHIP = 4        /* a kernel launch failed */
} moe_status;

typedef enum {
  MOE_F32 = 0,   /* IEEE float32 */
  MOE_BF16 = 1,  /* bfloat16, round-to-nearest-even on every store */
  MOE_MXFP8 = 2  /* expert-GEMM operands only: FP8 E4M3 + one E8M0 scale per 32 along K */
} moe_dtype;

/* Problem shape.
 *   T tokens, d = d_model, E experts, k experts per token, d_ff = f (SwiGLU
 *   hidden size per expert).
 *   act:  storage type of x, weights, dout and the outputs (MOE_F32 or MOE_BF16).
 *   gemm: expert-GEMM operand format: MOE_F32 (requires act == MOE_F32),
 *         MOE_BF16 or MOE_MXFP8 (both require act == MOE_BF16).
 *   round_tile: 0 = no token rounding; otherwise the tile multiple (128 on the
 *         pages; any even value up to 4096) that moe_round_tokens rounds
 *         per-expert counts to.
 * Routing variants ("Beam" blog sections 2.2, 2.3 and 3.3; distributed-MoE
 * article, challenge 1; Trinity Large commentary, code example 2).  All zero
 * is the base layer:
 *   gate_mode: MOE_GATE_TOPK (0): gates = softmax over the k selected logits;
 *         MOE_GATE_ALL (1): gates = the softmax over all E logits at the
 *         selected experts, not renormalised (pairs added by token rounding
 *         then get P_te too).
 *   capacity_factor: 0 = none; else expert e keeps only its first
 *         C = ceil(capacity_factor * T * k / E) rows in token order (computed
 *         in double precision from the float value); the other pairs are
 *         dropped (row_of_slot = -1), kept gates unchanged.  Not combined with
 *         token rounding (MOE_ENOTSUP).
 *   lb_coef: weight of the load-balance loss lb_coef * CV(Pbar)^2, Pbar_e =
 *         mean over tokens of the full softmax P_te, CV = population standard
 *         deviation over the E entries / their mean.
 *   z_coef: weight of the z-loss z_coef * mean_t (log sum_e exp z_te)^2.
 *   Both losses are part of the training loss: moe_route writes their values
 *   to plan.aux and moe_backward adds their gradients to dlogits.
 * Supported (else MOE_ENOTSUP): 1 <= k <= min(E, 8), 1 <= E <= 256,
 * d % 64 == 0, d_ff % 64 == 0 (d_ff % 128 == 0 with bf16/MXFP8 GEMMs),
 * d, d_ff <= 16384, T <= 2^20, T*k + E*round_tile/2 < 2^31.  gate_mode
 * outside {0, 1}, or a negative or non-finite capacity_factor, lb_coef or
 * z_coef: MOE_EINVAL. */
enum { MOE_GATE_TOPK = 0, MOE_GATE_ALL = 1 };
typedef struct moe_shape {
  int32_t T, d, E, k, d_ff;
  int32_t act;
  int32_t gemm;
  int32_t round_tile;
  int32_t gate_mode;
  float   capacity_factor;
  float   lb_coef;
  float   z_coef;
} moe_shape;

/* The routing plan: device arrays carved from one caller-allocated blob by
 * moe_plan_init.  N = plan rows = offsets[E] (device-resident; N <= N_max =
 * T*k + E*round_tile/2).  Rows are token-expert pairs grouped by expert, and
 * inside one expert ordered by ascending token. */
typedef struct moe_plan {
  float   *logits;       /* [T,E]  router logits, bias (and routing noise) included  */
  float   *probs_t;      /* [E,T]  full softmax, expert-major (token rounding only)  */
  int32_t *topk_idx;     /* [T,k]  selected experts, descending logit, ties -> lower index */
  float   *topk_gate;    /* [T,k]  gates of the selected experts (see gate_mode)     */
  int32_t *counts_raw;   /* [E]    rows per expert before rounding                   */
  int32_t *counts;       /* [E]    rows per expert (after rounding when enabled)     */
  int32_t *offsets;      /* [E+1]  exclusive scan of counts; offsets[E] = N          */
  int32_t *token_of_row; /* [N_max] token of row r                                   */
  int32_t *expert_of_row;/* [N_max] expert of row r                                  */
  float   *gate_of_row;  /* [N_max] gate of row r                                    */
  int32_t *row_of_slot;  /* [T,k]  row of slot j of token t, -1 if rounding or the capacity dropped it */
  int32_t *tok_ptr;      /* [T+1]  CSR token -> rows                                 */
  int32_t *tok_rows;     /* [N_max] rows of each token, ascending                    */
  uint32_t *keep_bits;   /* [T, ceil(E/32)] bit (t,e) set when token t has a row at e */
  float   *aux;          /* [4+E] router loss terms written by moe_route: [0] lb_coef*CV^2,
                          * [1] z-loss, [2] mean_e (c_e - mean c)^2 of the per-expert counts
                          * of selected pairs (counts_raw; a monitor, no gradient), [3] CV^2,
                          * [4..4+E) Pbar.  [2] is always written; the others only when
                          * lb_coef or z_coef is nonzero.                           */
  int32_t *sched;        /* internal: per-expert tile prefixes and the tile-to-expert map of the grouped GEMMs */
} moe_plan;

/* Sizes.  All are pure host arithmetic. */
int64_t    moe_max_rows(const moe_shape *s);            /* N_max */
size_t     moe_plan_bytes(const moe_shape *s);
/* Fill `plan` with pointers into `blob` (device memory of >= moe_plan_bytes). */
moe_status moe_plan_init(const moe_shape *s, void *blob, size_t blob_bytes, moe_plan *plan);

/* Workspace queries, one per entry point that takes a workspace. */
enum { MOE_WS_ROUTE = 0, MOE_WS_ROUND = 1, MOE_WS_EXPERTS = 2, MOE_WS_BACKWARD = 3, MOE_WS_EXPERTS_COMBINE = 4 };
size_t     moe_workspace_bytes(const moe_shape *s, int which);

/* Router GEMM, top-k softmax and the plan (histogram, prefix scan, stable
 * scatter by token).  x [T,d] (act), w_gate [E,d] (act), bias [E] float32 or
 * NULL (added to the logits before top-k and softmax; receives no gradient).
 * noise [T,E] float32 or NULL: routing noise drawn by the caller ("Beam" blog
 * section 3.3, noisy top-k), added to the logits after the bias; top-k, gates
 * and the router losses use the noisy logits; no gradient flows to it.
 * With capacity_factor > 0 the plan is built, then each expert's pairs past
 * its capacity are dropped and the plan rebuilt.  With lb_coef or z_coef
 * nonzero the loss values go to plan.aux.  With round_tile == 0 the plan is
 * final; otherwise call moe_round_tokens. */
moe_status moe_route(const moe_shape *s, const void *x, const void *w_gate, const float *bias,
                     const float *noise, moe_plan *plan, void *ws, size_t ws_bytes, void *stream);

/* Token rounding (SonicMoE article, section 3): every expert's row count moves
 * to the nearest multiple of round_tile (half rounds up; if that exceeds T it
 * rounds down).  Fewer rows: the selected pairs with the smallest full-softmax
 * probability are dropped (ties: larger token first).  More rows: the
 * unselected tokens with the largest probability are added (ties: smaller token
 * first) with gate P_te / sum over the token's top-k of P.  Rebuilds the plan. */
moe_status moe_round_tokens(const moe_shape *s, moe_plan *plan, void *ws, size_t ws_bytes,
                            void *stream);

/* Permute: dst[r] = src[token_of_row[r]] for r < N (rows past N untouched).
 * src [T,d], dst [N_max,d], both act dtype.  Each source row is read once and
 * written to every row of its token.  The backward does the same for dout. */
moe_status moe_permute(const moe_shape *s, const void *src, const moe_plan *plan, void *dst,
                       void *stream);

/* Grouped expert FFN on the permuted rows.
 *   x_perm [N_max,d], w1 [E,2f,d] (gate rows first), w2 [E,d,f], all act dtype.
 *   h_saved [N_max,2f] (act): H = x_perm W1_e^T, kept for the backward.
 *   y [N_max,d] (act): Y = A W2_e^T with A = silu(H_gate) * H_up (A is rounded
 *   to the act dtype and computed from the stored H).
 * With gemm == MOE_MXFP8 every GEMM operand is quantised to MXFP8 along its K
 * inside this call: x_perm and the weights by quantiser passes, A by the
 * SwiGLU epilogue (A then exists only as MXFP8 codes, in the workspace).  The
 * quantiser passes read x_perm, w1 and w2 once each and also write their codes
 * along the other axis (W1, W2 along their first axes, x_perm along tokens):
 * moe_backward can take them from ws instead of quantising again.
 * ws: moe_workspace_bytes(s, MOE_WS_EXPERTS) bytes, 16-byte aligned. */
moe_status moe_grouped_gemm_swiglu(const moe_shape *s, const void *x_perm, const void *w1,
                                   const void *w2, const moe_plan *plan, void *h_saved, void *y,
                                   void *ws, size_t ws_bytes, void *stream);

/* The same expert FFN reading x [T,d] (act) directly: row r of every GEMM
 * operand built from x is x[token_of_row[r]], fetched through the plan inside
 * the GEMM's operand loads (with MXFP8: inside the quantiser pass), so no
 * permuted copy is written or read (Olmo-core 3 article, "three splits"
 * section: tokens go straight into the expert buffers; here the buffers are
 * never materialised).  Results are bitwise identical to moe_permute followed
 * by moe_grouped_gemm_swiglu.  Requires act == MOE_BF16 and T*d*2 < 2^31
 * bytes, else MOE_ENOTSUP.  Same workspace as moe_grouped_gemm_swiglu. */
moe_status moe_grouped_gemm_swiglu_gather(const moe_shape *s, const void *x, const void *w1,
                                          const void *w2, const moe_plan *plan, void *h_saved, void *y,
                                          void *ws, size_t ws_bytes, void *stream);

/* The expert FFN of moe_grouped_gemm_swiglu (same arguments, same kernels, same
 * bits) for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Its workspace
 * is a device array inside the library (MOE_NOALLOC_SCRATCH_BYTES per GPU,
 * reserved when the library's code is loaded on that GPU and held until the
 * process ends); the call allocates nothing.  The array of the caller's
 * current device is used, so the stream must belong to that device.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams, host threads) race and must be serialised by the
 * caller; the array keeps the last call's contents.
 * Errors: as moe_grouped_gemm_swiglu, and MOE_EWORKSPACE (nothing launched)
 * when the problem's workspace, moe_workspace_bytes(s, MOE_WS_EXPERTS), exceeds
 * MOE_NOALLOC_SCRATCH_BYTES. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_grouped_gemm_swiglu_noalloc(const moe_shape *s, const void *x_perm, const void *w1,
                                           const void *w2, const moe_plan *plan, void *h_saved, void *y,
                                           void *stream);

/* Weighted combine: out[t] = sum over the rows of t (ascending) of
 * gate_of_row[r] * y[r], accumulated in float32.  y [N_max,d], out [T,d]. */
moe_status moe_unpermute_combine(const moe_shape *s, const void *y, const moe_plan *plan,
                                 void *out, void *stream);

/* Backward for the loss sum_t <out_t, dout_t>.
 *   Inputs: x [T,d], w_gate [E,d], w1, w2, the plan, h_saved, dout [T,d];
 *   x_perm [N_max,d] (act) = what moe_permute wrote for x with this plan, or NULL.
 *   Without it x and dout are read through plan.token_of_row inside the GEMM
 *   and quantiser loads (bf16 activations and T*d*2 < 2^31 bytes), else they
 *   are permuted into the workspace; the results are identical either way.
 *   fwd_ws = the workspace of this step's moe_grouped_gemm_swiglu call (same
 *   shape, plan, x_perm, w1 and w2, unchanged since), or NULL.  With MXFP8 the
 *   backward then reads the transposed weight codes and x_perm's token-axis
 *   codes from it instead of quantising them again (identical codes, so
 *   identical results); ignored for the other GEMM types.  Only read.
 *   Outputs: dx [T,d] (act), dw_gate [E,d] f32, dw1 [E,2f,d] f32, dw2 [E,d,f] f32;
 *   optional dlogits [T,E] f32 and ds [N_max] f32 (per-row gate gradient) when
 *   not NULL.
 * dS_r = <dA'_r, A_r> with dA' = dO_perm W2_e and A recomputed from h_saved
 * (SonicMoE article, section 1); the chain rule gives the rest.  The weight
 * gradients reduce each expert's rows in chunks (partial results summed in a
 * fixed order), so their cost does not depend on how unevenly experts are
 * loaded.  ws: moe_workspace_bytes(s, MOE_WS_BACKWARD) bytes, 16-byte aligned
 * (it includes the partial slabs and, with MXFP8, the quantised operands). */
moe_status moe_backward(const moe_shape *s, const void *x, const void *w_gate, const void *w1,
                        const void *w2, const moe_plan *plan, const void *h_saved, const void *x_perm,
                        const void *fwd_ws, const void *dout, void *dx, float *dw_gate, float *dw1, float *dw2,
                        float *dlogits, float *ds, void *ws, size_t ws_bytes, void *stream);

/* Kernel timing from the caller's side (instrumentation; the results are the
 * same as without it).  The caller creates `capacity` hipEvent_t handles (passed
 * as void*) and passes this struct to a *_traced entry point, which records
 * events[0] on the stream before its first kernel and events[i + 1] after its
 * i-th kernel, and names that kernel in names[i]; `count` is the number of
 * events recorded (kernels + 1, at most capacity and MOE_TRACE_MAX_KERNELS + 1).
 * hipEventElapsedTime(events[i], events[i + 1]) is then the device time of
 * kernel names[i].  Names are static strings owned by the library, e.g. "up_swiglu",
 * "down" (forward), "dact", "dw1", "dw2", "dx_perm", "router_bwd",
 * "router_dx", "router_dwg" (backward), "mx_*" for the MXFP8 kernels.
 * Errors: MOE_EINVAL for a negative capacity or a NULL event among the first
 * `capacity`; a failed hipEventRecord stops the call with MOE_EHIP. */
#define MOE_TRACE_MAX_KERNELS 48
typedef struct moe_trace {
  void **events;
  int32_t capacity;
  int32_t count;
  const char *names[MOE_TRACE_MAX_KERNELS];
} moe_trace;

/* moe_grouped_gemm_swiglu, moe_grouped_gemm_swiglu_gather and moe_backward with
 * kernel timing (above). */
moe_status moe_grouped_gemm_swiglu_gather_traced(const moe_shape *s, const void *x, const void *w1,
                                                 const void *w2, const moe_plan *plan, void *h_saved, void *y,
                                                 void *ws, size_t ws_bytes, void *stream, moe_trace *trace);
moe_status moe_grouped_gemm_swiglu_traced(const moe_shape *s, const void *x_perm, const void *w1,
                                          const void *w2, const moe_plan *plan, void *h_saved, void *y,
                                          void *ws, size_t ws_bytes, void *stream, moe_trace *trace);
moe_status moe_backward_traced(const moe_shape *s, const void *x, const void *w_gate, const void *w1,
                               const void *w2, const moe_plan *plan, const void *h_saved, const void *x_perm,
                               const void *fwd_ws, const void *dout, void *dx, float *dw_gate, float *dw1,
                               float *dw2, float *dlogits, float *ds, void *ws, size_t ws_bytes, void *stream,
                               moe_trace *trace);

/* The expert FFN and the weighted combine in one call, with the combine's gate
 * and scatter in GEMM2's epilogue (Olmo-core 3 article, "three splits" section:
 * the expert output goes straight to where its token is reduced).  GEMM1 +
 * SwiGLU as moe_grouped_gemm_swiglu (h_saved as there; x is x_perm [N_max,d]
 * when x_gathered = 0, x [T,d] read through the plan when x_gathered = 1, with
 * moe_grouped_gemm_swiglu_gather's requirements); GEMM2's epilogue multiplies
 * row r of A W2_e^T by gate_of_row[r] in fp32, rounds it to bf16 and stores it
 * at the row's token-order position (the order of plan.tok_rows), so that each
 * token's rows are contiguous; out[t] [T,d] is then their sum in fp32,
 * ascending, rounded to bf16.  Y itself is never stored.  Deterministic (no
 * atomics): the per-token sum is a separate pass over the gated rows, because
 * a token's k rows are produced by tiles of k different experts.  Differs from
 * moe_grouped_gemm_swiglu + moe_unpermute_combine only in where the gate meets
 * the bf16 rounding (there the rounded Y is gated inside the fp32 sum).
 * act = gemm = MOE_BF16 only, else MOE_ENOTSUP.
 * ws: moe_workspace_bytes(s, MOE_WS_EXPERTS_COMBINE) bytes (the expert
 * workspace plus N_max rows of gated output and N_max positions).
 * trace: as the *_traced calls ("up_swiglu", "row_positions",
 * "down_gate_scatter", "segment_sum"), or NULL. */
moe_status moe_grouped_gemm_swiglu_combine(const moe_shape *s, const void *x, int x_gathered,
                                           const void *w1, const void *w2, const moe_plan *plan,
                                           void *h_saved, void *out, void *ws, size_t ws_bytes,
                                           void *stream, moe_trace *trace);

/* MXFP8 weight codes kept across the micro-batches of one optimizer step
 * (gradient accumulation: w1 and w2 do not change between them).  The
 * Olmo-core 3 article's MXFP8 switch ("three splits" section) quantises every
 * expert-GEMM operand; the codes of a weight depend on that weight alone, so
 * quantising w1 and w2 once per optimizer step instead of once per micro-batch
 * gives the same codes and bitwise the same results.
 *
 * moe_quantize_weights_mx writes the codes of w1 [E,2f,d] and w2 [E,d,f] (bf16)
 * along both of their axes into ws, the expert workspace
 * (moe_workspace_bytes(s, MOE_WS_EXPERTS) bytes), where moe_grouped_gemm_swiglu
 * keeps them.  Where they sit depends only on E, d and d_ff, so micro-batches
 * of different T may share one ws sized for the largest.
 * moe_grouped_gemm_swiglu_wcodes is the expert FFN of moe_grouped_gemm_swiglu
 * taking those codes from ws instead of quantising w1 and w2 (neither is
 * passed): x is x_perm [N_max,d] (x_gathered = 0) or x [T,d] read through the
 * plan (x_gathered = 1, as moe_grouped_gemm_swiglu_gather, with its
 * requirements).  It rewrites the rest of ws, so moe_backward with fwd_ws = ws
 * works as after moe_grouped_gemm_swiglu (and reads the transposed weight codes
 * from there too).  trace: as the *_traced calls, or NULL.  The library cannot
 * tell stale codes: the caller quantises again whenever w1 or w2 change.
 * Errors: MOE_ENOTSUP unless gemm == MOE_MXFP8 (nothing launched); otherwise
 * as moe_grouped_gemm_swiglu and moe_grouped_gemm_swiglu_gather. */
moe_status moe_quantize_weights_mx(const moe_shape *s, const void *w1, const void *w2, void *ws,
                                   size_t ws_bytes, void *stream);
moe_status moe_grouped_gemm_swiglu_wcodes(const moe_shape *s, const void *x, int x_gathered,
                                          const moe_plan *plan, void *h_saved, void *y, void *ws,
                                          size_t ws_bytes, void *stream, moe_trace *trace);

/* MXFP8 quantiser (OCP Microscaling v1.0; the pages only name the format):
 * blocks of 32 consecutive values along the reduction axis; shared exponent
 * X = floor(log2(max|v|)) - 8 clamped to [-127,127] (-127 for an all-zero
 * block); scale byte = X + 127; element = v / 2^X rounded to nearest-even
 * E4M3 (bias 7, max 448), saturating, sign bit kept.  This is the hook that
 * exposes the two quantisers the MXFP8 GEMMs use:
 *   k_axis = 1: blocks along each row.  src [rows, cols] bf16, cols % 32 == 0;
 *     codes [rows, cols] u8; scales [rows, cols/32] u8.
 *   k_axis = 0: blocks down each column, written transposed (K-contiguous, as
 *     the GEMMs read a weight used along its first axis).  rows % 64 == 0 and
 *     cols % 64 == 0; codes [cols, rows] u8; scales [cols, rows/32] u8.
 * Errors: MOE_EINVAL for null/misaligned pointers, sizes <= 0 or not matching
 * the rules above, or k_axis not 0/1. */
moe_status moe_quantize_mx(const void *src_bf16, int64_t rows, int64_t cols, int k_axis, uint8_t *codes,
                           uint8_t *scales, void *stream);

/* Measurement reference, not part of the layer: streams `bytes` through HBM so
 * the data-movement kernels above can be compared with the rates plain kernels
 * reach on this GPU.  mode 0: read src (non-temporal loads); 1: write dst;
 * 2: copy src to dst with non-temporal loads; 3: the same with non-temporal
 * stores too.  src (modes 0, 2, 3) and dst device pointers, 16-byte aligned,
 * bytes a positive multiple of 16 (mode 0 needs 16 bytes of dst, written only
 * for a data pattern the inputs of a measurement never hold).  Errors:
 * MOE_EINVAL for a bad pointer, size or mode. */
moe_status moe_ref_stream(const void *src, void *dst, int64_t bytes, int mode, void *stream);

const char *moe_status_str(moe_status st);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
