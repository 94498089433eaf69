/*
 * moe.h -- C ABI of the routed SwiGLU mixture-of-experts layer on one AMD
 * Instinct MI355X (gfx950): router projection, routing + sort by expert,
 * forward, backward, router backward.
 *
 * Method: the LigerCute package README (liger-cute-kernels 0.8.3), section
 * "LigerMoE design" (sub-sections "Forward pass" and "Backward pass"): sort
 * the routed tokens by expert, run every expert's MLP on its tokens, combine
 * the expert results with the router weights; in the backward, form the
 * routed output gradients, recompute the activations, compute input and
 * expert-weight gradients (weight gradients summed over all of an expert's
 * token tiles) and reduce the routed dX back onto the tokens.  The same
 * README's overview section asks for buffers sized from the total routed
 * capacity (no per-expert capacity, no dropped tokens) so that the calls stay
 * capturable into a graph despite data-dependent routing; every call below
 * therefore takes its sizes from the host-side dims only and never reads
 * device data back to the host.
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are HIP device pointers on the current device,
 *     row-major (last index contiguous), 16-byte aligned.  bf16 arrays are
 *     passed as `void*` (raw bfloat16 bits).
 *   - The caller owns every buffer, including the workspace; the library never
 *     allocates, frees or keeps a pointer after the call returns (the one
 *     exception, moe_route_sort_noalloc, uses a static device array of the
 *     library's own instead of a workspace).
 *   - `stream` is a hipStream_t passed as `void*` (NULL = the default stream).
 *     Work is enqueued asynchronously; nothing synchronises with the host.
 *   - Host-side validation only.  On any error nothing is launched and the
 *     status tells why.  Device *contents* are not validated (expert ids out
 *     of range, offsets that do not match the ids): that is undefined
 *     behaviour, because checking it would need a device-to-host read.
 *   - Outputs are overwritten, except where an `accumulate_*` flag asks for
 *     addition and for the in/out `dx` of moe_router_bwd.
 *     Results are bitwise deterministic run to run (no floating-point atomics).
 *   - Symbols: the library exports only `moe_*`.
 *
 * Weight layout (linear-layer convention [out_features, in_features]):
 *   w_gate, w_up  [E, I, D]   gate/up projection of expert e: D -> I
 *   w_down        [E, D, I]   down projection of expert e:    I -> D
 * so that  h = silu(x W_gate[e]^T) * (x W_up[e]^T),  o = h W_down[e]^T.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

/* Router score functions. */
#define MOE_SCORE_SOFTMAX_TOPK 0 /* softmax over E, keep top K, renormalise over the K */
#define MOE_SCORE_SIGMOID 1      /* sigmoid of each selected logit, no renormalisation */

/* Status codes. */
#define MOE_OK 0
#define MOE_ERR_BAD_ARG 1        /* null / misaligned pointer, bad dims, K > E, T*K >= 2^31 */
#define MOE_ERR_UNSUPPORTED 2    /* valid but unsupported: D or I not a multiple of 64,
                                    E > 1024, K > 64, a grid too large for 32 bits, or
                                    an operand the GEMMs address with 32-bit byte
                                    offsets reaching 2 GiB: T*K*max(D, 2I)*2 or I*D*2
                                    >= 2^31 (at D = 2048, I = 768, K = 8: T <= 65535) */
#define MOE_ERR_WORKSPACE 3      /* workspace smaller than moe_workspace_bytes() */
#define MOE_ERR_HIP 4            /* a HIP launch or runtime call failed */
#define MOE_ERR_SCRATCH 5        /* the shape needs more than the static scratch buffer of
                                    moe_route_sort_noalloc (never for dims that pass the
                                    other checks: E <= 1024 needs at most 1 MiB) */

/* Workspace phases for moe_workspace_bytes(). */
#define MOE_PHASE_ROUTE 0
#define MOE_PHASE_FWD 1
#define MOE_PHASE_BWD 2
#define MOE_PHASE_ROUTER_BWD 3

typedef int32_t moe_status;

/* Layer dimensions.  T tokens, model width D, expert hidden width I, E
 * experts, K experts per token, score = MOE_SCORE_*.  R = T*K routed rows. */
typedef struct moe_dims {
    int32_t T, D, I, E, K;
    int32_t score;
} moe_dims;

/* Bytes of device workspace that the given phase needs (pure host, touches
 * no device).  Returns 0 for invalid dims or an unknown phase. */
size_t moe_workspace_bytes(const moe_dims *dims, int32_t phase);

/* Routing and sort by expert ("LigerMoE design / Forward pass": the routed
 * tokens are sorted by expert before the expert loop).
 *
 *   logits          device fp32 [T, E]   router logits (finite)
 *   topk_idx        device i32  [T, K]   out: selected experts; slot k holds the
 *                                        rank-k expert (larger logit first, equal
 *                                        logits toward the lower expert id)
 *   topk_w          device fp32 [T, K]   out: router weights (per dims->score)
 *   counts          device i32  [E]      out: routed rows per expert
 *   offsets         device i32  [E+1]    out: exclusive prefix of counts, offsets[E] = T*K
 *   sorted_to_flat  device i32  [T*K]    out: sorted row p -> flat slot f = t*K + k;
 *                                        inside an expert rows are in ascending f
 *   flat_to_sorted  device i32  [T*K]    out: inverse permutation
 *   ws, ws_bytes    device workspace of at least moe_workspace_bytes(dims, MOE_PHASE_ROUTE)
 * All index outputs are unique and must match a plain CPU reference bit for bit. */
moe_status moe_route_sort(const moe_dims *dims, const float *logits, int32_t *topk_idx,
                          float *topk_w, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_to_flat, int32_t *flat_to_sorted, void *ws,
                          size_t ws_bytes, void *stream);

/* moe_route_sort without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments (minus ws, ws_bytes), same kernels and bitwise
 * the same outputs as moe_route_sort.  The per-block expert histograms live in
 * a static 1 MiB device array inside the library, one copy per GPU, held until
 * the process ends and looked up on each device's first call; the call
 * allocates and frees nothing.  Every call on one GPU shares that array, so
 * calls that overlap on one GPU (concurrent streams, or host threads) race:
 * serialise them.  MOE_ERR_SCRATCH if the shape would need more than 1 MiB of
 * histograms (at most E * 256 blocks * 4 bytes, so no accepted shape does). */
moe_status moe_route_sort_noalloc(const moe_dims *dims, const float *logits, int32_t *topk_idx,
                                  float *topk_w, int32_t *counts, int32_t *offsets,
                                  int32_t *sorted_to_flat, int32_t *flat_to_sorted,
                                  void *stream);

/* Forward ("LigerMoE design / Forward pass"): grouped gate/up GEMM over the
 * routed rows in expert order (gathered from x inside the GEMM's operand
 * loads) with the SwiGLU fused into its epilogue, grouped down GEMM, then the
 * router-weighted combine
 *     y[t] = sum_{k<K} topk_w[t,k] * o[t,k]      (fp32 accumulation, k ascending)
 *
 *   x               device bf16 [T, D]
 *   w_gate, w_up    device bf16 [E, I, D]
 *   w_down          device bf16 [E, D, I]
 *   topk_w, offsets, sorted_to_flat, flat_to_sorted   as produced by moe_route_sort
 *   y               device bf16 [T, D]   out
 *   ws, ws_bytes    device workspace of at least moe_workspace_bytes(dims, MOE_PHASE_FWD)
 * Intermediates live in the workspace: the SwiGLU activations H as fp16 (the
 * down GEMM multiplies fp16, its bf16 weights converted exactly where they are
 * in fp16's normal range), the unweighted expert outputs as bf16; all GEMMs
 * accumulate in fp32.  Range: |h| = |silu(g) u| <= 65504 (fp16); beyond it
 * the affected outputs come out +-inf or NaN, never finite and wrong (the
 * backward has the same limit on w h).
 * With 16 to 64 row tiles of 256 routed rows per XCD (at most
 * (T K + 255 E) / 256 row tiles over 8 XCDs) the two GEMMs run as one launch:
 * each XCD takes a range of row tiles, and a down tile starts once the
 * gate/up tiles of its rows, on the same XCD, have stored H.  The first 4
 * bytes of the workspace then hold the call's status word once the call has
 * run on the stream: 0, or nonzero if a wait of that launch gave up after
 * about a second (bit 0) or the GPU dealt workgroups to its XCDs other than
 * round-robin (bit 1); the outputs of such a call are not valid.  Concurrent
 * calls need separate workspaces. */
moe_status moe_fwd(const moe_dims *dims, const void *x, const void *w_gate, const void *w_up,
                   const void *w_down, const float *topk_w, const int32_t *offsets,
                   const int32_t *sorted_to_flat, const int32_t *flat_to_sorted, void *y,
                   void *ws, size_t ws_bytes, void *stream);

/* Backward ("LigerMoE design / Backward pass"), routing held fixed, for the
 * loss L with dL/dy = dy:
 *   dx        device bf16 [T, D]   out: dL/dx through the experts
 *                                  (sum over the K routed copies, fp32, k ascending)
 *   dw_gate   device fp32 [E, I, D] out: dL/dW_gate
 *   dw_up     device fp32 [E, I, D] out: dL/dW_up
 *   dw_down   device fp32 [E, D, I] out: dL/dW_down
 *   d_topk_w  device fp32 [T, K]   out: dL/dtopk_w[t,k] = <dy[t], o[t,k]>
 *   accumulate_dw  0: overwrite dw_*;  1: add into dw_* (fp32; for an expert
 *                  whose rows span several dW row chunks, the first chunk's
 *                  tile is added, then the sum of the others: two roundings)
 * dA = dOu W_down runs first (fp32); the gate/up activations are then
 * recomputed (not read from the forward), and the SwiGLU backward and the
 * router-weight gradient come out of that recompute GEMM's epilogue; the
 * routed rows of x and dy are gathered inside the GEMMs' operand loads.  Each
 * weight-gradient tile reduces over its expert's rows in chunks of at most
 * 4096 rows, one workgroup per chunk; the chunks' partial tiles are added in
 * chunk order (no atomics, deterministic).  The weight-gradient GEMMs multiply
 * fp16 operands; for an expert with n rows whose squared router weights sum
 * to S, with S * (1 + 100 / n) * max(1, 3 D / (8 I)) > 16, the rounded
 * operand (dG, dU or the weighted activations) is split
 * into fp16 high and low parts, both multiplied into the same accumulators
 * (row block by row block).  The fp16 gradient operands carry a power-of-two
 * scale s with s * max|dy| in [1, 2), removed from the fp32 results, so the
 * gradients of 2^c dy are exactly 2^c times those of dy whatever c (within
 * fp32 range): no loss scaling is needed.  x enters the weight gradients as
 * fp16 without a scale (rounded to nearest): |x| from 65520 on becomes
 * infinite there, so dW_gate and dW_up of the experts such a token reaches
 * come out non-finite (never finite and wrong), and values below 2^-14 keep
 * less relative precision (activations are far inside that range).  Range of the fp16 gradient operands: with w the router weight,
 * h = silu(g) u and dA = dOu W_down, the backward needs |w h| <= 65504 (the
 * dW_down operand) and s |dG|, s |dU| <= 65504 (the dX and dW_gate/up
 * operands); roughly, |g u| below ~6e4 for unit router weights.  Beyond it
 * the gradients that pass through the overflowing operand come out +-inf or
 * NaN (never finite and wrong), as in fp16 loss-scaled training: dW_down
 * for Hw, dX, dW_gate and dW_up for dG and dU.  The forward output and
 * d_topk_w (fp32 partials) are unaffected.  Experts with no
 * rows get exact zeros (or are left unchanged when accumulating).
 * dA and the recompute GEMM run as one launch under the same rule as the
 * forward's gate/up and down GEMMs (a recompute tile reads dA in its
 * epilogue, once the dA tiles of its rows have stored it), with the same
 * status word in the first 4 bytes of the workspace.
 *   ws, ws_bytes   device workspace of at least moe_workspace_bytes(dims, MOE_PHASE_BWD) */
moe_status moe_bwd(const moe_dims *dims, const void *x, const void *w_gate, const void *w_up,
                   const void *w_down, const float *topk_w, const int32_t *offsets,
                   const int32_t *sorted_to_flat, const int32_t *flat_to_sorted,
                   const void *dy, void *dx, float *dw_gate, float *dw_up, float *dw_down,
                   float *d_topk_w, int32_t accumulate_dw, void *ws, size_t ws_bytes,
                   void *stream);

/* Router projection, the input side of the layer: the logits that
 * moe_route_sort selects on ("LigerMoE design / Forward pass": the router
 * weights that the final combine applies come from these logits).
 *     logits[t, e] = sum_d x[t, d] w_r[d, e]
 *   x        device bf16 [T, D]
 *   w_r      device fp32 [D, E]   router projection (note: [in, out], so that
 *                                 logits = x w_r)
 *   logits   device fp32 [T, E]   out
 * Computed on the bf16 matrix cores: each fp32 weight is split exactly into
 * three bf16 terms (w0 = bf16(w), w1 = bf16(w - w0), w2 = w - w0 - w1), every
 * product of a bf16 x with a term is exact in fp32, and the three products are
 * accumulated in fp32 -- the precision of fp32 products at the bf16 rate.  Only dims->T, D, E are used; the other dims must still be
 * valid (the router is part of the layer the dims describe). */
moe_status moe_router_fwd(const moe_dims *dims, const void *x, const float *w_r, float *logits,
                          void *stream);

/* Router backward, the step before the input side of "LigerMoE design /
 * Backward pass": with the top-K selection held fixed (it is piecewise
 * constant in the logits), the router-weight gradient d_topk_w that moe_bwd
 * returns flows back through the score function into the selected logits,
 *   softmax-renormalised:  dl[t, idx_k] = w_k (d_k - sum_j w_j d_j)
 *   sigmoid:               dl[t, idx_k] = d_k w_k (1 - w_k)
 * (dl = 0 for unselected experts), and from there into the projection and
 * the layer input:
 *   dw_r = x^T dl          [D, E]
 *   dx  += dl w_r^T        [T, D]
 *   x, w_r              as for moe_router_fwd
 *   topk_idx, topk_w    as produced by moe_route_sort (the selection and its weights)
 *   d_topk_w            device fp32 [T, K]  dL/dtopk_w, as produced by moe_bwd
 *   dx                  device bf16 [T, D]  in/out: the expert-path input gradient
 *                       from moe_bwd on entry; on return dx + the router path's
 *                       contribution (fp32 sum over k ascending, one rounding)
 *   dw_r                device fp32 [D, E]  out: dL/dw_r
 *   accumulate_dwr      0: overwrite dw_r;  1: add into dw_r (fp32)
 *   ws, ws_bytes        device workspace of at least
 *                       moe_workspace_bytes(dims, MOE_PHASE_ROUTER_BWD)
 * dw_r is reduced over fixed token ranges whose partials are summed in range
 * order (no atomics: bitwise deterministic). */
moe_status moe_router_bwd(const moe_dims *dims, const void *x, const float *w_r,
                          const int32_t *topk_idx, const float *topk_w, const float *d_topk_w,
                          void *dx, float *dw_r, int32_t accumulate_dwr, void *ws,
                          size_t ws_bytes, void *stream);

/* Static description of a status code (never NULL). */
const char *moe_status_string(moe_status status);

/* MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

/* Text of the HIP error behind the calling thread's last MOE_ERR_HIP (which
 * launch, HIP's message and code); "" if the last call succeeded. */
const char *moe_last_error(void);

/* ---- Per-kernel timing (a measurement aid, off by default).
 * moe_prof_enable(1) clears what was recorded and starts bracketing every
 * kernel the library launches with two hipEvents recorded on that kernel's
 * stream; moe_prof_enable(0) clears and stops.  moe_prof_read() waits for the
 * recorded events and writes, for kernel ids 0..n-1, the summed elapsed time
 * in milliseconds and the number of launches since the last enable.  Kernel
 * ids run 0..moe_prof_num_kernels()-1; moe_prof_kernel_name() names them (NULL
 * for an unknown id).  Timing state (the flag and the records) is process-wide
 * and thread-safe; each launch's two events are paired per host thread.
 * Launches on a stream that is being captured into a graph are not timed.
 * Returns MOE_ERR_HIP if an event
 * query fails, MOE_ERR_BAD_ARG for null arrays with n > 0.
 * moe_prof_only(id) restricts the bracketing to one kernel id (-1: every
 * kernel, the default), so that a timed loop carries two events per launch
 * of that kernel instead of two per kernel; MOE_ERR_BAD_ARG for an unknown id. */
int32_t moe_prof_enable(int32_t on);
moe_status moe_prof_only(int32_t kernel_id);
int32_t moe_prof_num_kernels(void);
const char *moe_prof_kernel_name(int32_t kernel_id);
moe_status moe_prof_read(double *total_ms, int64_t *launches, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
