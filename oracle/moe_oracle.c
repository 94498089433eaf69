/*
 * moe_oracle.c -- plain, slow, CPU reference of the routed SwiGLU
 * mixture-of-experts layer (forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package's smoke check
 * and the benchmark's CPU-baseline leg may load this library.  The GPU
 * library shares no code, header, table or constant with it, and no product
 * code path may call it.
 *
 * Everything is computed in float64 from float64 copies of the exact bf16 /
 * float32 inputs.  No blocking, fusion or reordering beyond the definitions
 * below: one routed (token, slot) row at a time, sums in index order.
 * OpenMP only splits independent outputs across threads (each output
 * element is produced by exactly one thread, in a fixed order), so results
 * do not depend on the thread count.
 *
 * Source of the method: the LigerCute package README (liger-cute-kernels
 * 0.8.3), section "LigerMoE design":
 *   - "Forward pass": routed tokens are sorted by expert, each expert runs
 *     its MLP on its tokens, and a final local combine applies the router
 *     weights to the expert results.
 *   - "Backward pass": routed expert-output gradients first, then activation
 *     recomputation, input gradients and expert-weight gradients (weight
 *     gradients accumulated over all token batches of an expert), and a final
 *     step that reduces the routed dX contributions back onto their tokens.
 * The page does not name the router function, the activation or the tie
 * rule; the readings taken here (softmax -> top-K -> renormalise or a
 * sigmoid score; SwiGLU expert MLP; ties to the lower expert id; the order of
 * an expert's rows = ascending flat slot t*K+k) are the plainest ones that
 * the rest of the description supports.
 *
 * Layouts (row-major, last index contiguous):
 *   x, dy            [T, D]
 *   logits           [T, E]   float32 (router logits, an input)
 *   w_gate, w_up     [E, I, D]  expert e maps D -> I   (linear-layer layout)
 *   w_down           [E, D, I]  expert e maps I -> D
 *   idx              [T, K]   int32   selected experts, slot order = rank
 *   w                [T, K]   float64 router weights of the selected experts
 *   w_r              [D, E]   router projection (logits = x w_r)
 *
 * The router projection and its backward (moe_oracle_router_*) extend the
 * page's layer by its input side: the logits the routing selects on, and
 * the gradient that flows back through the router weights into the logits,
 * the projection weights and the layer input.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t T;
    int32_t D, I, E, K;
    int32_t score; /* 0: softmax over E, top-K, renormalise; 1: sigmoid */
} moe_oracle_dims;

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

static int dims_ok(const moe_oracle_dims *d) {
    return d && d->T >= 0 && d->D > 0 && d->I > 0 && d->E > 0 && d->K > 0 &&
           d->K <= d->E && (d->score == 0 || d->score == 1);
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu(double z) { return z * sigmoid(z); }

/* d silu(z) / dz = sigmoid(z) * (1 + z * (1 - sigmoid(z))) */
static double silu_grad(double z) {
    double s = sigmoid(z);
    return s * (1.0 + z * (1.0 - s));
}

/* SwiGLU of one hidden unit: h = silu(g) * u. */
static double swiglu(double g, double u) { return silu(g) * u; }

/* Its gradient given dh = dL/dh:  dg = dh * u * silu'(g),  du = dh * silu(g). */
static void swiglu_backward(double dh, double g, double u, double *dg, double *du) {
    *dg = dh * u * silu_grad(g);
    *du = dh * silu(g);
}

/* ---------------------------------------------------------------------------
 * Routing.  For each token the experts are ranked by logit, larger first,
 * equal logits broken toward the lower expert id; the first K form the
 * token's selection and slot k holds the rank-k expert.
 *   score 0: w_k = exp(l_k) / sum_{j<K} exp(l_j): the softmax over all E
 *            experts restricted to the K selected and renormalised (the full
 *            softmax denominator cancels).  Evaluated with the usual max
 *            shift, which is exact algebra.
 *   score 1: w_k = sigmoid(l_k), no renormalisation.
 * ------------------------------------------------------------------------- */
int moe_oracle_route(const moe_oracle_dims *d, const float *logits,
                     int32_t *idx, double *w) {
    if (!dims_ok(d) || !logits || !idx || !w) return ORACLE_BAD_ARG;
    const int E = d->E, K = d->K;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < d->T; ++t) {
        const float *l = logits + t * E;
        int32_t *sel = idx + t * K;
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int j = 0; j < k; ++j)
                    if (sel[j] == e) taken = 1;
                if (taken) continue;
                if (best < 0 || l[e] > l[best] || (l[e] == l[best] && e < best))
                    best = e;
            }
            sel[k] = best;
        }
        double *wt = w + t * K;
        if (d->score == 0) {
            double lmax = (double)l[sel[0]];
            double den = 0.0;
            for (int k = 0; k < K; ++k) den += exp((double)l[sel[k]] - lmax);
            for (int k = 0; k < K; ++k) wt[k] = exp((double)l[sel[k]] - lmax) / den;
        } else {
            for (int k = 0; k < K; ++k) wt[k] = sigmoid((double)l[sel[k]]);
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Sort by expert (counting sort, stable in the flat slot f = t*K + k).
 *   counts[e]        number of routed rows of expert e
 *   offsets[e]       first sorted row of expert e; offsets[E] = T*K
 *   sorted_to_flat   sorted row p -> flat slot f
 *   flat_to_sorted   inverse permutation
 * ------------------------------------------------------------------------- */
int moe_oracle_sort(const moe_oracle_dims *d, const int32_t *idx,
                    int32_t *counts, int32_t *offsets,
                    int32_t *sorted_to_flat, int32_t *flat_to_sorted) {
    if (!dims_ok(d) || !idx || !counts || !offsets || !sorted_to_flat ||
        !flat_to_sorted)
        return ORACLE_BAD_ARG;
    const int64_t R = d->T * d->K;
    const int E = d->E;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t f = 0; f < R; ++f) {
        if (idx[f] < 0 || idx[f] >= E) return ORACLE_BAD_ARG;
        counts[idx[f]] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return ORACLE_NO_MEMORY;
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int64_t f = 0; f < R; ++f) {
        int32_t p = cursor[idx[f]]++;
        sorted_to_flat[p] = (int32_t)f;
        flat_to_sorted[f] = p;
    }
    free(cursor);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * One expert applied to one token row.
 *   g_i = sum_d w_gate[e,i,d] x_d        u_i = sum_d w_up[e,i,d] x_d
 *   h_i = silu(g_i) * u_i                (SwiGLU)
 *   o_j = sum_i w_down[e,j,i] h_i
 * ------------------------------------------------------------------------- */
typedef struct {
    const moe_oracle_dims *d;
    const double *x, *w_gate, *w_up, *w_down;
} layer_t;

static void gate_up_at(const layer_t *L, int e, int i, const double *xt,
                       double *g, double *u) {
    const int D = L->d->D, I = L->d->I;
    const double *wg = L->w_gate + ((size_t)e * I + i) * D;
    const double *wu = L->w_up + ((size_t)e * I + i) * D;
    double sg = 0.0, su = 0.0;
    for (int c = 0; c < D; ++c) {
        sg += wg[c] * xt[c];
        su += wu[c] * xt[c];
    }
    *g = sg;
    *u = su;
}

static double down_at(const layer_t *L, int e, int j, const double *h) {
    const int D = L->d->D, I = L->d->I;
    const double *wd = L->w_down + ((size_t)e * D + j) * I;
    double s = 0.0;
    for (int i = 0; i < I; ++i) s += wd[i] * h[i];
    return s;
}

/* dh_i = sum_j w_down[e,j,i] * do_j   (transpose of the down projection) */
static double down_t_at(const layer_t *L, int e, int i, const double *dov) {
    const int D = L->d->D, I = L->d->I;
    const double *wd = L->w_down + (size_t)e * D * I;
    double s = 0.0;
    for (int j = 0; j < D; ++j) s += wd[(size_t)j * I + i] * dov[j];
    return s;
}

/* Full forward of expert e on token row xt: g, u, h [I] and o [D]. */
static void expert_forward(const layer_t *L, int e, const double *xt,
                           double *g, double *u, double *h, double *o) {
    const int D = L->d->D, I = L->d->I;
    for (int i = 0; i < I; ++i) {
        gate_up_at(L, e, i, xt, &g[i], &u[i]);
        h[i] = swiglu(g[i], u[i]);
    }
    if (o)
        for (int j = 0; j < D; ++j) o[j] = down_at(L, e, j, h);
}

/* Gradient through one expert's SwiGLU for one row, given the recomputed
 * g, u and the gradient `dov` of the expert output:
 *   dh_i = sum_j w_down[e,j,i] do_j,  then swiglu_backward per unit.      */
static void expert_backward(const layer_t *L, int e, const double *g,
                            const double *u, const double *dov, double *dg,
                            double *du) {
    for (int i = 0; i < L->d->I; ++i)
        swiglu_backward(down_t_at(L, e, i, dov), g[i], u[i], &dg[i], &du[i]);
}

/* ---------------------------------------------------------------------------
 * Forward for a list of tokens (tokens == NULL: all T, in order).
 *   y_t = sum_{k=0..K-1} w[t,k] * expert_{idx[t,k]}(x_t)     (k ascending)
 *   o (optional) [ntok, K, D]: the unweighted expert outputs.
 * ------------------------------------------------------------------------- */
int moe_oracle_forward(const moe_oracle_dims *d, const double *x,
                       const double *w_gate, const double *w_up,
                       const double *w_down, const int32_t *idx,
                       const double *w, int64_t ntok, const int64_t *tokens,
                       double *y, double *o) {
    if (!dims_ok(d) || !x || !w_gate || !w_up || !w_down || !idx || !w || !y)
        return ORACLE_BAD_ARG;
    if (!tokens) ntok = d->T;
    const int D = d->D, I = d->I, K = d->K;
    layer_t L = {d, x, w_gate, w_up, w_down};
    int status = ORACLE_OK;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (3 * (size_t)I + D));
        if (!buf) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < ntok; ++n) {
            if (!buf) continue;
            int64_t t = tokens ? tokens[n] : n;
            double *g = buf, *u = buf + I, *h = buf + 2 * I, *ok = buf + 3 * I;
            double *yt = y + n * D;
            for (int j = 0; j < D; ++j) yt[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                int e = idx[t * K + k];
                expert_forward(&L, e, x + t * D, g, u, h, ok);
                double wk = w[t * K + k];
                for (int j = 0; j < D; ++j) yt[j] += wk * ok[j];
                if (o) memcpy(o + (n * K + k) * D, ok, sizeof(double) * D);
            }
        }
        free(buf);
    }
    return status;
}

/* ---------------------------------------------------------------------------
 * Backward, routing held fixed, for a list of tokens.  With L = <dY, y>:
 *   dRW[t,k] = dL/dw[t,k] = <dY_t, o_tk>
 *   do       = w[t,k] * dY_t                     (gradient of o_tk)
 *   dh_i     = sum_j w_down[e,j,i] do_j
 *   dg_i     = dh_i * u_i * silu'(g_i)
 *   du_i     = dh_i * silu(g_i)
 *   dX_t     = sum_k ( sum_i w_gate[e,i,:] dg_i + w_up[e,i,:] du_i )
 * dx [ntok, D], drw [ntok, K].
 * ------------------------------------------------------------------------- */
int moe_oracle_backward_tokens(const moe_oracle_dims *d, const double *x,
                               const double *w_gate, const double *w_up,
                               const double *w_down, const int32_t *idx,
                               const double *w, const double *dy,
                               int64_t ntok, const int64_t *tokens, double *dx,
                               double *drw) {
    if (!dims_ok(d) || !x || !w_gate || !w_up || !w_down || !idx || !w ||
        !dy || !dx || !drw)
        return ORACLE_BAD_ARG;
    if (!tokens) ntok = d->T;
    const int D = d->D, I = d->I, K = d->K;
    layer_t L = {d, x, w_gate, w_up, w_down};
    int status = ORACLE_OK;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (5 * (size_t)I + 2 * D));
        if (!buf) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < ntok; ++n) {
            if (!buf) continue;
            int64_t t = tokens ? tokens[n] : n;
            double *g = buf, *u = buf + I, *h = buf + 2 * I;
            double *dg = buf + 3 * I, *du = buf + 4 * I;
            double *ok = buf + 5 * I, *dov = buf + 5 * I + D;
            const double *dyt = dy + t * D;
            double *dxt = dx + n * D;
            for (int j = 0; j < D; ++j) dxt[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                int e = idx[t * K + k];
                double wk = w[t * K + k];
                expert_forward(&L, e, x + t * D, g, u, h, ok);
                double s = 0.0;
                for (int j = 0; j < D; ++j) s += dyt[j] * ok[j];
                drw[n * K + k] = s;
                for (int j = 0; j < D; ++j) dov[j] = wk * dyt[j];
                expert_backward(&L, e, g, u, dov, dg, du);
                const double *wg = w_gate + (size_t)e * I * D;
                const double *wu = w_up + (size_t)e * I * D;
                for (int j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < I; ++i)
                        acc += wg[(size_t)i * D + j] * dg[i] + wu[(size_t)i * D + j] * du[i];
                    dxt[j] += acc;
                }
            }
        }
        free(buf);
    }
    return status;
}

/* Routed rows of expert e among the given tokens, ascending flat slot order. */
static int64_t rows_of_expert(const moe_oracle_dims *d, const int32_t *idx,
                              int64_t ntok, const int64_t *tokens, int e,
                              int64_t *out) {
    int64_t n = 0;
    for (int64_t m = 0; m < ntok; ++m) {
        int64_t t = tokens ? tokens[m] : m;
        for (int k = 0; k < d->K; ++k)
            if (idx[t * d->K + k] == e) out[n++] = t * d->K + k;
    }
    return n;
}

/* ---------------------------------------------------------------------------
 * Expert-weight gradients over a list of tokens (tokens == NULL: all T),
 * summed over each expert's rows in ascending flat slot order:
 *   dW_down[e,j,i] = sum_rows do_j h_i
 *   dW_gate[e,i,c] = sum_rows dg_i x_c
 *   dW_up[e,i,c]   = sum_rows du_i x_c
 * Experts with no rows get exact zeros.  One thread per expert.
 * ------------------------------------------------------------------------- */
int moe_oracle_backward_dw(const moe_oracle_dims *d, const double *x,
                           const double *w_gate, const double *w_up,
                           const double *w_down, const int32_t *idx,
                           const double *w, const double *dy, int64_t ntok,
                           const int64_t *tokens, double *dw_gate,
                           double *dw_up, double *dw_down) {
    if (!dims_ok(d) || !x || !w_gate || !w_up || !w_down || !idx || !w ||
        !dy || !dw_gate || !dw_up || !dw_down)
        return ORACLE_BAD_ARG;
    if (!tokens) ntok = d->T;
    const int D = d->D, I = d->I, E = d->E, K = d->K;
    layer_t L = {d, x, w_gate, w_up, w_down};
    int status = ORACLE_OK;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (5 * (size_t)I + D));
        int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ntok * K + 1));
        if (!buf || !rows) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        }
#pragma omp for schedule(dynamic, 1)
        for (int e = 0; e < E; ++e) {
            if (!buf || !rows) continue;
            double *g = buf, *u = buf + I, *h = buf + 2 * I;
            double *dg = buf + 3 * I, *du = buf + 4 * I, *dov = buf + 5 * I;
            double *dwg = dw_gate + (size_t)e * I * D;
            double *dwu = dw_up + (size_t)e * I * D;
            double *dwd = dw_down + (size_t)e * D * I;
            memset(dwg, 0, sizeof(double) * (size_t)I * D);
            memset(dwu, 0, sizeof(double) * (size_t)I * D);
            memset(dwd, 0, sizeof(double) * (size_t)D * I);
            int64_t n = rows_of_expert(d, idx, ntok, tokens, e, rows);
            for (int64_t r = 0; r < n; ++r) {
                int64_t f = rows[r], t = f / K;
                const double *xt = x + t * D;
                expert_forward(&L, e, xt, g, u, h, NULL);
                for (int j = 0; j < D; ++j) dov[j] = w[f] * dy[t * D + j];
                expert_backward(&L, e, g, u, dov, dg, du);
                for (int j = 0; j < D; ++j)
                    for (int i = 0; i < I; ++i) dwd[(size_t)j * I + i] += dov[j] * h[i];
                for (int i = 0; i < I; ++i)
                    for (int c = 0; c < D; ++c) {
                        dwg[(size_t)i * D + c] += dg[i] * xt[c];
                        dwu[(size_t)i * D + c] += du[i] * xt[c];
                    }
            }
        }
        free(buf);
        free(rows);
    }
    return status;
}

/* ---------------------------------------------------------------------------
 * Single expert-weight-gradient entries, for spot checks at sizes where the
 * full gradient is too slow.  which: 0 = dW_gate[e,r,c] (r < I, c < D),
 * 1 = dW_up[e,r,c], 2 = dW_down[e,r,c] (r < D, c < I).  Same definitions and
 * the same row order as moe_oracle_backward_dw, over all T tokens; only the
 * components that the entry needs are evaluated.
 * ------------------------------------------------------------------------- */
int moe_oracle_dw_entries(const moe_oracle_dims *d, const double *x,
                          const double *w_gate, const double *w_up,
                          const double *w_down, const int32_t *idx,
                          const double *w, const double *dy, int64_t n,
                          const int32_t *which, const int32_t *ee,
                          const int32_t *rr, const int32_t *cc, double *out) {
    if (!dims_ok(d) || !x || !w_gate || !w_up || !w_down || !idx || !w ||
        !dy || !which || !ee || !rr || !cc || !out)
        return ORACLE_BAD_ARG;
    const int D = d->D, I = d->I, K = d->K;
    for (int64_t q = 0; q < n; ++q) {
        int lim_r = which[q] == 2 ? D : I, lim_c = which[q] == 2 ? I : D;
        if (which[q] < 0 || which[q] > 2 || ee[q] < 0 || ee[q] >= d->E ||
            rr[q] < 0 || rr[q] >= lim_r || cc[q] < 0 || cc[q] >= lim_c)
            return ORACLE_BAD_ARG;
    }
    layer_t L = {d, x, w_gate, w_up, w_down};
    int status = ORACLE_OK;
#pragma omp parallel
    {
        double *dov = (double *)malloc(sizeof(double) * (size_t)D);
        int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(d->T * K + 1));
        if (!dov || !rows) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n; ++q) {
            if (!dov || !rows) continue;
            int e = ee[q];
            int64_t nr = rows_of_expert(d, idx, d->T, NULL, e, rows);
            double acc = 0.0;
            for (int64_t r = 0; r < nr; ++r) {
                int64_t f = rows[r], t = f / K;
                const double *xt = x + t * D;
                double g, u;
                if (which[q] == 2) {
                    int j = rr[q], i = cc[q];
                    gate_up_at(&L, e, i, xt, &g, &u);
                    acc += (w[f] * dy[t * D + j]) * swiglu(g, u);
                } else {
                    int i = rr[q], c = cc[q];
                    for (int j = 0; j < D; ++j) dov[j] = w[f] * dy[t * D + j];
                    gate_up_at(&L, e, i, xt, &g, &u);
                    double dg, du;
                    swiglu_backward(down_t_at(&L, e, i, dov), g, u, &dg, &du);
                    acc += (which[q] == 0 ? dg : du) * xt[c];
                }
            }
            out[q] = acc;
        }
        free(dov);
        free(rows);
    }
    return status;
}

/* ---------------------------------------------------------------------------
 * Router projection:  logits[t, e] = sum_d x[t, d] * w_r[d, e]   (d ascending)
 * x [T, D], w_r [D, E] -> logits [T, E].
 * ------------------------------------------------------------------------- */
int moe_oracle_router_logits(const moe_oracle_dims *d, const double *x,
                             const double *w_r, double *logits) {
    if (!dims_ok(d) || !x || !w_r || !logits) return ORACLE_BAD_ARG;
    const int D = d->D, E = d->E;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < d->T; ++t) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int j = 0; j < D; ++j) s += x[t * D + j] * w_r[(size_t)j * E + e];
            logits[t * E + e] = s;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Router backward, with the selection held fixed (the top-K choice is
 * piecewise constant in the logits).  drw[t, k] = dL/dw[t, k] is the
 * router-weight gradient of the layer.
 *   score 0, w_k = exp(l_k) / sum_{j in selected} exp(l_j):
 *     dw_k/dl_m = w_k (delta_km - w_m) for selected m, so
 *     dl[t, idx_m] = w_m (drw_m - sum_k w_k drw_k);  0 for unselected experts
 *   score 1, w_k = sigmoid(l_k):
 *     dl[t, idx_k] = drw_k w_k (1 - w_k)
 *   dw_r[d, e] = sum_t x[t, d] dl[t, e]        (t ascending)
 *   dx_r[t, d] = sum_e dl[t, e] w_r[d, e]      (e ascending)
 * dl [T, E], dw_r [D, E], dx_r [T, D]  (dx_r is the router's contribution to
 * the layer's input gradient; the expert path adds its own).
 * ------------------------------------------------------------------------- */
int moe_oracle_router_backward(const moe_oracle_dims *d, const double *x,
                               const double *w_r, const int32_t *idx,
                               const double *w, const double *drw, double *dl,
                               double *dw_r, double *dx_r) {
    if (!dims_ok(d) || !x || !w_r || !idx || !w || !drw || !dl || !dw_r || !dx_r)
        return ORACLE_BAD_ARG;
    const int D = d->D, E = d->E, K = d->K;
    const int64_t T = d->T;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double *dlt = dl + t * E;
        for (int e = 0; e < E; ++e) dlt[e] = 0.0;
        const double *wt = w + t * K, *gt = drw + t * K;
        if (d->score == 0) {
            double s = 0.0;
            for (int k = 0; k < K; ++k) s += wt[k] * gt[k];
            for (int m = 0; m < K; ++m) dlt[idx[t * K + m]] = wt[m] * (gt[m] - s);
        } else {
            for (int k = 0; k < K; ++k) dlt[idx[t * K + k]] = gt[k] * wt[k] * (1.0 - wt[k]);
        }
    }
#pragma omp parallel for schedule(static)
    for (int j = 0; j < D; ++j) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t t = 0; t < T; ++t) s += x[t * D + j] * dl[t * E + e];
            dw_r[(size_t)j * E + e] = s;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < D; ++j) {
            double s = 0.0;
            for (int e = 0; e < E; ++e) s += dl[t * E + e] * w_r[(size_t)j * E + e];
            dx_r[t * D + j] = s;
        }
    }
    return ORACLE_OK;
}

/* Threads the OpenMP loops above run on (what a timing of the oracle used). */
int32_t moe_oracle_threads(void) { return (int32_t)omp_get_max_threads(); }
