/*
 * oracle.c -- plain, slow, single-threaded CPU reference for one MoE layer's
 * hot path: router top-k gating, demand counting, the equal-load replica plan,
 * dispatch permutation, the SwiGLU expert FFN, the gate-weighted combine and
 * the load statistics; and the layer's backward (combine, expert FFN,
 * dispatch, gate).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file. It shares no code, header,
 * table or helper with the HIP library and must never be used as a fallback
 * for it.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -lm
 * (no contraction, so every float expression below rounds exactly as written).
 *
 * Sources (web pages, cited by title and section):
 *  [MoonEP]  "Moonshot AI drops MoonEP, claims 2.5x scaling boost for
 *            trillion-parameter models" (news article), paragraphs 2-4.
 *  [Primer]  "DeepEP-on-EFA Guidance, section 1: what is MoE", the
 *            four-phase pipeline (router, dispatch, grouped GEMM, combine).
 *  [Hotspot] "MoE Load Balancing: Find Expert Hotspots", sections
 *            "Separate expert demand from rank placement",
 *            "Make expert capacity, overflow, and padding explicit",
 *            "Count remote routes before celebrating balance",
 *            "Work the 16-token hotspot fixture".
 *  [Interview] "MoE load balancing: 90/10 routing in production" (summary
 *            and editor's note): per-expert bias kept out of the gate.
 *
 * One function follows no page: orc_bias_update (an assumed update rule,
 * labelled as such below). The router's linear layer, the fixed-capacity and
 * repacking rules and the replica slot assignment are readings of the pages,
 * also labelled.
 *
 * Every function with a pin in tests/ is pinned there; none is "parity
 * unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_ERR_NONFINITE 1
#define ORC_ERR_RANGE 2
#define ORC_ERR_REPEAT 4

/* ------------------------------------------------------------------------ */
/* Router: [Primer] phase (a) -- score every expert per token, keep the top-k,
 * emit expert ids plus per-expert combine weights.
 * [Interview] editor's note: the balancing bias lives outside the gate, so it
 * shifts which experts are selected but not the weights they get.
 *
 * Selection score: s_e = logit_e + bias_e, one IEEE fp32 add. The k winners
 * are taken in order of decreasing score; equal scores go to the lower id.
 * Weights: softmax of the RAW logits over the selected experts (computed in
 * double), i.e. the full softmax renormalised over the top-k.
 * Returns an error word: bit 1 if any logit or bias is not finite.          */
int orc_route(int T, int E, int k, const float *logits, const float *bias,
              int32_t *ids, double *w)
{
    int err = 0;
    unsigned char *taken = (unsigned char *)malloc((size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E && bias; ++e)
        if (!isfinite(bias[e])) err |= ORC_ERR_NONFINITE;
    for (int t = 0; t < T; ++t) {
        const float *row = logits + (size_t)t * E;
        for (int e = 0; e < E; ++e)
            if (!isfinite(row[e])) err |= ORC_ERR_NONFINITE;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            float best_s = 0.0f;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                float s = row[e] + (bias ? bias[e] : 0.0f);
                /* strict '>' while scanning ids upward: ties keep the lower id */
                if (best < 0 || s > best_s) {
                    best = e;
                    best_s = s;
                }
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        double m = -INFINITY;
        for (int j = 0; j < k; ++j) {
            double l = row[ids[(size_t)t * k + j]];
            if (l > m) m = l;
        }
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += exp((double)row[ids[(size_t)t * k + j]] - m);
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = exp((double)row[ids[(size_t)t * k + j]] - m) / den;
    }
    free(taken);
    return err;
}

/* ------------------------------------------------------------------------ */
/* Demand counting: [Hotspot] "Separate expert demand from rank placement"
 * (count assignments per expert, ignoring ownership; then sum by rank under
 * the contiguous home mapping {0,1},{2,3},...) and "Work the 16-token hotspot
 * fixture" (stop when an id is unknown or a token repeats an expert).
 *
 * counts[e]  = number of (t,j) with ids[t][j] == e
 * offsets    = exclusive prefix of counts, E+1 entries
 * eidx[t*k+j]= number of EARLIER assignments in flat order t*k+j that chose
 *              the same expert (stable within-expert index)
 * rank_load[r] = sum of counts over r's home experts e / (E/R) == r
 * Returns an error word: bit 2 id out of range, bit 4 repeated id in a token.
 * Out-of-range ids are not counted.                                        */
int orc_count(int T, int k, int E, int R, const int32_t *ids, int32_t *counts,
              int32_t *offsets, int32_t *eidx, int32_t *rank_load)
{
    int err = 0;
    int n = E / R;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t e = ids[(size_t)t * k + j];
            for (int jj = 0; jj < j; ++jj)
                if (ids[(size_t)t * k + jj] == e) err |= ORC_ERR_REPEAT;
            if (e < 0 || e >= E) {
                err |= ORC_ERR_RANGE;
                eidx[(size_t)t * k + j] = -1;
                continue;
            }
            eidx[(size_t)t * k + j] = counts[e];
            counts[e] += 1;
        }
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int r = 0; r < R; ++r) {
        int32_t s = 0;
        for (int e = r * n; e < (r + 1) * n; ++e) s += counts[e];
        rank_load[r] = s;
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Equal-load replica plan: [MoonEP] paragraph 3 -- every rank receives exactly
 * the same number of tokens however skewed the routing, by planning a few
 * redundant expert copies straight from the router output; paragraph 4 --
 * with as many prefetch slots as experts per rank, every expert a rank's GEMM
 * touches is local.
 *
 * The pages give the invariant, not the algorithm. The rule below is the
 * reading adopted here (an alias-method style transfer):
 *   quota C_r = floor(N/R) + [r < N mod R]; window W_r = sum_{r'<r} C_r'.
 *   L_r starts as the home rank load; rem_e starts as counts[e].
 *   Repeat while some not-yet-filled rank has L_r < C_r:
 *     s = that rank with the largest deficit C_s - L_s (ties: lower rank);
 *     l = the rank with the largest excess L_l - C_l (ties: lower rank);
 *     move d = C_s - L_s assignments from l's home experts to s, draining
 *       l's experts in order of (count desc, id asc), skipping empty ones;
 *     L_l -= d, L_s = C_s, s is filled (a donor pushed below its quota
 *       becomes a deficit rank later and is filled once).
 *   What is left of each expert stays home.
 * Layout: in window r, segments are ordered by expert id (home and replica
 * mixed) from W_r. An expert's pieces are ordered by rank; its assignments,
 * in eidx order, fill those pieces in that order.
 * Tables (unused entries are -1):
 *   quota[R], win_off[R+1], seg_num[R], seg_{expert,row,cnt}[R][2n],
 *   slots_needed[R], slot_expert[R][n] (replica experts of r ascending),
 *   donor[R] (rank that filled r, -1 if none), piece_num[E],
 *   piece_{rank,row,cnt}[E][R].
 * Returns 0, or -1 if E is not a multiple of R (a caller error).            */
int orc_plan(int E, int R, const int32_t *counts, int32_t *quota, int32_t *win_off,
             int32_t *seg_num, int32_t *seg_expert, int32_t *seg_row, int32_t *seg_cnt,
             int32_t *slots_needed, int32_t *slot_expert, int32_t *donor,
             int32_t *piece_num, int32_t *piece_rank, int32_t *piece_row,
             int32_t *piece_cnt)
{
    if (R <= 0 || E % R != 0) return -1;
    const int n = E / R;
    int64_t N = 0;
    for (int e = 0; e < E; ++e) N += counts[e];

    int64_t *load = (int64_t *)calloc((size_t)R, sizeof(int64_t));
    int64_t *rem = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *take = (int64_t *)calloc((size_t)R * n, sizeof(int64_t)); /* take[s][i] from donor's i-th home expert */
    int *filled = (int *)calloc((size_t)R, sizeof(int));

    const int64_t q = N / R, extra = N % R;
    win_off[0] = 0;
    for (int r = 0; r < R; ++r) {
        quota[r] = (int32_t)(q + (r < extra ? 1 : 0));
        win_off[r + 1] = win_off[r] + quota[r];
        donor[r] = -1;
    }
    for (int e = 0; e < E; ++e) {
        rem[e] = counts[e];
        load[e / n] += counts[e];
    }

    for (;;) {
        int s = -1;
        int64_t best_def = 0;
        for (int r = 0; r < R; ++r) {
            int64_t def = (int64_t)quota[r] - load[r];
            if (!filled[r] && def > best_def) {
                best_def = def;
                s = r;
            }
        }
        if (s < 0) break;
        int l = -1;
        int64_t best_exc = 0;
        for (int r = 0; r < R; ++r) {
            int64_t exc = load[r] - (int64_t)quota[r];
            if (exc > best_exc) {
                best_exc = exc;
                l = r;
            }
        }
        if (l < 0) break; /* cannot happen: total load equals total quota */
        int64_t d = best_def;
        while (d > 0) {
            /* next expert in l's donor order that still has assignments */
            int pick = -1;
            for (int e = l * n; e < (l + 1) * n; ++e) {
                if (rem[e] <= 0) continue;
                if (pick < 0 || counts[e] > counts[pick]) pick = e;
            }
            if (pick < 0) break; /* cannot happen: a donor holds >= d */
            int64_t t = rem[pick] < d ? rem[pick] : d;
            take[(size_t)s * n + (pick - l * n)] += t;
            rem[pick] -= t;
            d -= t;
        }
        donor[s] = l;
        load[l] -= best_def;
        load[s] = quota[s];
        filled[s] = 1;
    }

    /* per-rank segments, expert id ascending */
    for (int r = 0; r < R; ++r) {
        int32_t row = win_off[r];
        int ns = 0, nslot = 0;
        for (int i = 0; i < 2 * n; ++i) {
            seg_expert[(size_t)r * 2 * n + i] = -1;
            seg_row[(size_t)r * 2 * n + i] = -1;
            seg_cnt[(size_t)r * 2 * n + i] = -1;
        }
        for (int i = 0; i < n; ++i) slot_expert[(size_t)r * n + i] = -1;
        for (int e = 0; e < E; ++e) {
            int64_t c = 0;
            if (e / n == r) c = rem[e];
            else if (donor[r] >= 0 && e / n == donor[r]) c = take[(size_t)r * n + (e - donor[r] * n)];
            if (c <= 0) continue;
            seg_expert[(size_t)r * 2 * n + ns] = e;
            seg_row[(size_t)r * 2 * n + ns] = row;
            seg_cnt[(size_t)r * 2 * n + ns] = (int32_t)c;
            row += (int32_t)c;
            ns++;
            if (e / n != r) slot_expert[(size_t)r * n + nslot++] = e;
        }
        seg_num[r] = ns;
        slots_needed[r] = nslot;
    }

    /* per-expert pieces, rank ascending */
    for (int e = 0; e < E; ++e) {
        int np = 0;
        for (int r = 0; r < R; ++r) {
            piece_rank[(size_t)e * R + r] = -1;
            piece_row[(size_t)e * R + r] = -1;
            piece_cnt[(size_t)e * R + r] = -1;
        }
        for (int r = 0; r < R; ++r) {
            for (int i = 0; i < seg_num[r]; ++i) {
                if (seg_expert[(size_t)r * 2 * n + i] != e) continue;
                piece_rank[(size_t)e * R + np] = r;
                piece_row[(size_t)e * R + np] = seg_row[(size_t)r * 2 * n + i];
                piece_cnt[(size_t)e * R + np] = seg_cnt[(size_t)r * 2 * n + i];
                np++;
            }
        }
        piece_num[e] = np;
    }
    free(load);
    free(rem);
    free(take);
    free(filled);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch: [Primer] phase (b) -- each token goes to where its k experts are
 * (only to those k); [MoonEP] paragraph 3 -- zero-copy placement into static
 * shapes: each assignment is written once, straight to its final row.
 * Assignment (t,j) of expert e with stable index v lands in the piece p of e
 * with cum_p <= v < cum_p + cnt_p (cum = running sum of piece counts in rank
 * order), at row piece_row[p] + v - cum_p. buf[row] = x[t], row_src[row] = t.
 * Rows are copied byte for byte (row_bytes each).                          */
void orc_permute(int T, int k, int E, int R, size_t row_bytes, const void *x,
                 const int32_t *ids, const int32_t *eidx, const int32_t *piece_num,
                 const int32_t *piece_row, const int32_t *piece_cnt, void *buf,
                 int32_t *dest_row, int32_t *row_src)
{
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            int v = eidx[(size_t)t * k + j];
            int dest = -1, cum = 0;
            for (int p = 0; p < piece_num[e]; ++p) {
                int c = piece_cnt[(size_t)e * R + p];
                if (v < cum + c) {
                    dest = piece_row[(size_t)e * R + p] + (v - cum);
                    break;
                }
                cum += c;
            }
            dest_row[(size_t)t * k + j] = dest;
            if (dest < 0) continue;
            row_src[dest] = t;
            memcpy((char *)buf + (size_t)dest * row_bytes, (const char *)x + (size_t)t * row_bytes,
                   row_bytes);
        }
    }
    (void)E;
}

/* ------------------------------------------------------------------------ */
/* Router scores: [Primer] phase (a), the router scores every expert for
 * every token. The pages do not print the router; the plain reading is a
 * linear layer, logit[t][e] = sum_h x[t][h] * W_r[e][h] (W_r row-major
 * [E][H]), evaluated here in double from the given (already rounded)
 * inputs. The top-k step that follows is orc_route.                       */
void orc_router_logits(int T, int E, int H, const float *x, const float *w_router, double *out)
{
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += (double)x[(size_t)t * H + h] * (double)w_router[(size_t)e * H + h];
            out[(size_t)t * E + e] = acc;
        }
}

/* Bias update -- NOT ON THE PAGES, a labelled assumption. [Interview] keeps
 * a per-expert balancing bias out of the gate (it shifts selection only) but
 * prints no update rule; [MoonEP] paragraph 2 only asks that maxvio go to
 * zero. The rule assumed here is the sign rule of auxiliary-loss-free
 * balancing: an expert above the mean demand N/E loses gamma, one below it
 * gains gamma, one at the mean keeps its bias. In fp32: delta = +-gamma (as
 * float) or 0, decided in integers by the sign of N - E * counts[e], then one
 * fp32 add.                                                                */
void orc_bias_update(int E, int64_t N, const int32_t *counts, float gamma, float *bias)
{
    for (int e = 0; e < E; ++e) {
        int64_t s = N - (int64_t)E * counts[e];
        float delta = s > 0 ? gamma : (s < 0 ? -gamma : 0.0f);
        bias[e] = bias[e] + delta;
    }
}

/* ------------------------------------------------------------------------ */
/* Fixed-capacity dispatch: the static-capacity baseline that the equal-load
 * plan replaces.
 * [Hotspot] "Make expert capacity, overflow, and padding explicit": every
 * expert has the same capacity; demand above it overflows (the assignment is
 * dropped) and the unused slots below it are padding.
 * Reading: an expert keeps its first cap assignments in stable order
 * (eidx < cap). The buffer is [E][cap] rows: assignment (t,j) of expert e
 * with eidx v < cap goes to row e*cap + v; padding rows are zero; a dropped
 * (or out-of-range) assignment gets dest_row = -1.                          */
void orc_capacity_dispatch(int T, int k, int E, int cap, size_t row_bytes, const void *x,
                           const int32_t *ids, const int32_t *eidx, void *buf, int32_t *dest_row)
{
    memset(buf, 0, (size_t)E * (size_t)cap * row_bytes);
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            int v = eidx[(size_t)t * k + j];
            int dest = -1;
            if (e >= 0 && e < E && v >= 0 && v < cap) dest = e * cap + v;
            dest_row[(size_t)t * k + j] = dest;
            if (dest < 0) continue;
            memcpy((char *)buf + (size_t)dest * row_bytes, (const char *)x + (size_t)t * row_bytes,
                   row_bytes);
        }
    }
}

/* Repacking (EPLB-style static placement, the other baseline): assign the E
 * experts to the R ranks, n = E/R each, so that rank demand is even.
 * [Hotspot] "Separate expert demand from rank placement": for the fixture
 * demand, the mapping {0,7},{1,6},{2,5},{3,4} takes rank demand from
 * [15,9,5,3] to [10,8,7,7]. The pages print the mapping, not the rule.
 * Reading: greedy balanced packing -- experts in order of decreasing demand
 * (equal demand: lower id first) each go to the least-loaded rank that still
 * holds fewer than n experts (equal load: lower rank). It reproduces the
 * printed mapping. mapping[e] = rank of expert e.                          */
void orc_repack(int E, int R, const int32_t *counts, int32_t *mapping)
{
    int n = E / R;
    int *order = (int *)malloc(sizeof(int) * (size_t)E);
    int64_t *load = (int64_t *)calloc((size_t)R, sizeof(int64_t));
    int *held = (int *)calloc((size_t)R, sizeof(int));
    for (int e = 0; e < E; ++e) order[e] = e;
    /* selection sort by (count desc, id asc) */
    for (int i = 0; i < E; ++i) {
        int best = i;
        for (int j = i + 1; j < E; ++j) {
            int a = order[j], b = order[best];
            if (counts[a] > counts[b] || (counts[a] == counts[b] && a < b)) best = j;
        }
        int tmp = order[i];
        order[i] = order[best];
        order[best] = tmp;
    }
    for (int i = 0; i < E; ++i) {
        int e = order[i], best = -1;
        for (int r = 0; r < R; ++r)
            if (held[r] < n && (best < 0 || load[r] < load[best])) best = r;
        mapping[e] = best;
        load[best] += counts[e];
        held[best] += 1;
    }
    free(order);
    free(load);
    free(held);
}

/* ------------------------------------------------------------------------ */
/* Backward of the layer. [Primer] phases (a)-(d) run in reverse: combine,
 * expert FFN, dispatch, router gate. [MoonEP] paragraph 3: in training the
 * replicas' weight gradients are reduced into the home expert; on one GPU
 * every piece of an expert contributes to that expert's one gradient, so the
 * reduction is the sum over all of its rows. The chain rule written out, in
 * double, from the same rounded inputs as the forward functions above.      */

/* Combine: out[t] = sum_j w[t][j] * y[dest[t][j]], so
 *   dy[dest[t][j]] += w[t][j] * dout[t]   (rows nobody reads stay zero),
 *   dw[t][j] = <dout[t], y[dest[t][j]]>   (zero for a dropped assignment). */
void orc_combine_backward(int T, int k, int H, int64_t nrows, const double *dout,
                          const double *y, const int32_t *dest_row, const double *w,
                          double *dy, double *dw)
{
    memset(dy, 0, sizeof(double) * (size_t)nrows * H);
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int d = dest_row[(size_t)t * k + j];
            double acc = 0.0;
            if (d >= 0 && d < nrows) {
                for (int c = 0; c < H; ++c) {
                    dy[(size_t)d * H + c] += w[(size_t)t * k + j] * dout[(size_t)t * H + c];
                    acc += dout[(size_t)t * H + c] * y[(size_t)d * H + c];
                }
            }
            dw[(size_t)t * k + j] = acc;
        }
    }
}

/* SwiGLU expert FFN on nrows rows of one expert, backward. With
 * g = W_gate x, u = W_up x, s = 1/(1+e^-g), h = g s u, y = W_down h:
 *   dh = W_down^T dy;  du = dh g s;  dg = dh u s (1 + g (1 - s));
 *   dx = W_gate^T dg + W_up^T du;
 *   dW_down += dy h^T, dW_gate += dg x^T, dW_up += du x^T  (accumulated).
 * x [nrows][H], w_gate/w_up [F][H], w_down [H][F] (float values); dy, dx
 * [nrows][H] and the weight gradients (same shapes as the weights) double. */
void orc_ffn_backward_rows(int nrows, int H, int F, const float *x, const double *dy,
                           const float *w_gate, const float *w_up, const float *w_down,
                           double *dx, double *dw_gate, double *dw_up, double *dw_down)
{
    size_t nf = (size_t)(F > 0 ? F : 1);
    double *g = (double *)malloc(sizeof(double) * nf);
    double *u = (double *)malloc(sizeof(double) * nf);
    double *dg = (double *)malloc(sizeof(double) * nf);
    double *du = (double *)malloc(sizeof(double) * nf);
    for (int i = 0; i < nrows; ++i) {
        const float *xr = x + (size_t)i * H;
        const double *dyr = dy + (size_t)i * H;
        for (int f = 0; f < F; ++f) {
            double a = 0.0, b = 0.0;
            for (int c = 0; c < H; ++c) {
                a += (double)w_gate[(size_t)f * H + c] * (double)xr[c];
                b += (double)w_up[(size_t)f * H + c] * (double)xr[c];
            }
            g[f] = a;
            u[f] = b;
        }
        for (int f = 0; f < F; ++f) {
            double s = 1.0 / (1.0 + exp(-g[f]));
            double h = g[f] * s * u[f];
            double dh = 0.0;
            for (int o = 0; o < H; ++o) {
                dh += (double)w_down[(size_t)o * F + f] * dyr[o];
                dw_down[(size_t)o * F + f] += dyr[o] * h;
            }
            du[f] = dh * g[f] * s;
            dg[f] = dh * u[f] * s * (1.0 + g[f] * (1.0 - s));
        }
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int f = 0; f < F; ++f)
                acc += (double)w_gate[(size_t)f * H + c] * dg[f] + (double)w_up[(size_t)f * H + c] * du[f];
            dx[(size_t)i * H + c] = acc;
        }
        for (int f = 0; f < F; ++f) {
            for (int c = 0; c < H; ++c) {
                dw_gate[(size_t)f * H + c] += dg[f] * (double)xr[c];
                dw_up[(size_t)f * H + c] += du[f] * (double)xr[c];
            }
        }
    }
    free(g);
    free(u);
    free(dg);
    free(du);
}

/* Dispatch: buf[dest[t][j]] = x[t], so dx[t] = sum_j dbuf[dest[t][j]]. */
void orc_permute_backward(int T, int k, int H, int64_t nrows, const double *dbuf,
                          const int32_t *dest_row, double *dx)
{
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int d = dest_row[(size_t)t * k + j];
                if (d >= 0 && d < nrows) acc += dbuf[(size_t)d * H + c];
            }
            dx[(size_t)t * H + c] = acc;
        }
    }
}

/* Gate: w[t][j] = softmax over the selected experts' RAW logits, so
 *   dlogits[t][ids[t][j]] = w_j (dw_j - sum_j' w_j' dw_j'),
 * zero for experts not selected (a small change of their logit does not
 * change the selection or the weights). The balancing bias only selects and
 * gets no gradient. */
void orc_route_backward(int T, int E, int k, const int32_t *ids, const double *w,
                        const double *dw, double *dlogits)
{
    memset(dlogits, 0, sizeof(double) * (size_t)T * E);
    for (int t = 0; t < T; ++t) {
        double dot = 0.0;
        for (int j = 0; j < k; ++j) dot += w[(size_t)t * k + j] * dw[(size_t)t * k + j];
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            if (e >= 0 && e < E)
                dlogits[(size_t)t * E + e] = w[(size_t)t * k + j] * (dw[(size_t)t * k + j] - dot);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Replica weight slots: [MoonEP] paragraph 3 -- the planner's redundant
 * expert copies are prefetched into a fixed number of weight slots per rank;
 * paragraph 4 -- as many slots as experts per rank make every expert the
 * grouped GEMM touches local, and a few slots usually suffice.
 * Reading: rank r's replica experts take its slots in the order of
 * slot_expert[r] (ascending expert id); slot j < S holds a copy of that
 * expert's three projections. Segment i of rank r (expert e) reads
 *   - the home weights when r is e's home rank (e / n == r),
 *   - slot j when e is rank r's j-th replica expert and j < S,
 *   - the home weights otherwise (a non-local read; orc_stats counts its
 *     rows as non-local).
 * src[r][i] = j, or -1 for the home weights; -2 for i >= seg_num[r].        */
void orc_slot_sources(int E, int R, int S, const int32_t *seg_num, const int32_t *seg_expert,
                      const int32_t *slot_expert, int32_t *src)
{
    int n = E / R;
    for (int r = 0; r < R; ++r) {
        for (int i = 0; i < 2 * n; ++i) {
            int32_t *o = src + (size_t)r * 2 * n + i;
            if (i >= seg_num[r]) {
                *o = -2;
                continue;
            }
            int e = seg_expert[(size_t)r * 2 * n + i];
            *o = -1;
            if (e / n == r) continue;
            for (int q = 0; q < n && q < S; ++q) {
                if (slot_expert[(size_t)r * n + q] == e) {
                    *o = q;
                    break;
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Expert FFN: [Primer] phase (c), each expert's feed-forward network on the
 * rows it received. The expert is a SwiGLU FFN:
 *   g = W_gate x, u = W_up x, h = silu(g) * u, silu(z) = z / (1 + e^-z),
 *   y = W_down h,
 * with W_gate, W_up of shape [F][H] and W_down of shape [H][F] (row-major),
 * evaluated in double from the given (already rounded) input values.
 * nrows rows of x (each H floats) -> nrows rows of y (each H doubles).     */
void orc_ffn_rows(int nrows, int H, int F, const float *x, const float *w_gate,
                  const float *w_up, const float *w_down, double *y)
{
    double *h = (double *)malloc(sizeof(double) * (size_t)(F > 0 ? F : 1));
    for (int i = 0; i < nrows; ++i) {
        const float *xr = x + (size_t)i * H;
        for (int f = 0; f < F; ++f) {
            double g = 0.0, u = 0.0;
            const float *wg = w_gate + (size_t)f * H;
            const float *wu = w_up + (size_t)f * H;
            for (int c = 0; c < H; ++c) {
                g += (double)wg[c] * (double)xr[c];
                u += (double)wu[c] * (double)xr[c];
            }
            h[f] = g / (1.0 + exp(-g)) * u;
        }
        for (int o = 0; o < H; ++o) {
            double acc = 0.0;
            const float *wd = w_down + (size_t)o * F;
            for (int f = 0; f < F; ++f) acc += (double)wd[f] * h[f];
            y[(size_t)i * H + o] = acc;
        }
    }
    free(h);
}

/* ------------------------------------------------------------------------ */
/* Combine: [Primer] phase (d) -- expert outputs go back to their token and are
 * summed with the gate weights (the transpose of dispatch).
 *   out[t] = sum_{j=0..k-1} w[t][j] * y[dest_row[t][j]]  (+ shared[t])
 * summed in j order, in double. shared may be NULL.                        */
void orc_combine(int T, int k, int H, const double *y, const int32_t *dest_row,
                 const double *w, const double *shared, double *out)
{
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int d = dest_row[(size_t)t * k + j];
                if (d < 0) continue; /* dropped by a fixed capacity: contributes nothing */
                acc += w[(size_t)t * k + j] * y[(size_t)d * H + c];
            }
            if (shared) acc += shared[(size_t)t * H + c];
            out[(size_t)t * H + c] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Statistics.
 * [Hotspot] "Separate expert demand from rank placement": balancedness is the
 *   average load divided by the maximum load (not the reverse).
 * [MoonEP] paragraph 2: maxvio scores a perfectly balanced load as zero. The
 *   formula is not printed; the reading here is max/mean - 1, i.e.
 *   (max * M - total) / total for M bins, 0 when the total is 0.
 * [Hotspot] "Make expert capacity, overflow, and padding explicit":
 *   capacity = ceil(assignments / experts * factor); processed = min(d,cap),
 *   overflow = max(d-cap,0), padding = max(cap-d,0), from raw demand.
 * [Hotspot] "Count remote routes": an assignment is remote when the token's
 *   origin rank differs from its destination rank.                         */
typedef struct {
    int64_t N;
    int32_t E, R;
    int32_t max_count, min_count, active_experts;
    double maxvio_expert, balancedness_expert;
    int32_t home_max;
    double maxvio_rank_home, balancedness_rank_home;
    int32_t mapped_max;
    double maxvio_rank_mapped, balancedness_rank_mapped;
    int32_t planned_max, planned_min;
    double maxvio_rank_planned, balancedness_rank_planned;
    int32_t capacity;
    int64_t processed, overflow, padding;
    int64_t remote_home, remote_mapped, remote_planned;
    int32_t replica_pieces, max_slots_needed, ranks_over_slots;
    int64_t nonlocal_rows;
} orc_stats_t;

static double orc_maxvio(int64_t mx, int M, int64_t total)
{
    if (total <= 0) return 0.0;
    return (double)(mx * (int64_t)M - total) / (double)total;
}

static double orc_balancedness(int64_t mx, int M, int64_t total)
{
    if (mx <= 0) return 1.0;
    return (double)total / (double)(mx * (int64_t)M);
}

/* Capacity from the page's formula, evaluated in the page's order. */
int32_t orc_capacity(int64_t N, int E, double factor)
{
    return (int32_t)ceil((double)N / (double)E * factor);
}

/* Share of the g hottest experts relative to their even share:
 * (sum of the g largest counts / N) / (g / E). [Interview] summary: 90% of
 * tokens on 26 of 256 experts is about nine times their share.             */
double orc_hot_share(int E, const int32_t *counts, int g)
{
    int64_t N = 0, top = 0;
    unsigned char *used = (unsigned char *)calloc((size_t)E, 1);
    for (int e = 0; e < E; ++e) N += counts[e];
    for (int i = 0; i < g; ++i) {
        int b = -1;
        for (int e = 0; e < E; ++e)
            if (!used[e] && (b < 0 || counts[e] > counts[b])) b = e;
        used[b] = 1;
        top += counts[b];
    }
    free(used);
    if (N == 0 || g == 0) return 0.0;
    return ((double)top / (double)N) / ((double)g / (double)E);
}

/* counts[E]; mapping[E] (may be NULL); origin[T] (may be NULL: t mod R);
 * ids[T*k] and dest_row[T*k] (dest_row may be NULL); the plan tables for the
 * planned statistics (may all be NULL). slots = S. The optional outputs
 * home_load / mapped_load / planned_load [R] receive the rank load vectors. */
void orc_stats(int T, int k, int E, int R, int S, const int32_t *counts, const int32_t *ids,
               const int32_t *mapping, const int32_t *origin, const int32_t *dest_row,
               const int32_t *win_off, const int32_t *seg_num, const int32_t *seg_expert,
               const int32_t *seg_cnt, const int32_t *slots_needed, const int32_t *slot_expert,
               double capacity_factor, int32_t *home_load, int32_t *mapped_load,
               int32_t *planned_load, orc_stats_t *out)
{
    const int n = E / R;
    memset(out, 0, sizeof(*out));
    out->E = E;
    out->R = R;
    int64_t N = 0;
    int32_t mx = 0, mn = 0;
    for (int e = 0; e < E; ++e) {
        N += counts[e];
        if (counts[e] > mx) mx = counts[e];
        if (e == 0 || counts[e] < mn) mn = counts[e];
        if (counts[e] > 0) out->active_experts++;
    }
    out->N = N;
    out->max_count = mx;
    out->min_count = mn;
    out->maxvio_expert = orc_maxvio(mx, E, N);
    out->balancedness_expert = orc_balancedness(mx, E, N);

    int64_t *rl = (int64_t *)calloc((size_t)R, sizeof(int64_t));
    int64_t *rm = (int64_t *)calloc((size_t)R, sizeof(int64_t));
    for (int e = 0; e < E; ++e) {
        rl[e / n] += counts[e];
        if (mapping) rm[mapping[e]] += counts[e];
    }
    int64_t hm = 0, mm = 0;
    for (int r = 0; r < R; ++r) {
        if (rl[r] > hm) hm = rl[r];
        if (rm[r] > mm) mm = rm[r];
        if (home_load) home_load[r] = (int32_t)rl[r];
        if (mapped_load && mapping) mapped_load[r] = (int32_t)rm[r];
    }
    out->home_max = (int32_t)hm;
    out->maxvio_rank_home = orc_maxvio(hm, R, N);
    out->balancedness_rank_home = orc_balancedness(hm, R, N);
    if (mapping) {
        out->mapped_max = (int32_t)mm;
        out->maxvio_rank_mapped = orc_maxvio(mm, R, N);
        out->balancedness_rank_mapped = orc_balancedness(mm, R, N);
    }

    out->capacity = orc_capacity(N, E, capacity_factor);
    for (int e = 0; e < E; ++e) {
        int64_t c = counts[e], cap = out->capacity;
        out->processed += c < cap ? c : cap;
        out->overflow += c > cap ? c - cap : 0;
        out->padding += cap > c ? cap - c : 0;
    }

    for (int t = 0; t < T; ++t) {
        int o = origin ? origin[t] : t % R;
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            if (e / n != o) out->remote_home++;
            if (mapping && mapping[e] != o) out->remote_mapped++;
            if (dest_row && win_off) {
                int d = dest_row[(size_t)t * k + j], pr = 0;
                while (pr + 1 < R && d >= win_off[pr + 1]) pr++;
                if (pr != o) out->remote_planned++;
            }
        }
    }

    if (seg_num && seg_cnt && win_off) {
        int64_t pmax = 0, pmin = -1;
        for (int r = 0; r < R; ++r) {
            int64_t s = 0;
            for (int i = 0; i < seg_num[r]; ++i) s += seg_cnt[(size_t)r * 2 * n + i];
            if (planned_load) planned_load[r] = (int32_t)s;
            if (s > pmax) pmax = s;
            if (pmin < 0 || s < pmin) pmin = s;
        }
        out->planned_max = (int32_t)pmax;
        out->planned_min = (int32_t)(pmin < 0 ? 0 : pmin);
        out->maxvio_rank_planned = orc_maxvio(pmax, R, N);
        out->balancedness_rank_planned = orc_balancedness(pmax, R, N);
    }
    if (slots_needed && slot_expert && seg_num && seg_expert && seg_cnt) {
        for (int r = 0; r < R; ++r) {
            out->replica_pieces += slots_needed[r];
            if (slots_needed[r] > out->max_slots_needed) out->max_slots_needed = slots_needed[r];
            if (slots_needed[r] > S) out->ranks_over_slots++;
            /* rows of replica experts past the first S slots are not local */
            for (int i = S; i < slots_needed[r]; ++i) {
                int e = slot_expert[(size_t)r * n + i];
                for (int q = 0; q < seg_num[r]; ++q)
                    if (seg_expert[(size_t)r * 2 * n + q] == e)
                        out->nonlocal_rows += seg_cnt[(size_t)r * 2 * n + q];
            }
        }
    }
    free(rl);
    free(rm);
}
