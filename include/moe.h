/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer hot path library, libmoe.so.
 *
 * One MoE layer, data-parallel forward, on one GPU:
 *   moe_route        router top-k gating               (phase a)
 *   moe_count        per-expert demand + stable index
 *   moe_plan         equal-load replica plan over R virtual ranks
 *   moe_permute      dispatch into a static-shape buffer (phase b)
 *   moe_grouped_gemm SwiGLU expert FFN over the plan    (phase c)
 *   moe_combine      gate-weighted gather back to tokens (phase d)
 *   moe_stats        maxvio / balancedness / capacity / remote statistics
 * the backward (moe_combine_backward, moe_ffn_backward, moe_permute_backward,
 * moe_route_backward); the replica slot pool (moe_prefetch_replicas,
 * moe_grouped_gemm_slots); the
 * two baselines the plan replaces: fixed-capacity dispatch (moe_capacity_*)
 * and static repacking (moe_repack); the router's scores (moe_router) and an
 * assumed balancing-bias update (moe_bias_update).
 *
 * Sources (web pages, cited by title and section):
 *   [Primer]  "DeepEP-on-EFA Guidance, section 1: what is MoE" -- the
 *             four-phase layer: router, dispatch, batched grouped GEMM,
 *             combine; a token travels only to its k experts.
 *   [MoonEP]  "Moonshot AI drops MoonEP, claims 2.5x scaling boost for
 *             trillion-parameter models", paragraphs 2-4 -- maxvio (zero when
 *             balanced), the equal-load invariant, replicas planned on device
 *             from the router output, zero-copy placement, static buffer
 *             shapes, one contiguous weight tensor per projection, prefetch
 *             slots (= experts per rank for training, 3-4 for inference).
 *   [Hotspot] "MoE Load Balancing: Find Expert Hotspots" -- demand counting,
 *             average/max balancedness, rank demand under a mapping, the
 *             fixed-capacity ledger, remote routes, validation before use.
 *   [Interview] "MoE load balancing: 90/10 routing in production" -- a
 *             per-expert bias that steers selection without touching the gate.
 *
 * Conventions
 *   - Every pointer named d_* is DEVICE memory owned by the caller; h_* is
 *     host memory owned by the caller. The library never allocates device
 *     memory and keeps no state between calls.
 *   - Every call except moe_stats is asynchronous and stream-ordered on
 *     `stream` (a hipStream_t; NULL means the default stream).
 *   - Host-detectable problems (bad shape, NULL pointer, workspace too small)
 *     return a status BEFORE anything is launched; outputs are untouched.
 *     A pointer to an array of zero length (T = 0) may be NULL.
 *   - Data problems found on the device (non-finite logits, bad ids) set bits
 *     in a caller-provided device int32 error word with an order-free atomic
 *     OR; the caller zeroes it. When it is non-zero the outputs are
 *     unspecified (but every kernel stays in bounds). moe_stats reports it.
 *   - All 2-D arrays are row-major. N = T*k assignments. n = E/R experts per
 *     rank. dtype is the element type of activations, weights, buffers and
 *     outputs (MOE_F32: float; MOE_BF16: bfloat16). Logits, biases and gate
 *     weights are always float; ids, indices and tables are int32.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,        /* bad shape, NULL pointer, or size out of range       */
    MOE_EUNSUPPORTED = 2,  /* valid request this build does not implement         */
    MOE_EDEVICE = 3,       /* a HIP runtime call failed                           */
    MOE_EDATA = 4          /* the device error word is non-zero (moe_stats only)  */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Device error word bits. */
#define MOE_ERR_NONFINITE 1 /* a logit or bias is NaN or infinite             */
#define MOE_ERR_RANGE 2     /* an expert id is outside [0, E)                 */
#define MOE_ERR_REPEAT 4    /* a token lists the same expert twice            */

typedef void *moe_stream_t; /* a hipStream_t */

/* Shape of one layer call.
 * Limits (checked by every entry point): 0 <= T, 1 <= k <= min(E, 64),
 * 1 <= E <= 256, 1 <= R <= 64, E % R == 0, 0 <= S, 1 <= H, 1 <= F,
 * T*k < 2^31, (T*k)*max(H,F) < 2^40.
 * MOE_BF16 additionally needs H % 64 == 0 and F % 64 == 0 (GEMM K-steps),
 * and (T*k)*H*2, F*H*2 and 512*F below 2^32 - 128 (the GEMM addresses operand
 * rows with 32-bit byte offsets); MOE_EUNSUPPORTED otherwise.
 * MOE_F32 needs H % 4 == 0 and F % 4 == 0 (16-byte rows). */
typedef struct moe_shape {
    int32_t T;     /* tokens in the batch                                  */
    int32_t H;     /* hidden width (row length of x, buf, y, out)          */
    int32_t E;     /* routed experts                                       */
    int32_t k;     /* experts per token (top-k)                            */
    int32_t F;     /* expert SwiGLU width                                  */
    int32_t R;     /* virtual expert-parallel ranks; rank r homes experts
                      [r*n, (r+1)*n)                                       */
    int32_t S;     /* prefetch slots per rank (locality budget, reported)  */
    int32_t dtype; /* moe_dtype_t                                          */
} moe_shape_t;

/* The plan is one caller-allocated int32 device block of `total` elements;
 * each table starts at the given element offset. Unused entries are -1.
 *   quota[R]          rows every rank receives: floor(N/R) + [r < N mod R]
 *   win_off[R+1]      first row of rank r's window in buf (prefix of quota)
 *   seg_num[R]        segments in rank r's window
 *   seg_expert[R][2n] expert of each segment, ascending within a window
 *   seg_row[R][2n]    first buf row of each segment
 *   seg_cnt[R][2n]    rows of each segment
 *   slots_needed[R]   replica (non-home) experts rank r holds
 *   slot_expert[R][n] those experts, ascending
 *   donor[R]          the rank whose experts r replicates, or -1
 *   piece_num[E]      pieces expert e is split into (<= R)
 *   piece_rank[E][R]  rank of each piece, ascending
 *   piece_row[E][R]   first buf row of each piece
 *   piece_cnt[E][R]   rows of each piece                                   */
typedef struct moe_plan_layout {
    int64_t quota, win_off, seg_num, seg_expert, seg_row, seg_cnt, slots_needed, slot_expert,
        donor, piece_num, piece_rank, piece_row, piece_cnt;
    int64_t total; /* int32 elements in the block */
} moe_plan_layout_t;

/* Host-side statistics (moe_stats). Integers are exact; every double is one
 * division of exact integers. */
typedef struct moe_stats {
    int64_t N;                       /* assignments T*k                          */
    int32_t E, R;
    int32_t max_count, min_count, active_experts;
    double maxvio_expert;            /* max/mean - 1 over expert demand          */
    double balancedness_expert;      /* mean/max over expert demand              */
    int32_t home_max;
    double maxvio_rank_home, balancedness_rank_home;      /* contiguous homes   */
    int32_t mapped_max;
    double maxvio_rank_mapped, balancedness_rank_mapped;  /* caller mapping     */
    int32_t planned_max, planned_min;
    double maxvio_rank_planned, balancedness_rank_planned;/* after the plan     */
    int32_t capacity;                /* ceil(N / E * capacity_factor)            */
    int64_t processed, overflow, padding; /* ledger sums from raw demand        */
    int64_t remote_home, remote_mapped, remote_planned;   /* origin != dest     */
    int32_t replica_pieces;          /* sum of slots_needed                      */
    int32_t max_slots_needed;
    int32_t ranks_over_slots;        /* ranks with slots_needed > S              */
    int64_t nonlocal_rows;           /* rows of replicas past the first S slots  */
    int32_t err;                     /* device error word                        */
} moe_stats_t;

/* Human-readable name of a status. Never NULL. */
const char *moe_status_str(moe_status_t status);

/* Validates a shape against the limits above. */
moe_status_t moe_check_shape(const moe_shape_t *shape);

/* Fills *out with the plan block layout for this shape. */
moe_status_t moe_plan_layout(const moe_shape_t *shape, moe_plan_layout_t *out);

/* The plan block's tables by name: pointers into one block (the layout
 * above). Every call that takes a plan takes the block's base, d_plan. */
typedef struct moe_plan {
    int32_t *quota, *win_off, *seg_expert, *seg_row, *seg_cnt, *seg_num, *slot_expert,
        *slots_needed, *piece_rank, *piece_row, *piece_cnt, *piece_num, *donor;
} moe_plan_t;

/* [MoonEP] paragraph 3 (static buffer shapes: the plan's tables have a size
 * fixed by the shape). Bytes of the plan block: layout.total * 4; 0 on a
 * bad shape. The caller allocates one block of this size. */
size_t moe_plan_bytes(const moe_shape_t *shape);

/* Carves a plan block of moe_plan_bytes(shape) bytes at `block` (device or
 * host memory; never dereferenced) into the named table pointers of *out.
 * MOE_EINVAL on a NULL block or out. */
moe_status_t moe_plan_bind(const moe_shape_t *shape, void *block, moe_plan_t *out);

/* Bytes of device workspace moe_count, moe_grouped_gemm and moe_stats need
 * (count scratch, GEMM tile schedule, the SwiGLU activations h[N][F], the
 * statistics reductions). 0 on a bad
 * shape. The caller allocates it once per shape and may reuse it. */
size_t moe_workspace_bytes(const moe_shape_t *shape);

/* [Primer] phase (a); [Interview] editor's note (bias outside the gate).
 * For every token t: score_e = logits[t][e] + bias[e] as one fp32 add; the k
 * experts with the largest score, largest first, equal scores to the lower
 * id, go to d_ids[t][0..k). The gate weights are the softmax of the RAW
 * logits of those k experts (they sum to 1), in the same order.
 *   d_logits float[T][E]; d_bias float[E] or NULL (no bias);
 *   d_ids int32[T][k] out; d_w float[T][k] out; d_err int32[1] in/out.
 * Non-finite logit or bias: d_err |= MOE_ERR_NONFINITE. */
moe_status_t moe_route(const moe_shape_t *shape, const float *d_logits, const float *d_bias,
                       int32_t *d_ids, float *d_w, int32_t *d_err, moe_stream_t stream);

/* [Hotspot] "Separate expert demand from rank placement", "Work the 16-token
 * hotspot fixture": demand counted per assignment, then per rank.
 *   d_counts int32[E] out: assignments per expert.
 *   d_offsets int32[E+1] out: exclusive prefix of counts.
 *   d_eidx int32[N] out: for assignment t*k+j, the number of earlier
 *     assignments (in flat order) with the same expert -- a stable index.
 *   d_rank_load int32[R] out: sum of counts over rank r's home experts.
 *   d_ws / ws_bytes: workspace of moe_workspace_bytes(shape) bytes.
 * Ids outside [0, E) set MOE_ERR_RANGE and are not counted; a token naming
 * an expert twice sets MOE_ERR_REPEAT. Results do not depend on thread
 * timing (no ordered atomics). */
moe_status_t moe_count(const moe_shape_t *shape, const int32_t *d_ids, int32_t *d_counts,
                       int32_t *d_offsets, int32_t *d_eidx, int32_t *d_rank_load, int32_t *d_err,
                       void *d_ws, size_t ws_bytes, moe_stream_t stream);

/* moe_count for callers that cannot allocate device memory (code under HIP
 * graph capture, allocation-free serving loops): the same results as
 * moe_count, bit for bit, with no workspace argument. Above 16384
 * assignments the count keeps two int32[ceil(N/1024)][E] tables (each
 * rounded up to 256 bytes) in a fixed 8 MiB device array of the library
 * instead: N up to 4194304 at E = 256 (up to 16384 at any E); a larger
 * shape returns MOE_EINVAL before anything is launched. Each GPU holds its
 * own copy of that array until the process ends; its address is looked up
 * on the first call on each device (the device current at the call). Calls
 * that overlap on one GPU (other streams or host threads) share the array
 * and race: order them. Allocates nothing. */
moe_status_t moe_count_noalloc(const moe_shape_t *shape, const int32_t *d_ids, int32_t *d_counts,
                               int32_t *d_offsets, int32_t *d_eidx, int32_t *d_rank_load,
                               int32_t *d_err, moe_stream_t stream);

/* [MoonEP] paragraphs 3-4: every rank receives the same number of
 * assignments, by replicas planned on the device from the router output;
 * with S = n slots every expert a rank computes is local.
 * The pages state the invariant only; the plan is this alias-style rule:
 * while an unfilled rank is below its quota, the rank with the largest
 * deficit (ties: lower rank) is topped up to its quota from the home experts
 * of the rank with the largest excess (ties: lower rank), taking the donor's
 * experts in (count desc, id asc) order; what remains stays home. Segments
 * within a window are ordered by expert id; an expert's pieces are ordered
 * by rank and filled in stable (eidx) order. Every rank receives from at
 * most one donor, so it holds at most n replica experts.
 *   d_counts int32[E] in; d_plan int32[layout.total] out (whole block
 *   written). Single workgroup; O(E*R) work; no host round trip. */
moe_status_t moe_plan(const moe_shape_t *shape, const int32_t *d_counts, int32_t *d_plan,
                      moe_stream_t stream);

/* [Hotspot] "Separate expert demand from rank placement" then [MoonEP]
 * paragraphs 3-4: moe_count followed by moe_plan on its counts, with the
 * same arguments and results, bit for bit. Up to 16384 assignments (the
 * decode regime, where a launch costs more than either step's work) both
 * run in one single-workgroup launch, the plan reading the counts from the
 * workgroup's LDS; above that it is the two calls' launches in turn.
 *   d_ids .. d_err, d_ws / ws_bytes as moe_count; d_plan as moe_plan. */
moe_status_t moe_count_plan(const moe_shape_t *shape, const int32_t *d_ids, int32_t *d_counts,
                            int32_t *d_offsets, int32_t *d_eidx, int32_t *d_rank_load,
                            int32_t *d_err, void *d_ws, size_t ws_bytes, int32_t *d_plan,
                            moe_stream_t stream);

/* [Primer] phase (b) (a token goes only to its k experts); [MoonEP]
 * paragraph 3 (zero-copy placement into static shapes). Assignment (t,j)
 * with expert e and stable index v goes to piece p of e with
 * cum_p <= v < cum_p + piece_cnt, row piece_row + v - cum_p.
 *   d_x dtype[T][H] in; d_ids, d_eidx in; d_plan in;
 *   d_buf dtype[N][H] out (every row written exactly once);
 *   d_dest_row int32[T][k] out; d_row_src int32[N] out (source token). */
moe_status_t moe_permute(const moe_shape_t *shape, const void *d_x, const int32_t *d_ids,
                         const int32_t *d_eidx, const int32_t *d_plan, void *d_buf,
                         int32_t *d_dest_row, int32_t *d_row_src, moe_stream_t stream);

/* [Primer] phase (c), batched grouped GEMM of every expert over the rows it
 * received; [MoonEP] paragraph 3: one contiguous weight tensor per
 * projection. For every row i of d_a held by expert e (per the plan):
 *   h = silu(W_gate[e] a_i) * (W_up[e] a_i),  silu(z) = z / (1 + e^-z),
 *   y_i = W_down[e] h.
 *   d_a dtype[N][H] (the permuted buffer); d_w_gate, d_w_up dtype[E][F][H];
 *   d_w_down dtype[E][H][F]; d_y dtype[N][H] out (same row order as d_a).
 * Replicas read their home expert's weights (one GPU holds every expert).
 * In MOE_BF16 the products accumulate in fp32 and h is rounded to bf16.
 * d_plan (from moe_plan) gives each expert's pieces of rows. A one-expert
 * shape (E = R = k = 1) planned from counts = {T} is a dense SwiGLU FFN
 * over T rows (e.g. an always-on shared expert).
 * d_ws / ws_bytes: workspace of moe_workspace_bytes(shape) bytes (holds the
 * tile schedule and h). */
moe_status_t moe_grouped_gemm(const moe_shape_t *shape, const void *d_a, const int32_t *d_plan,
                              const void *d_w_gate, const void *d_w_up, const void *d_w_down,
                              void *d_y, void *d_ws, size_t ws_bytes, moe_stream_t stream);

/* The three steps of moe_grouped_gemm, for callers that time or overlap them
 * separately (same arguments, same d_ws, in this order): moe_gemm_schedule
 * builds the per-expert tile schedule and the expert-sorted row -> buf row
 * map in d_ws from the plan; moe_gemm_gateup computes h; moe_gemm_down
 * computes y. */
moe_status_t moe_gemm_schedule(const moe_shape_t *shape, const int32_t *d_plan, void *d_ws,
                               size_t ws_bytes, moe_stream_t stream);
moe_status_t moe_gemm_gateup(const moe_shape_t *shape, const void *d_a, const int32_t *d_plan,
                             const void *d_w_gate, const void *d_w_up, void *d_ws,
                             size_t ws_bytes, moe_stream_t stream);
moe_status_t moe_gemm_down(const moe_shape_t *shape, const int32_t *d_plan, const void *d_w_down,
                           void *d_y, void *d_ws, size_t ws_bytes, moe_stream_t stream);

/* ---- Replica weight slots ------------------------------------------------
 * [MoonEP] paragraphs 3-4: the planned redundant expert copies are prefetched
 * into a fixed number S of weight slots per rank; S = experts per rank makes
 * every expert the grouped GEMM touches local, and 3-4 slots usually suffice
 * in inference. One pool serves every layer of a model (it holds only the
 * current layer's replicas). Reading: rank r's replica experts take its
 * slots in slot_expert[r] order (ascending expert id); slot j < min(S, n)
 * holds that expert's three projections. */

/* [MoonEP] paragraphs 3-4 (S prefetch slots per rank, one pool for every
 * layer). Bytes of the slot pool for this shape: R * min(S, n) * 3 * F * H * dtype
 * bytes, laid out pool[r][j][q][F*H] with q = 0 gate [F][H], 1 up [F][H],
 * 2 down [H][F] (each exactly the home expert's slice). 0 on a bad shape or
 * when S = 0. */
size_t moe_pool_bytes(const moe_shape_t *shape);

/* [MoonEP] paragraph 3 (the planned replicas' weights prefetched before the
 * GEMM). The prefetch: copies, for every rank r and slot j < min(S, n) that the plan
 * fills (slot_expert[r][j] >= 0), that expert's gate, up and down slices into
 * pool[r][j], bit for bit. Slots without an expert are not written.
 *   d_plan the moe_plan block; d_w_gate, d_w_up dtype[E][F][H];
 *   d_w_down dtype[E][H][F]; d_pool / pool_bytes >= moe_pool_bytes(shape)
 *   (d_pool may be NULL when that is 0). */
moe_status_t moe_prefetch_replicas(const moe_shape_t *shape, const int32_t *d_plan,
                                   const void *d_w_gate, const void *d_w_up, const void *d_w_down,
                                   void *d_pool, size_t pool_bytes, moe_stream_t stream);

/* [Primer] phase (c) on each rank's local experts; [MoonEP] paragraph 4
 * (with S = n slots every expert a rank computes is local).
 * moe_grouped_gemm as the R ranks would run it: one group per plan segment
 * (rank r's i-th expert run, contiguous rows of d_a), each with its own
 * weights -- the slot pool[r][j] for a replica segment whose expert holds
 * slot j < min(S, n) of rank r, the home slices for a home segment and for
 * a replica without a slot (a non-local read). y is the same function of the
 * weights as moe_grouped_gemm's when the pool holds moe_prefetch_replicas'
 * copies. Arguments as moe_grouped_gemm plus d_pool / pool_bytes (as
 * moe_prefetch_replicas); d_ws: moe_workspace_bytes(shape). */
moe_status_t moe_grouped_gemm_slots(const moe_shape_t *shape, const void *d_a,
                                    const int32_t *d_plan, const void *d_w_gate,
                                    const void *d_w_up, const void *d_w_down, const void *d_pool,
                                    size_t pool_bytes, void *d_y, void *d_ws, size_t ws_bytes,
                                    moe_stream_t stream);

/* [Primer] phase (d): expert outputs return to their token and are summed
 * with the gate weights (the transpose of dispatch).
 *   out[t] = sum_{j=0..k-1} w[t][j] * y[dest_row[t][j]]  (+ shared_y[t])
 * accumulated in fp32 in j order, rounded once to dtype.
 *   d_y dtype[N][H]; d_dest_row int32[T][k]; d_w float[T][k];
 *   d_shared_y dtype[T][H] or NULL; d_out dtype[T][H] out. */
moe_status_t moe_combine(const moe_shape_t *shape, const void *d_y, const int32_t *d_dest_row,
                         const float *d_w, const void *d_shared_y, void *d_out,
                         moe_stream_t stream);

/* [MoonEP] paragraph 2 (maxvio, zero when balanced; read as max/mean - 1);
 * [Hotspot] (average/max balancedness; rank demand under a mapping; the
 * fixed-capacity ledger ceil(N / E * factor) with processed, overflow and
 * padding from raw demand; remote routes where origin rank != destination
 * rank). Reduces on the device, copies a few hundred bytes back and
 * SYNCHRONISES the stream; not for the timed path.
 *   d_counts int32[E]; d_ids int32[T][k]; d_plan (planned figures);
 *   d_dest_row int32[T][k] or NULL (planned remote routes);
 *   d_mapping int32[E] or NULL (expert -> rank for the "mapped" figures);
 *   d_origin int32[T] or NULL (origin rank; NULL means t mod R);
 *   d_err int32[1] or NULL; d_ws / ws_bytes: the moe_workspace_bytes(shape)
 *   workspace (a small region of it receives the reductions; the count and
 *   GEMM regions are left alone). capacity_factor > 0 and finite.
 *   Returns MOE_EDATA (after filling *h_out) when the error word is non-zero. h_rank_loads, if not NULL, receives
 *   int32[3][R]: home, mapped (zeros without a mapping) and planned loads. */
moe_status_t moe_stats(const moe_shape_t *shape, const int32_t *d_counts, const int32_t *d_ids,
                       const int32_t *d_plan, const int32_t *d_dest_row,
                       const int32_t *d_mapping, const int32_t *d_origin, const int32_t *d_err,
                       double capacity_factor, void *d_ws, size_t ws_bytes, moe_stats_t *h_out,
                       int32_t *h_rank_loads, moe_stream_t stream);

/* ---- Backward (training) ---------------------------------------------------
 * [Primer] phases (a)-(d) in reverse, with the plan tables of the forward.
 * [MoonEP] paragraph 3: replica gradients are reduced into the home expert --
 * here every piece of an expert (home or replica) adds into that expert's one
 * weight gradient. bf16 runs on MFMA; fp32 (small shapes such as the
 * hotspot fixture) on plain FMA kernels, one thread per output element. */

/* [Primer] phase (c) in reverse. Device workspace moe_ffn_backward needs: x and dy in expert order, the
 * recomputed g | u, dg | du and h (about N * (2H + 5F) * dtype bytes), a
 * schedule, a zero page and (bf16, few wide experts) fp32 partials of dx.
 * 0 on a bad shape. */
size_t moe_backward_workspace_bytes(const moe_shape_t *shape);

/* [Primer] phase (d) in reverse. Combine backward. With out[t] = sum_j w[t][j] y[dest_row[t][j]]:
 *   dy[dest_row[t][j]] = w[t][j] * dout[t]   (bf16, one rounding)
 *   dw[t][j] = sum_h dout[t][h] * y[dest_row[t][j]][h]   (fp32 accumulate)
 * Rows of dy that no assignment names are not written (with the equal-load
 * plan every row is named once). d_dout dtype[T][H]; d_y dtype[N][H];
 * d_dest_row int32[T][k]; d_w float[T][k]; d_dy dtype[N][H] out;
 * d_dw float[T][k] out. */
moe_status_t moe_combine_backward(const moe_shape_t *shape, const void *d_dout, const void *d_y,
                                  const int32_t *d_dest_row, const float *d_w, void *d_dy,
                                  float *d_dw, moe_stream_t stream);

/* [Primer] phase (c) in reverse; [MoonEP] paragraph 3 (every piece of an
 * expert adds into its home expert's gradient). SwiGLU expert FFN backward over the plan (the moe_grouped_gemm forward's
 * adjoint): recomputes g | u from d_buf, then
 *   dh = dy W_down, dg = dh u s (1 + g (1 - s)), du = dh silu(g) (s the
 *   logistic of g), dbuf = dg W_gate + du W_up,
 *   dW_down[e] = sum over e's rows of dy h^T, dW_gate[e] = sum dg x^T,
 *   dW_up[e] = sum du x^T   (fp32, overwritten; zero for idle experts).
 * d_buf dtype[N][H] (the permuted input); d_plan the moe_plan block;
 * weights as moe_grouped_gemm; d_gu: NULL to recompute g | u, or the buffer
 * moe_grouped_gemm_train filled in this step's forward (bf16); d_dy
 * dtype[N][H] (buffer order); d_dbuf
 * dtype[N][H] out (buffer order); d_dw_gate, d_dw_up float[E][F][H] out;
 * d_dw_down float[E][H][F] out; d_ws / ws_bytes >=
 * moe_backward_workspace_bytes(shape). */
moe_status_t moe_ffn_backward(const moe_shape_t *shape, const void *d_buf, const int32_t *d_plan,
                              const void *d_w_gate, const void *d_w_up, const void *d_w_down,
                              const void *d_gu, const void *d_dy, void *d_dbuf, float *d_dw_gate,
                              float *d_dw_up, float *d_dw_down, void *d_ws, size_t ws_bytes,
                              moe_stream_t stream);

/* [MoonEP] paragraph 3 (replica gradients reduced home). Bytes of the replica weight-gradient slots: R * n * 3 * F * H * 4 (fp32),
 * laid out [R][n][3][F*H] -- slot r*n + j holds the gradient of rank r's
 * j-th replica expert (slot_expert order), gate | up | down. 0 on a bad
 * shape. */
size_t moe_replica_grad_bytes(const moe_shape_t *shape);

/* moe_ffn_backward with the replica-gradient reduction made explicit, as R
 * ranks run it ([MoonEP] paragraph 3): each replica piece's weight gradient
 * (its rows on the rank that holds the replica) is written to its slot in
 * d_rgrad; each expert's home piece writes the expert's gradient (zero when
 * the plan moved all of its rows away); then every slot is added into its
 * home expert's gradient, after the home part, in rank order. The result
 * equals moe_ffn_backward's up to fp32 summation order; the slots keep the
 * per-replica gradients. bf16 only (MOE_EUNSUPPORTED for fp32).
 *   d_rgrad / rgrad_bytes >= moe_replica_grad_bytes(shape); slots of ranks
 *   without that replica are not written; other arguments as
 *   moe_ffn_backward. */
moe_status_t moe_ffn_backward_replicas(const moe_shape_t *shape, const void *d_buf,
                                       const int32_t *d_plan, const void *d_w_gate,
                                       const void *d_w_up, const void *d_w_down, const void *d_gu,
                                       const void *d_dy, void *d_dbuf, float *d_dw_gate,
                                       float *d_dw_up, float *d_dw_down, float *d_rgrad,
                                       size_t rgrad_bytes, void *d_ws, size_t ws_bytes,
                                       moe_stream_t stream);

/* [Primer] phase (c), training. The forward grouped GEMM of a training step: moe_grouped_gemm, and (bf16)
 * the gate and up projections kept in d_gu bf16[N][2F] (row x in expert
 * order -- the order moe_ffn_backward uses -- g in columns [0, F), u in
 * [F, 2F)), so that moe_ffn_backward(d_gu = this buffer) skips its
 * recompute. fp32: d_gu is not written (the fp32 backward recomputes). */
moe_status_t moe_grouped_gemm_train(const moe_shape_t *shape, const void *d_a,
                                    const int32_t *d_plan, const void *d_w_gate,
                                    const void *d_w_up, const void *d_w_down, void *d_y,
                                    void *d_gu, void *d_ws, size_t ws_bytes, moe_stream_t stream);

/* [Primer] phase (b) in reverse. Dispatch backward: dx[t] = sum_j dbuf[dest_row[t][j]] (fp32 accumulate in
 * j order, one rounding). d_dbuf dtype[N][H]; d_dest_row int32[T][k];
 * d_dx dtype[T][H] out. */
moe_status_t moe_permute_backward(const moe_shape_t *shape, const void *d_dbuf,
                                  const int32_t *d_dest_row, void *d_dx, moe_stream_t stream);

/* [Primer] phase (a) in reverse. Gate backward: w is the softmax of the selected raw logits, so
 *   dlogits[t][ids[t][j]] = w[t][j] * (dw[t][j] - sum_j' w[t][j'] dw[t][j']),
 * and 0 for experts not selected ([Interview] editor's note: the balancing
 * bias only selects; it has no gradient here). d_ids int32[T][k];
 * d_w, d_dw float[T][k]; d_dlogits float[T][E] out. */
moe_status_t moe_route_backward(const moe_shape_t *shape, const int32_t *d_ids, const float *d_w,
                                const float *d_dw, float *d_dlogits, moe_stream_t stream);

/* ---- Router scores and the balancing bias ---------------------------------
 * [Primer] phase (a): the router scores every expert for every token. The
 * pages do not print the router; it is read as a linear layer. */

/* [Primer] phase (a). Device workspace moe_router needs for this shape, in bytes: 0 when one
 * K-range covers H (fp32, or enough token tiles to fill the GPU); else
 * parts * T * E * 4 for the per-range fp32 partial logits. 0 on a bad shape. */
size_t moe_router_workspace_bytes(const moe_shape_t *shape);

/* [Primer] phase (a): the router scores, read as a linear layer, then the
 * top-k gating. logits[t][e] = sum_h x[t][h] * W_r[e][h], accumulated in fp32 (bf16 x and
 * W_r: MFMA; where H is split into K-ranges, the ranges' fp32 partial sums
 * are added in range order, so results are the same on every call; fp32: FMA
 * in h order), written to d_logits, then exactly moe_route on those logits
 * (same bias, tie and error rules).
 *   d_x dtype[T][H]; d_w_router dtype[E][H]; d_bias float[E] or NULL;
 *   d_logits float[T][E] out; d_ids int32[T][k] out; d_w float[T][k] out;
 *   d_err int32[1] (bit 1: non-finite logit or bias);
 *   d_ws: moe_router_workspace_bytes(shape) bytes of device scratch (may be
 *   NULL when that is 0), ws_bytes its size; MOE_EINVAL if too small.
 * bf16 needs E * H * 2 < 2^32 (MOE_EUNSUPPORTED otherwise). */
moe_status_t moe_router(const moe_shape_t *shape, const void *d_x, const void *d_w_router,
                        const float *d_bias, float *d_logits, int32_t *d_ids, float *d_w,
                        int32_t *d_err, void *d_ws, size_t ws_bytes, moe_stream_t stream);

/* Balancing-bias update. NOT ON THE PAGES: [Interview] keeps a per-expert
 * bias out of the gate but prints no update rule; this is the sign rule of
 * auxiliary-loss-free balancing, an assumption. bias[e] += gamma if
 * counts[e] < N/E, -= gamma if counts[e] > N/E (decided in integers from
 * N - E*counts[e], N = T*k), one fp32 add. d_counts int32[E];
 * d_bias float[E] in/out; gamma >= 0 and finite. */
moe_status_t moe_bias_update(const moe_shape_t *shape, const int32_t *d_counts, float *d_bias,
                             float gamma, moe_stream_t stream);

/* ---- Baselines the equal-load plan replaces ------------------------------
 * [Hotspot] "Make expert capacity, overflow, and padding explicit": a fixed
 * capacity per expert; demand above it overflows (the assignment is
 * dropped), unused slots below it are padding. And "Separate expert demand
 * from rank placement": a static expert -> rank mapping that pairs hot and
 * cold experts. */

/* [Hotspot] "Make expert capacity, overflow, and padding explicit".
 * Per-expert capacity ceil(N / E * capacity_factor) (the moe_stats figure),
 * or -1 for an invalid shape or factor, or when E * capacity does not fit
 * int32. */
int32_t moe_capacity_rows(const moe_shape_t *shape, double capacity_factor);

/* [Hotspot] "Make expert capacity, overflow, and padding explicit".
 * Fixed-capacity dispatch into a static [E][cap] buffer. An expert keeps its
 * first cap assignments in stable order: assignment (t,j) of expert e with
 * eidx v < cap goes to row e*cap + v; the others are dropped (dest_row -1).
 * Rows e*cap + v with v >= counts[e] are padding and are written as zeros.
 *   cap >= 1, E*cap < 2^31; d_counts int32[E] (moe_count); d_x dtype[T][H];
 *   d_ids, d_eidx int32[T][k]; d_buf dtype[E*cap][H] out (every row
 *   written); d_dest_row int32[T][k] out. */
moe_status_t moe_capacity_dispatch(const moe_shape_t *shape, int32_t cap, const int32_t *d_counts,
                                   const void *d_x, const int32_t *d_ids, const int32_t *d_eidx,
                                   void *d_buf, int32_t *d_dest_row, moe_stream_t stream);

/* [Hotspot] "Make expert capacity, overflow, and padding explicit"; [Primer]
 * phase (c). The plan block (moe_plan_layout) of the capacity layout: expert e is home
 * on rank e / (E/R) with one piece of cap rows at row e*cap, no replicas.
 * With it, moe_grouped_gemm over the shape {T = E*cap, k = 1, H, E, F, R, S,
 * dtype} runs the expert FFN over the whole static buffer, padding rows
 * included (they are zero and give zero rows). */
moe_status_t moe_capacity_plan(const moe_shape_t *shape, int32_t cap, int32_t *d_plan,
                               moe_stream_t stream);

/* [Hotspot] "Make expert capacity, overflow, and padding explicit"; [Primer]
 * phase (d). moe_combine over the capacity buffer: d_y dtype[E*cap][H]; dropped
 * assignments (dest_row -1) contribute nothing; other arguments as in
 * moe_combine. */
moe_status_t moe_capacity_combine(const moe_shape_t *shape, int32_t cap, const void *d_y,
                                  const int32_t *d_dest_row, const float *d_w,
                                  const void *d_shared_y, void *d_out, moe_stream_t stream);

/* [Hotspot] "Separate expert demand from rank placement" (the proposed
 * mapping). Greedy balanced repacking: experts in order of decreasing demand (equal
 * demand: lower id first) each go to the least-loaded rank that holds fewer
 * than E/R experts (equal load: lower rank). Reproduces the page's mapping
 * {0,7},{1,6},{2,5},{3,4} for the fixture demand. d_counts int32[E];
 * d_mapping int32[E] out (expert -> rank; usable as moe_stats' d_mapping). */
moe_status_t moe_repack(const moe_shape_t *shape, const int32_t *d_counts, int32_t *d_mapping,
                        moe_stream_t stream);

/* ---- Calibration (measurement only) --------------------------------------
 * Not a step of the method: a probe for measured peaks beside the spec
 * ones. Runs `workgroups` workgroups of 256 threads; every wave performs
 * 4 * iters v_mfma_f32_32x32x16_bf16 (2*32*32*16 flops each) on registers
 * only, four independent chains on four operand pairs of bf16 values of
 * magnitude 2^-7..2^-6 with hashed signs and mantissas. d_sink float[] out,
 * at least workgroups * 256 entries (one sum per lane, only to keep the
 * work). MOE_EINVAL for workgroups < 1, iters < 1, a NULL or short sink. */
moe_status_t moe_probe_mfma(int32_t workgroups, int32_t iters, float *d_sink, size_t sink_floats,
                            moe_stream_t stream);

/* Calibration probe for HBM: copies `bytes` from d_src to d_dst (device
 * buffers, 16-byte aligned, bytes a multiple of 16, not overlapping) with
 * `workgroups` workgroups of 256 threads, each thread moving four 16-byte
 * vectors per round (loads before stores). MOE_EINVAL for NULL or
 * misaligned buffers, bytes 0 or not a multiple of 16, workgroups < 1. */
moe_status_t moe_probe_copy(const void *d_src, void *d_dst, size_t bytes, int32_t workgroups,
                            moe_stream_t stream);

/* Calibration probe for HBM reads: reads `bytes` of d_src (device, 16-byte
 * aligned, bytes a multiple of 16) with `workgroups` workgroups of 256
 * threads, workgroup b taking the b-th of `workgroups` equal contiguous
 * chunks (the last one may be shorter or empty), eight 16-byte loads in
 * flight per thread. d_sink uint32[] out, at least workgroups * 256 entries:
 * thread t of workgroup b stores the XOR of the four words of every vector
 * i of its chunk with i mod 256 == t. MOE_EINVAL for NULL or misaligned
 * buffers, bytes 0 or not a multiple of 16, workgroups < 1, a short sink, or
 * a chunk above 2^31 - 32768 bytes. */
moe_status_t moe_probe_read(const void *d_src, size_t bytes, int32_t workgroups, uint32_t *d_sink,
                            size_t sink_words, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
