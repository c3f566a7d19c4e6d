// common.h -- internal helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// bf16 storage is the upper half of an IEEE fp32; conversions are exact one
// way and round-to-nearest-even the other (gfx950's v_cvt_pk_bf16_f32; NaN
// stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two bf16 values packed in a uint32 (low half = lower address).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Plan block layout (int32 element offsets), the single definition used by
// the host API and every kernel that reads the plan.
struct PlanLayout {
    int64_t quota, win_off, seg_num, seg_expert, seg_row, seg_cnt, slots_needed, slot_expert,
        donor, piece_num, piece_rank, piece_row, piece_cnt, total;
};

__host__ __device__ inline PlanLayout plan_layout(int E, int R)
{
    const int64_t n = E / R;
    PlanLayout L;
    int64_t o = 0;
    L.quota = o;        o += R;
    L.win_off = o;      o += R + 1;
    L.seg_num = o;      o += R;
    L.seg_expert = o;   o += R * 2 * n;
    L.seg_row = o;      o += R * 2 * n;
    L.seg_cnt = o;      o += R * 2 * n;
    L.slots_needed = o; o += R;
    L.slot_expert = o;  o += R * n;
    L.donor = o;        o += R;
    L.piece_num = o;    o += E;
    L.piece_rank = o;   o += (int64_t)E * R;
    L.piece_row = o;    o += (int64_t)E * R;
    L.piece_cnt = o;    o += (int64_t)E * R;
    L.total = o;
    return L;
}

// Workspace carve-up (bytes, 256-byte aligned regions).
struct WsLayout {
    size_t blk_hist, blk_base;  // count: int32[B][E] each
    size_t sched;               // gemm: int32 schedule (see gemm.hip), up to 2E groups
    size_t wtab;                // gemm by segment: uint64[2E][3] weight addresses
    size_t vrow;                // gemm: int32[N] expert-sorted row -> buf row
    size_t part;                // gemm bf16: float[units][256][256] partial tiles (K-split leftovers)
    size_t skpart;              // gemm bf16: float[2 grid][32 + 64][256] skinny partial tiles
    size_t h;                   // gemm: dtype[N][F] SwiGLU activations
    size_t stats;               // stats: int64[kStatsSlots(R)]
    size_t total;
    int count_blocks;
};

constexpr int kCountChunk = 1024;  // assignments per counting workgroup

// Counting workgroups of the multi-launch count, and the bytes of one of its
// two per-workgroup tables (int32[B][E], 256-byte aligned).
inline int count_blocks(int64_t N) { return (int)((N + kCountChunk - 1) / kCountChunk); }
inline size_t count_table_bytes(int64_t N, int E)
{
    const int64_t B = count_blocks(N);
    return ((size_t)(B > 0 ? B : 1) * (size_t)E * 4 + 255) & ~size_t(255);
}
// Fixed device scratch of moe_count_noalloc: both tables must fit.
constexpr size_t kCountScratchBytes = size_t(8) << 20;

// bf16 grouped GEMM geometry shared by the workspace layout and the kernels:
// 256 x 256 tiles, K in 64-deep stages, at most kGemmMaxGrid persistent
// workgroups. Tiles left over after the last full round of workgroups are
// split along K; each part writes a fp32 256 x 256 partial tile.
constexpr int kGemmTile = 256;
constexpr int kGemmStageK = 64;
constexpr int kGemmMaxGrid = 256;

// Upper bound on the partial tiles one bf16 GEMM launch can write: at most
// one per workgroup, and at most (M-tiles x N-tiles) x stages.
inline int64_t gemm_part_units(const moe_shape_t& s)
{
    if (s.dtype != MOE_BF16) return 0;
    const int64_t N = (int64_t)s.T * s.k;
    if (N == 0) return 0;
    const int64_t mt = N / kGemmTile + 2 * s.E;  // at most 2E groups (by segment)
    const int64_t gu = mt * ((s.F + kGemmTile / 2 - 1) / (kGemmTile / 2)) * (s.H / kGemmStageK);
    const int64_t dn = mt * ((s.H + kGemmTile - 1) / kGemmTile) * (s.F / kGemmStageK);
    const int64_t u = gu > dn ? gu : dn;
    return u < kGemmMaxGrid ? u : kGemmMaxGrid;
}

// Statistics reduction slots (int64): fixed scalars, then three R-vectors.
enum StatSlot {
    kStN = 0, kStMax, kStMin, kStActive, kStProcessed, kStOverflow, kStPadding, kStRemoteHome,
    kStRemoteMapped, kStRemotePlanned, kStReplicas, kStMaxSlots, kStOverSlots, kStNonlocal,
    kStErr, kStScalars
};
__host__ __device__ inline int stats_slots(int R) { return kStScalars + 3 * R; }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(const moe_shape_t& s)
{
    WsLayout w;
    const int64_t N = (int64_t)s.T * s.k;
    w.count_blocks = count_blocks(N);
    size_t o = 0;
    w.blk_hist = o;  o += count_table_bytes(N, s.E);
    w.blk_base = o;  o += count_table_bytes(N, s.E);
    w.sched = o;     o = align256(o + (size_t)(4 * (2 * s.E + 1) + 64) * 4);
    w.wtab = o;      o = align256(o + (size_t)2 * s.E * 3 * 8);
    w.vrow = o;      o = align256(o + (size_t)(N > 0 ? N : 1) * 4);
    w.part = o;      o = align256(o + (size_t)gemm_part_units(s) * kGemmTile * kGemmTile * 4);
    w.skpart = o;    o = align256(o + (s.dtype == MOE_BF16 ? (size_t)2 * kGemmMaxGrid * (32 + 64) * kGemmTile * 4 : 0));
    w.h = o;         o = align256(o + (size_t)N * s.F * (s.dtype == MOE_BF16 ? 2 : 4));
    w.stats = o;     o = align256(o + (size_t)stats_slots(s.R) * 8);
    w.total = o;
    return w;
}

// Workspace of the FFN backward (bytes, 256-byte aligned regions): the
// by-expert schedule with 256-row M-tiles, the expert-order row map, a zero
// page, x and dy in expert order, the recomputed g | u, dg | du and h.
struct BwdWsLayout {
    size_t sched, vrow, zero, xs, dys, gu, dgu, hb, dxpart, rgroups, slot_of, total;
};
// Replica weight-gradient slots (training, one per rank and replica
// position): [R][n][3][F*H] fp32, gate | up | down of the replica held there.
inline size_t replica_grad_bytes(const moe_shape_t& s)
{
    return (size_t)s.R * (s.E / s.R) * 3 * s.F * s.H * 4;
}
// Bound on the dx GEMM's K-split: 4 when its tiles (at most N/256 + E
// M-tiles x H/256 N-tiles) cannot fill four rounds of the persistent grid.
inline int bwd_dx_split_max(const moe_shape_t& s)
{
    const int64_t N = (int64_t)s.T * s.k;
    const int64_t tiles = (N / kGemmTile + s.E) * ((s.H + kGemmTile - 1) / kGemmTile);
    return tiles >= 4 * kGemmMaxGrid ? 1 : 4;
}
inline BwdWsLayout bwd_ws_layout(const moe_shape_t& s)
{
    const size_t N = (size_t)s.T * s.k;
    const size_t n1 = N > 0 ? N : 1;
    BwdWsLayout b;
    size_t o = 0;
    b.sched = o; o = align256(o + (size_t)(4 * (s.E + 1) + 64) * 4);
    b.vrow = o;  o = align256(o + n1 * 4);
    b.zero = o;  o = align256(o + 512);
    const size_t eb = s.dtype == MOE_BF16 ? 2 : 4;
    b.xs = o;    o = align256(o + n1 * s.H * eb);
    b.dys = o;   o = align256(o + n1 * s.H * eb);
    b.gu = o;    o = align256(o + n1 * 2 * s.F * eb);
    b.dgu = o;   o = align256(o + n1 * 2 * s.F * eb);
    b.hb = o;    o = align256(o + n1 * s.F * eb);
    const int sp = s.dtype == MOE_BF16 ? bwd_dx_split_max(s) : 1;
    b.dxpart = o; o = align256(o + (sp > 1 ? (size_t)sp * n1 * s.H * 4 : 4));
    b.rgroups = o; o = align256(o + (size_t)2 * s.E * 4 * 4);   // {e, k0, k1, out} per group
    b.slot_of = o; o = align256(o + (size_t)s.E * s.R * 4);      // [E][R] replica slot or -1
    b.total = o;
    return b;
}

// Grouping of the grouped GEMM. By expert: G = E groups, an expert's pieces
// gathered into one run of rows through a row map, weights at base + e*F*H.
// By segment (replica slots): G = 2E groups, one per (rank r, segment
// position i) of the plan (group r*2n + i), each a contiguous run of buffer
// rows, with weights from a per-group table of byte addresses [G][3]
// (gate, up, down) that may point into the replica slot pool.
constexpr int kMaxGroups = 512;
struct GemmGroups {
    int G;
    bool seg;
    const uint64_t* wtab;
};
inline GemmGroups expert_groups(const moe_shape_t& s) { return GemmGroups{s.E, false, nullptr}; }

// Replica slot pool: pool[r][j][3][F*H] for j < min(S, n) slots per rank.
inline int pool_slots(const moe_shape_t& s)
{
    const int n = s.E / s.R;
    return s.S < n ? s.S : n;
}
inline size_t pool_bytes(const moe_shape_t& s)
{
    return (size_t)s.R * pool_slots(s) * 3 * s.F * s.H * (s.dtype == MOE_BF16 ? 2 : 4);
}

// Router GEMM work split (bf16): TM tokens per workgroup tile and `parts`
// K-ranges of kt_part 64-deep stages each. With parts > 1 every range writes
// an fp32 partial plane [T][E] to the caller's workspace and the top-k step
// sums the planes in range order, so the result does not depend on timing.
// Small T splits K until about 256 workgroups run (each range keeps at least
// 4 stages; at most 16 ranges).
struct RouterSplit {
    int tm, parts, kt_part;
};
inline RouterSplit router_split(const moe_shape_t& s)
{
    if (s.dtype != MOE_BF16 || s.T <= 0) return {32, 1, 0};
    const int KT = s.H / kGemmStageK;
    const int eb = s.E <= 32 ? 32 : s.E <= 64 ? 64 : s.E <= 128 ? 128 : 256;
    const int tm = (eb >= 128 && s.T >= 64 * 128) ? 64 : 32;
    const int tiles = (s.T + tm - 1) / tm;
    int parts = 1;
    if (tiles < 256) {
        parts = (256 + tiles - 1) / tiles;
        const int most = KT / 4 > 1 ? KT / 4 : 1;
        if (parts > most) parts = most;
        if (parts > 16) parts = 16;
    }
    const int ktp = (KT + parts - 1) / parts;
    return {tm, (KT + ktp - 1) / ktp, ktp};
}
inline size_t router_ws_bytes(const moe_shape_t& s)
{
    const RouterSplit r = router_split(s);
    return r.parts > 1 ? (size_t)r.parts * s.T * s.E * 4 : 0;
}

}  // namespace moe

// ---- launchers (one per kernel family; all asynchronous on `st`) ----------
// logits: `nplanes` fp32 planes [T][E], `plane` floats apart, summed in
// plane order; with logits_out != NULL the sums are also written there.
hipError_t moe_launch_route(const moe_shape_t& s, const float* logits, const float* bias,
                            int32_t* ids, float* w, int32_t* err, hipStream_t st,
                            int nplanes = 1, int64_t plane = 0, float* logits_out = nullptr);
hipError_t moe_launch_count(const moe_shape_t& s, const int32_t* ids, int32_t* counts,
                            int32_t* offsets, int32_t* eidx, int32_t* rank_load, int32_t* err,
                            char* ws, hipStream_t st);
// moe_count with its tables in the library's fixed device scratch
// (kCountScratchBytes per GPU) instead of a workspace; the caller checks
// 2 * count_table_bytes(N, E) <= kCountScratchBytes.
hipError_t moe_launch_count_noalloc(const moe_shape_t& s, const int32_t* ids, int32_t* counts,
                                    int32_t* offsets, int32_t* eidx, int32_t* rank_load,
                                    int32_t* err, hipStream_t st);
hipError_t moe_launch_plan(const moe_shape_t& s, const int32_t* counts, int32_t* plan,
                           hipStream_t st);
// moe_launch_count then moe_launch_plan, in one launch up to 16384
// assignments.
hipError_t moe_launch_count_plan(const moe_shape_t& s, const int32_t* ids, int32_t* counts,
                                 int32_t* offsets, int32_t* eidx, int32_t* rank_load,
                                 int32_t* err, char* ws, int32_t* plan, hipStream_t st);
hipError_t moe_launch_permute(const moe_shape_t& s, const void* x, const int32_t* ids,
                              const int32_t* eidx, const int32_t* plan, void* buf,
                              int32_t* dest_row, int32_t* row_src, hipStream_t st);
hipError_t moe_launch_combine(const moe_shape_t& s, const void* y, const int32_t* dest_row,
                              const float* w, const void* shared_y, void* out, hipStream_t st);
hipError_t moe_launch_gemm_schedule(const moe_shape_t& s, const int32_t* plan, char* ws,
                                    hipStream_t st, const moe::GemmGroups& g);
// gu_out (bf16 [N][2F] in expert order, g | u), when not NULL, also receives
// the gate and up projections (training: the backward then skips its recompute)
hipError_t moe_launch_gemm_gateup(const moe_shape_t& s, const void* a, const int32_t* plan,
                                  const void* w_gate, const void* w_up, char* ws,
                                  hipStream_t st, const moe::GemmGroups& g,
                                  void* gu_out = nullptr);
hipError_t moe_launch_gemm_down(const moe_shape_t& s, const int32_t* plan, const void* w_down,
                                void* y, char* ws, hipStream_t st, const moe::GemmGroups& g);
// by-expert schedule with 256-row M-tiles only (no skinny tiles) + row map
hipError_t moe_launch_gemm_schedule_bm(const moe_shape_t& s, const int32_t* plan, int32_t* sched,
                                       int32_t* vrow, hipStream_t st);
// the expert FFN backward (bf16): gathers, recompute, dgrad, wgrad
// rgrad (bf16 layers): NULL, or the replica gradient slots -- then each
// replica piece's weight gradient goes to its slot and a reduction adds the
// slots into their home experts (rank order)
hipError_t moe_launch_ffn_backward(const moe_shape_t& s, const void* buf, const int32_t* plan,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const void* gu, const void* dy, void* dbuf, float* dw_gate,
                                   float* dw_up, float* dw_down, char* ws, hipStream_t st,
                                   float* rgrad = nullptr);
// combine / dispatch / gate backward
hipError_t moe_launch_combine_backward(const moe_shape_t& s, const void* dout, const void* y,
                                       const int32_t* dest_row, const float* w, void* dy,
                                       float* dw, hipStream_t st);
hipError_t moe_launch_route_backward(const moe_shape_t& s, const int32_t* ids, const float* w,
                                     const float* dw, float* dlogits, hipStream_t st);
// replica slots: the pool copy, and the per-segment weight table
hipError_t moe_launch_prefetch(const moe_shape_t& s, const int32_t* plan, const void* w_gate,
                               const void* w_up, const void* w_down, void* pool, hipStream_t st);
hipError_t moe_launch_slot_table(const moe_shape_t& s, const int32_t* plan, const void* w_gate,
                                 const void* w_up, const void* w_down, const void* pool,
                                 uint64_t* wtab, hipStream_t st);
hipError_t moe_launch_combine_rows(const moe_shape_t& s, int64_t nrows, const void* y,
                                   const int32_t* dest_row, const float* w, const void* shared_y,
                                   void* out, hipStream_t st);
hipError_t moe_launch_capacity_dispatch(const moe_shape_t& s, int cap, const int32_t* counts,
                                        const void* x, const int32_t* ids, const int32_t* eidx,
                                        void* buf, int32_t* dest_row, hipStream_t st);
hipError_t moe_launch_capacity_plan(const moe_shape_t& s, int cap, int32_t* plan, hipStream_t st);
hipError_t moe_launch_repack(const moe_shape_t& s, const int32_t* counts, int32_t* mapping,
                             hipStream_t st);
// router_split(s).parts == 1: logits [T][E]; else the partial planes.
hipError_t moe_launch_router_logits(const moe_shape_t& s, const void* x, const void* w_router,
                                    float* logits, hipStream_t st);
hipError_t moe_launch_bias_update(const moe_shape_t& s, const int32_t* counts, float gamma,
                                  float* bias, hipStream_t st);
hipError_t moe_launch_stats(const moe_shape_t& s, const int32_t* counts, const int32_t* ids,
                            const int32_t* plan, const int32_t* dest_row, const int32_t* mapping,
                            const int32_t* origin, const int32_t* err, int32_t capacity,
                            int64_t* d_out, hipStream_t st);
