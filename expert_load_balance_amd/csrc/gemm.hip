// gemm.hip -- the grouped SwiGLU expert GEMM over the plan.
//
// "DeepEP-on-EFA Guidance, section 1", phase (c): every expert runs its FFN
// over the rows it received, as a batched grouped GEMM.
// "Moonshot AI drops MoonEP ..." paragraph 3: one contiguous weight tensor
// per projection ([E][F][H] gate and up, [E][H][F] down); replicas of an
// expert read the same slice (one GPU holds every expert).
//
// Rows of expert e are its pieces in rank order, i.e. the virtual rows
// v = 0 .. c_e-1 map to buf rows piece_row[p] + (v - cum_p). M-tiles are cut
// per expert over these virtual rows (not per piece), so a replica split
// costs no extra tile. A device-side schedule (prefix of per-expert tile
// counts) lets a static grid find its tile with no host round trip.
//
// Two launches:
//   gate/up: h[row_start[e] + v][f] = silu(a_v . Wg[e][f]) * (a_v . Wu[e][f])
//            (h stored expert-contiguous, rounded to bf16 in bf16 mode);
//   down:    y[buf row of v][o] = h[row_start[e] + v] . Wd[e][o].
// bf16 path: a persistent MFMA kernel (below); fp32 path: plain LDS-tiled
// VALU kernels for small shapes.
#include <type_traits>

#include "common.h"
#include "lds_pipe.h"

namespace {

using namespace moe::lds;


constexpr int kThreads = 256;

// Relative cost of one K-stage of a bf16 tile on one CU: a skinny tile
// streams 36 or 40 KB of operands (per-CU copy rate bound), a 256-row tile
// runs 64 MFMAs per wave on 64 KB. For splitting a launch between the two
// kinds. The 256-row cost was swept from 1.0 to 3.2 over six workloads:
// 1.6-1.8 is best; from 2.0 up the skinny side gets 8 workgroups too few on
// some and finishes last.
constexpr float kCostSk32 = 1.0f, kCostSk64 = 1.1f, kCostMain = 1.6f;
// Least share of that cost on skinny tiles for which the last rows of
// larger groups go to skinny tiles (below it, the split's granularity of 8
// workgroups decides the balance).
constexpr float kTailMinShare = 1.0f / 16;

// schedule layout inside the workspace region (int32), G groups (experts, or
// plan segments; see moe::GemmGroups):
//   [0 .. G]            tile_start: prefix of the group's M-tiles of bm rows
//   [G+1 .. 2G+1]       row_start:  prefix of the group's rows c_g
//   [2G+2 .. 3G+2]      prefix of (0 < t_g <= sk1): one sk1-row tile each
//   [3G+3 .. 4G+3]      prefix of (sk1 < t_g <= sk2): one sk2-row tile each
// Groups of at most sk2 rows get one skinny tile (t_g = c_g), larger ones
// bm-row M-tiles. With tails, the last t_g = c_g mod bm rows of a larger
// group go to one skinny tile instead when t_g <= sk2; tails are taken when
// the skinny tiles then hold at least kTailMinShare of the estimated cost.
// sk1 = sk2 = 0: every group is cut into M-tiles only.

// rows of group g: by expert, the sum of its pieces; by segment, the
// segment's count (group r*2n + i, none past seg_num[r])
__device__ __forceinline__ int group_rows(int g, int E, int R, bool seg, const int32_t* plan,
                                          const moe::PlanLayout& L)
{
    if (seg) {
        const int n2 = 2 * (E / R);
        const int r = g / n2, i = g % n2;
        return i < plan[L.seg_num + r] ? plan[L.seg_cnt + g] : 0;
    }
    const int np = plan[L.piece_num + g];
    int c = 0;
    for (int p = 0; p < np && p < R; ++p) c += plan[L.piece_cnt + (size_t)g * R + p];
    return c;
}

// Thread t of a workgroup owns groups 2t and 2t+1 (G <= kMaxGroups). Every
// workgroup computes the schedule; workgroup 0 writes it. With vrow, the
// same launch then fills vrow (below), workgroup b its rows 256 b ..
// 256 b + 255, from the row prefix it holds in LDS: one launch instead of two
// dependent ones.
__global__ __launch_bounds__(kThreads) void schedule_kernel(int G, int E, int R, int seg, int bm,
                                                            int sk1, int sk2, int N,
                                                            const int32_t* __restrict__ plan,
                                                            int32_t* __restrict__ sched,
                                                            int32_t* __restrict__ vrow)
{
    __shared__ int32_t sh[4][kThreads];
    __shared__ int32_t rs[moe::kMaxGroups + 1];
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int tid = threadIdx.x;
    int cg[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int g = 2 * tid + h;
        cg[h] = g < G ? group_rows(g, E, R, seg != 0, plan, L) : 0;
    }
    // the tiles with tails, summed over the groups: tails or not
    int tm = 0, ts1 = 0, ts2 = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int full = cg[h] / bm, tail = cg[h] - full * bm;
        tm += full + (tail > sk2 ? 1 : 0);
        ts1 += tail > 0 && tail <= sk1 ? 1 : 0;
        ts2 += tail > sk1 && tail <= sk2 ? 1 : 0;
    }
    sh[0][tid] = tm;
    sh[1][tid] = ts1;
    sh[2][tid] = ts2;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (tid < off)
#pragma unroll
            for (int q = 0; q < 3; ++q) sh[q][tid] += sh[q][tid + off];
        __syncthreads();
    }
    const float cost_sk = kCostSk32 * (float)sh[1][0] + kCostSk64 * (float)sh[2][0];
    const bool tails = sk2 > 0 && cost_sk >= kTailMinShare * (cost_sk + kCostMain * (float)sh[0][0]);
    __syncthreads();
    int v[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = cg[h];
        const int full = c / bm;
        const int tail = tails || c <= sk2 ? c - full * bm : 0;  // rows for a skinny tile
        v[h][0] = full + (tail > sk2 || (tail == 0 && c > full * bm) ? 1 : 0);
        v[h][1] = c;
        v[h][2] = tail > 0 && tail <= sk1 ? 1 : 0;
        v[h][3] = tail > sk1 && tail <= sk2 ? 1 : 0;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) sh[q][tid] = v[0][q] + v[1][q];
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        int a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = tid >= off ? sh[q][tid - off] : 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) sh[q][tid] += a[q];
        __syncthreads();
    }
    // inclusive prefix through group 2t+1 is sh[q][tid]; through 2t, minus v[1]
    if (blockIdx.x == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int32_t* out = sched + q * (G + 1);
            if (tid == 0) out[0] = 0;
            if (2 * tid < G) out[2 * tid + 1] = sh[q][tid] - v[1][q];
            if (2 * tid + 1 < G) out[2 * tid + 2] = sh[q][tid];
        }
    }
    if (vrow == nullptr) return;

    // vrow[x] = buf row of the x-th row in group order (group g owns x in
    // [row_start[g], row_start[g+1])). By expert: its v-th row lives in the
    // piece that covers v, pieces taken in rank order. By segment: seg_row + v.
    if (tid == 0) rs[0] = 0;
    if (2 * tid < G) rs[2 * tid + 1] = sh[1][tid] - v[1][1];
    if (2 * tid + 1 < G) rs[2 * tid + 2] = sh[1][tid];
    __syncthreads();
    const int x = blockIdx.x * kThreads + tid;
    if (x >= N) return;
    const int32_t* row_start = rs;
    int lo = 0, hi = G - 1;  // last group with row_start <= x (that group is non-empty)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (row_start[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    const int vr = x - row_start[lo];
    if (seg) {
        vrow[x] = plan[L.seg_row + lo] + vr;
        return;
    }
    const int np = plan[L.piece_num + lo];
    int cum = 0, row = 0;
    for (int p = 0; p < np && p < R; ++p) {
        const int c = plan[L.piece_cnt + (size_t)lo * R + p];
        if (vr < cum + c) {
            row = plan[L.piece_row + (size_t)lo * R + p] + (vr - cum);
            break;
        }
        cum += c;
    }
    vrow[x] = row;
}

struct Tile {
    int e, v0, rows, hrow0;  // expert, first virtual row, rows in tile, h row of v0
};

// Finds the tile of M-tile index mt; rows == 0 if past the end.
__device__ __forceinline__ Tile find_tile(int mt, int E, int bm, const int32_t* sched)
{
    Tile t{0, 0, 0, 0};
    if (mt >= sched[E]) return t;
    int lo = 0, hi = E - 1;  // largest e with tile_start[e] <= mt
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sched[mid] <= mt) lo = mid;
        else hi = mid - 1;
    }
    const int c = sched[E + 1 + lo + 1] - sched[E + 1 + lo];
    t.e = lo;
    t.v0 = (mt - sched[lo]) * bm;
    t.rows = min(bm, c - t.v0);
    t.hrow0 = sched[E + 1 + lo] + t.v0;
    return t;
}

// Virtual row v of expert e -> buf row (walks at most R pieces).
__device__ __forceinline__ int buf_row_of(int e, int v, int R, const int32_t* plan,
                                          const moe::PlanLayout& L)
{
    const int np = plan[L.piece_num + e];
    int cum = 0;
    for (int p = 0; p < np && p < R; ++p) {
        const int c = plan[L.piece_cnt + (size_t)e * R + p];
        if (v < cum + c) return plan[L.piece_row + (size_t)e * R + p] + (v - cum);
        cum += c;
    }
    return 0;
}

// ---------------------------------------------------------------- bf16 ----
// Persistent kernel, one 256-thread workgroup per CU. Workgroup tile: 256
// rows x 256 B-rows (gate/up: 128 F-columns of gate and the same 128 of up;
// down: 256 output columns); K in 64-deep stages.
//  * LDS holds a ring of operand slots of 32 KB: two for A, three for B, so
//    the weights (from HBM, unlike the activation rows every N-tile of an
//    expert shares in L2) are copied two stages ahead. A slot row is 128
//    bytes, one full L1/L2 line of the source row, so every line is fetched
//    once. K-chunk c of row r sits in slot c ^ swz(r), which keeps the MFMA
//    fragment reads (32 consecutive rows, one chunk each) free of bank
//    conflicts.
//  * Global -> LDS with global_load_lds_dwordx4: lane l of an instruction
//    lands at its LDS base + 16 l (8 rows of 128 bytes per instruction), so
//    the swizzle is applied on the source side: each lane's source is a
//    fixed 32-bit offset from a uniform base.
//  * 4 waves in 2 x 2, each 128 rows x 128 B-rows with
//    v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane, in AGPRs).
//    Operands are swapped so a lane holds 4 consecutive output columns: the
//    epilogue stores 8 bytes per lane straight to global memory.
//  * Stage s, hand-scheduled over its 4 k-steps of 16 MFMAs: the fragments
//    of all four k-steps are read from its slots during k-steps 0 and 1; one
//    workgroup barrier follows (the slots are then free, and stage s+1 has
//    landed: each wave waits for its own copies first); the copies of A of
//    stage s+2 and B of stage s+3 into the freed slots and the first
//    fragments of stage s+1 are spread over k-steps 2 and 3.
//  * The next tile's first two stages are issued right after the last
//    stage's barrier, ahead of this tile's epilogue, whose arithmetic and
//    stores then hide their latency.
//  * Tile order: expert, N-tile, M-tile (M fastest), so the M-tiles sharing
//    a weight tile run together; each XCD takes a contiguous run of tiles so
//    they share its L2.
//  * Balance: workgroup p takes work units p, p + P, ... Whole tiles fill as
//    many full rounds of the P workgroups as they can; the tiles left over
//    (fewer than P) are split along K into as many parts as the idle
//    workgroups allow, each part writing a fp32 partial tile that
//    fixup_kernel sums (parts in order) and finishes. No workgroup waits on
//    another.
constexpr int kTM = moe::kGemmTile, kTN = moe::kGemmTile, kTK = moe::kGemmStageK;
constexpr int kOpBytes = kTM * kTK * 2;           // 32 KB: one operand of one stage
constexpr int kCopiesWave = kOpBytes / 1024 / 4;  // 8 copies per operand per wave
constexpr int kASlots = 2, kBSlots = 3;           // LDS ring: 5 x 32 KB = 160 KB
enum { kGateUp = 0, kDown = 1 };

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (both about
// 1 ulp); the product is rounded to bf16 right after.
__device__ __forceinline__ float fast_silu(float z)
{
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// Fragment-read slots. A fragment set (one k-step) is 8 reads: A blocks
// 0..3 and B blocks 0..3 (ids 0..3 and 4..7), issued in the order a0 b0 b1
// b2 b3 a1 a2 a3 (the first MFMAs of a k-step need every B block). During
// k-steps 0 and 1 a read follows MFMAs m % 4 != 3 (12 per k-step): k-step 0
// reads set 1 and the first half of set 2, k-step 1 the rest of set 2 and
// set 3. During k-steps 2 and 3 a read follows MFMAs m % 4 == 0 (set 0 of the
// next stage, half each) and a copy follows every odd MFMA.
__host__ __device__ constexpr int read_order(int n) { return n == 0 ? 0 : n <= 4 ? n + 3 : n - 4; }

// Tile t of the launch (expert-major, then N-tile, then M-tile) from the
// schedule (tile_start[E+1], row_start[E+1]); sc(i) reads its entry i.
struct TileRef {
    int e, n0, rows, hrow0;
};
// The tile t of group lo (lo: the group whose tiles hold t).
template <int MODE, bool SKINNY, typename SC>
__device__ __forceinline__ TileRef tile_in_group(int t, int lo, int E, int ntiles_n, SC sc)
{
    const int mt_e = sc(lo + 1) - sc(lo);
    const int local = t - sc(lo) * ntiles_n;
    const int nt = local / mt_e, mt = local % mt_e;
    const int c_e = sc(E + 1 + lo + 1) - sc(E + 1 + lo);
    const int v0 = SKINNY ? c_e / kTM * kTM : mt * kTM;
    TileRef r;
    r.e = lo;
    r.n0 = nt * (MODE == kGateUp ? kTN / 2 : kTN);
    r.rows = min(kTM, c_e - v0);
    r.hrow0 = sc(E + 1 + lo) + v0;
    return r;
}

// SKINNY: t indexes a skinny-tile table (one tile per group and N-tile),
// whose tile holds the group's rows past its whole M-tiles.
template <int MODE, bool SKINNY = false, typename SC>
__device__ __forceinline__ TileRef tile_of(int t, int E, int ntiles_n, SC sc)
{
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sc(mid) * ntiles_n <= t) lo = mid;
        else hi = mid - 1;
    }
    return tile_in_group<MODE, SKINNY>(t, lo, E, ntiles_n, sc);
}

// tile_of for a whole workgroup (every thread calls it, with the same t):
// the group is found in one round of independent loads, thread i testing
// whether t falls in groups i, i + 256, ... (one non-empty interval holds
// it), instead of a binary search of dependent loads. For kernels whose
// first step is the lookup (the fixups).
template <int MODE, bool SKINNY = false, typename SC>
__device__ __forceinline__ TileRef tile_of_wg(int t, int E, int ntiles_n, SC sc)
{
    __shared__ int grp;
    for (int i = threadIdx.x; i < E; i += kThreads)
        if (sc(i) * ntiles_n <= t && t < sc(i + 1) * ntiles_n) grp = i;
    __syncthreads();
    // (callers pass a tile of the launch, so one group matched; the clamp
    // only keeps the reads in the table)
    return tile_in_group<MODE, SKINNY>(t, min(max(grp, 0), E - 1), E, ntiles_n, sc);
}

// Work split of `tiles` tiles over P workgroups: `full` whole-tile units,
// then L leftover tiles in S K-parts of KTp stages (S == 1: no split).
struct Balance {
    int full, L, S, KTp;
};
__device__ __forceinline__ Balance balance_of(int tiles, int P, int KT_all)
{
    Balance b;
    b.full = tiles / P * P;
    b.L = tiles - b.full;
    b.S = 1;
    b.KTp = KT_all;
    if (b.L > 0) {
        const int s0 = min(P / b.L, KT_all);
        if (s0 > 1) {
            b.KTp = (KT_all + s0 - 1) / s0;
            b.S = (KT_all + b.KTp - 1) / b.KTp;  // every part non-empty
        }
    }
    if (b.S == 1) {
        b.full = tiles;
        b.L = 0;
    }
    return b;
}

// g | u of one row (bf16) at row x of gu [N][2F]: 4 columns from col, taken
// from accumulator group g4 of the gate and up fragments
__device__ __forceinline__ void store_gu(uint16_t* gu, int x, int F, int col, const f32x16& g,
                                         const f32x16& u, int g4)
{
    uint16_t* d = gu + (size_t)x * 2 * F + col;
    uint2 pk;
    pk.x = moe::pack_bf16x2(g[g4 * 4], g[g4 * 4 + 1]);
    pk.y = moe::pack_bf16x2(g[g4 * 4 + 2], g[g4 * 4 + 3]);
    *reinterpret_cast<uint2*>(d) = pk;
    pk.x = moe::pack_bf16x2(u[g4 * 4], u[g4 * 4 + 1]);
    pk.y = moe::pack_bf16x2(u[g4 * 4 + 2], u[g4 * 4 + 3]);
    *reinterpret_cast<uint2*>(d + F) = pk;
}

struct Unit {
    int e, n0, rows, hrow0, KT, kofs, pidx;  // e: group; pidx: partial-tile slot, -1 for a whole tile
    int rot;                                 // first K-stage of the unit's loop (see kst)
};

// Weights of projection q (0 gate, 1 up, 2 down) for group g: from the
// per-group table when there is one (grouping by segment), else expert g's
// slice of the base tensor (F x H elements each).
template <typename T>
__device__ __forceinline__ const T* group_w(const uint64_t* wtab, const T* base, int g, int q, int F,
                                            int H)
{
    if (wtab) return reinterpret_cast<const T*>(wtab[3 * g + q]);
    return base + (size_t)g * F * H;
}

// The 256-row tiles on P workgroups of the launch, this one being bid
// (0 <= bid < P, P a multiple of 8). slots: the whole LDS, A slots 0, 1,
// then B slots 0, 1, 2.
template <int MODE>
__device__ __forceinline__ void main_tiles(
    int P, int bid, char* slots, int G, int ntiles_n, int H, int F,
    const uint16_t* __restrict__ a_src, const int32_t* __restrict__ sched,
    const int32_t* __restrict__ vrow, const uint16_t* __restrict__ w0,
    const uint16_t* __restrict__ w1, const uint64_t* __restrict__ wtab,
    uint16_t* __restrict__ out, float* __restrict__ part, uint16_t* __restrict__ gu_out)
{
    auto sc = [&](int i) { return ldc(sched, i); };

    const int K = MODE == kGateUp ? H : F;
    const int KT_all = K / kTK;
    const Balance bal = balance_of(sc(G) * ntiles_n, P, KT_all);
    const int total = bal.full + bal.L * bal.S;
    const int per_xcd = P / 8;
    const int my_slot = (bid % 8) * per_xcd + bid / 8;

    const int tid = threadIdx.x;
    const int wave = uni(tid >> 6), lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31, fh = lane >> 5;
    const uint32_t slots_u = (uint32_t)(uintptr_t)slots;
    // fragment byte offsets inside an operand stage, k-steps 0..3
    uint32_t fa[4], fb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint32_t ch = (uint32_t)(((2 * kk + fh) ^ swz(fr)) * 16);
        fa[kk] = (uint32_t)(wm * 128 + fr) * 128u + ch;
        fb[kk] = (uint32_t)((MODE == kGateUp ? wn * 64 : wn * 128) + fr) * 128u + ch;
    }

    // work unit -> (tile, K range, partial slot); uniform. Partial units go
    // part-major so that neighbouring workgroups share weight tiles.
    auto decode = [&](int Lu) {
        int t = Lu, k0 = 0, KT = KT_all, pidx = -1;
        if (Lu >= bal.full) {
            pidx = Lu - bal.full;
            const int kp = pidx / bal.L;
            t = bal.full + pidx % bal.L;
            k0 = kp * bal.KTp;
            KT = min(KT_all - k0, bal.KTp);
        }
        const TileRef r = tile_of<MODE>(t, G, ntiles_n, sc);
        Unit u;
        u.e = uni(r.e);
        u.n0 = uni(r.n0);
        u.rows = uni(r.rows);
        u.hrow0 = uni(r.hrow0);
        u.KT = uni(KT);
        u.kofs = uni(k0 * kTK);
        u.pidx = uni(pidx);
        u.rot = MODE == kDown && F % 2048 == 0 ? uni((r.n0 >> 7) % KT) : 0;
        return u;
    };

    // Rows a lane needs from vrow, per unit: gate/up, the activation row of
    // each of its copies (slot row 8 (wave + 4 i) + lane / 8); down, the
    // output row of each of its accumulator blocks i (tile row
    // wm * 128 + 32 i + lane % 32). Rows past the unit's end look up row 0's
    // (their A copies land zeros, see setup).
    constexpr int kRowLoads = MODE == kGateUp ? kCopiesWave : 4;
    auto load_rows = [&](const Unit& u, int* rw) {
#pragma unroll
        for (int i = 0; i < kRowLoads; ++i) {
            const int r = MODE == kGateUp ? 8 * (wave + 4 * i) + (lane >> 3) : wm * 128 + 32 * i + fr;
            rw[i] = vrow[u.hrow0 + (r < u.rows ? r : 0)];
        }
    };

    // per-unit copy sources: uniform bases + per-lane 32-bit offsets. Copy
    // instruction q (0..31) of an operand fills slot rows 8q .. 8q+7; wave w
    // issues q = w + 4 i; lane l takes row 8q + l/8, slot chunk l % 8. A rows
    // past the unit's end take the out-of-range offset and land as zeros.
    const char *abase = nullptr, *bbase0 = nullptr, *bbase1 = nullptr;
    uint32_t aoff[kCopiesWave], boff[kCopiesWave];
    int krot = 0, kkt = 1;
    auto setup = [&](const Unit& u, const int* rw) {
        krot = u.rot;
        kkt = u.KT;
        if (MODE == kGateUp) {
            abase = uni_ptr(reinterpret_cast<const char*>(a_src + u.kofs));
            bbase0 = uni_ptr(reinterpret_cast<const char*>(group_w(wtab, w0, u.e, 0, F, H) + u.kofs));
            bbase1 = uni_ptr(reinterpret_cast<const char*>(group_w(wtab, w1, u.e, 1, F, H) + u.kofs));
        } else {
            abase = uni_ptr(reinterpret_cast<const char*>(a_src + (size_t)u.hrow0 * F + u.kofs));
            bbase0 = uni_ptr(reinterpret_cast<const char*>(group_w(wtab, w0, u.e, 2, F, H) + u.kofs));
            bbase1 = bbase0;
        }
#pragma unroll
        for (int i = 0; i < kCopiesWave; ++i) {
            const int r = 8 * (wave + 4 * i) + (lane >> 3);
            const uint32_t ch = (uint32_t)(((lane & 7) ^ swz(r)) * 16);
            if (MODE == kGateUp) {
                aoff[i] = r < u.rows ? (uint32_t)rw[i] * (uint32_t)H * 2u + ch : kZeroRow;
                boff[i] = (uint32_t)min(u.n0 + (r & 127), F - 1) * (uint32_t)H * 2u + ch;
            } else {
                aoff[i] = r < u.rows ? (uint32_t)r * (uint32_t)F * 2u + ch : kZeroRow;
                boff[i] = (uint32_t)min(u.n0 + r, H - 1) * (uint32_t)F * 2u + ch;
            }
        }
    };
    // LDS byte offsets of stage st's A and B operands. zo is zero, set by an
    // opaque move at the top of every unit: offsets of fixed stages (the
    // prologue's, the first reads) are then computed where they are used,
    // not hoisted out of the unit loop to hold registers across it.
    uint32_t zo = 0;
    auto a_slot = [&](int st) { return zo + (uint32_t)(st & 1) * kOpBytes; };
    auto b_slot = [&](int st) { return zo + (uint32_t)(kASlots + st % kBSlots) * kOpBytes; };
    // Stage st of a unit covers K-stage kst(st) = (st + rot) mod KT of its
    // range. With rot = 0 every workgroup walks K from the same stage, so the
    // lines in flight across the chip lie at the same offset within their
    // rows; when the rows are a multiple of 4 KB apart those lines share
    // their low address bits and crowd a few memory channels. The down
    // projection then starts each N-tile two stages after the previous one
    // (units of one N-tile, which share its weight tile, stay in step), and
    // only the order of the fp32 sum over K changes. Measured on the
    // DeepSeek-V3 shape's down projection (F = 2048, 4 KB rows): 11 % faster
    // at maxvio 0, 1 % at maxvio 20. Not done elsewhere: on rows of 1.5 and
    // 3 KB the same stagger cost 2-5 %, and on gate/up it changed nothing.
    auto kst = [&](int st) {
        const int x = st + krot;
        return x >= kkt ? x - kkt : x;
    };
    // copies of stage st (gate/up: B instructions q < 16, i.e. i < 4, hold
    // gate rows)
    auto copy_a = [&](int st, int i) {
        copy16_or_zero(abase + kst(st) * (kTK * 2), aoff[i], slots_u + a_slot(st) + wave * 1024 + i * 4096);
    };
    auto copy_b = [&](int st, int i) {
        copy16((i < 4 ? bbase0 : bbase1) + kst(st) * (kTK * 2), boff[i],
               slots_u + b_slot(st) + wave * 1024 + i * 4096);
    };
    // A and B of stage 0 (head), then of stage 1 (tail), in this order: the
    // waits below count the copies issued after the ones they wait for.
    // Between the two a finished tile can be staged in the slots the tail
    // fills.
    auto prologue_head = [&]() {
#pragma unroll
        for (int i = 0; i < kCopiesWave; ++i) copy_a(0, i);
#pragma unroll
        for (int i = 0; i < kCopiesWave; ++i) copy_b(0, i);
    };
    auto prologue_tail = [&](const Unit& u) {
        if (u.KT > 1) {
#pragma unroll
            for (int i = 0; i < kCopiesWave; ++i) copy_a(1, i);
#pragma unroll
            for (int i = 0; i < kCopiesWave; ++i) copy_b(1, i);
        }
    };

    f32x16 acc[4][4];
    bf16x8 af[4][4], bf[4][4];
    // fragment id (0..3 A block, 4..7 B block) of k-step kk of stage st
    auto read = [&](int st, int kk, int id) {
        if (id < 4) {
            af[kk][id] = lds_frag(slots + a_slot(st) + fa[kk] + id * 4096);
        } else {
            const int j = id - 4;
            bf[kk][j] = lds_frag(slots + b_slot(st) + fb[kk] +
                                 (MODE == kGateUp ? (j >> 1) * 16384 + (j & 1) * 4096 : j * 4096));
        }
    };
    auto mfma = [&](int kk, int m) {
        const int i = m >> 2, j = m & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[kk][j], af[kk][i], acc[i][j], 0, 0, 0);
    };

    // k-steps 0 and 1 of stage s: MFMAs interleaved with the reads of sets
    // 1, 2, 3 and, CB, the copies of B of stage s+2 into the B slot stage s-1
    // freed at its barrier (one copy per four MFMAs); then the wait for this
    // wave's copies of stage s+1 (WAIT: the copies issued after them, those
    // B copies) and the barrier. Reads: n-th read of k-step kk covers
    // set-read index 12 kk + n over the sequence (set 1: 8 reads, set 2: 8,
    // set 3: 8).
    auto first_half = [&](auto wait_tag, auto cb_tag, int s) {
        constexpr int WAIT = decltype(wait_tag)::value;
        constexpr bool CB = decltype(cb_tag)::value;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            int n = 0;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                mfma(kk, m);
                if ((m & 3) != 3) {
                    const int idx = 12 * kk + n++;  // 0..23
                    read(s, 1 + idx / 8, read_order(idx % 8));
                } else if (CB) {
                    copy_b(s + 2, 4 * kk + (m >> 2));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vm_lgkm<WAIT>();
        slot_barrier();
    };
    // k-steps 2 and 3 of stage s: stage s's slots are free; CA copies A of
    // stage s+2 into its A slot (one copy per four MFMAs); NEXT reads set 0
    // of stage s+1. So every quarter of a stage issues a quarter of the
    // copies.
    auto second_half = [&](auto ca_tag, auto next_tag, int s) {
        constexpr bool CA = decltype(ca_tag)::value;
        constexpr bool NEXT = decltype(next_tag)::value;
#pragma unroll
        for (int kk = 2; kk < 4; ++kk) {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                mfma(kk, m);
                if (NEXT && (m & 3) == 0) read(s + 1, 0, read_order(4 * (kk - 2) + (m >> 2)));
                if (CA && (m & 3) == 1) copy_a(s + 2, 4 * (kk - 2) + (m >> 2));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    using Yes = std::true_type;
    using No = std::false_type;
    using W0 = std::integral_constant<int, 0>;
    using W8 = std::integral_constant<int, kCopiesWave>;

    // The whole tiles, then the K-parts of split tiles, in two loops of their
    // own (each with its epilogue: one loop holding both would not fit its
    // registers). Workgroup p takes units p, p + P, ... of each range. The
    // first loop's last unit already issues the first K-part's copies and
    // hands it over (carry_*), as between any two units.
    int carry_Lu = -1;
    Unit carry_u{};
    int carry_rw[kRowLoads];
    auto run = [&](auto split_tag) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    const int end = SPLIT ? total : bal.full;
    int Lu;
    Unit u;
    int rw[kRowLoads];
    if (SPLIT && carry_Lu >= 0) {
        Lu = carry_Lu;
        u = carry_u;
#pragma unroll
        for (int i = 0; i < kRowLoads; ++i) rw[i] = carry_rw[i];
    } else {
        Lu = (SPLIT ? bal.full : 0) + my_slot;
        if (Lu >= end) return;
        u = decode(Lu);
        load_rows(u, rw);
        setup(u, rw);
        prologue_head();
        prologue_tail(u);
    }

    for (;;) {
        asm volatile("s_mov_b32 %0, 0" : "=s"(zo));
        // next unit and its rows (read now, used at the end of this unit;
        // these loads go out after this unit's first copies)
        const int Ln = Lu + P;
        const bool has_next = Ln < total;
        Unit un = u;
        int nrw[kRowLoads];
#pragma unroll
        for (int i = 0; i < kRowLoads; ++i) nrw[i] = 0;
        if (has_next) {
            un = decode(Ln);
            load_rows(un, nrw);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
        // stage 0 landed: the copies of stage 1 (and, with a next unit, its
        // row loads) were issued after it
        if (has_next) {
            if (u.KT >= 2) wait_vm_lgkm<2 * kCopiesWave + kRowLoads>();
            else wait_vm_lgkm<kRowLoads>();
        } else {
            if (u.KT >= 2) wait_vm_lgkm<2 * kCopiesWave>();
            else wait_vm_lgkm<0>();
        }
        slot_barrier();
#pragma unroll
        for (int n = 0; n < 8; ++n) read(0, 0, read_order(n));

        // stage s issues B and A of stage s+2 (while that exists) and waits
        // for stage s+1 (while that exists)
        int s = 0;
        for (; s + 2 < u.KT; ++s) {
            first_half(W8{}, Yes{}, s);
            second_half(Yes{}, Yes{}, s);
        }
        if (s + 1 < u.KT) {
            first_half(W0{}, No{}, s);
            second_half(No{}, Yes{}, s);
            ++s;
        }
        // last stage: after its barrier every slot is free, so the next
        // unit's first stage goes out before this unit's last MFMAs. Its row
        // loads completed with the wait above; the empty asm keeps their
        // first use here, where no copy is in flight to wait for.
        first_half(W0{}, No{}, s);
        if (has_next) {
#pragma unroll
            for (int i = 0; i < kRowLoads; ++i) asm volatile("" : "+v"(nrw[i]));
            setup(un, nrw);
            prologue_head();
        }
        second_half(No{}, No{}, s);

        // ---- epilogue: acc[i][j][4*g4 + q] is row wm*128 + 32 i + (lane & 31),
        // column (block j) 8 g4 + 4 (lane >> 5) + q, q = 0..3.
        // The finished tile is staged in B slots 1 and 2 (64 KB at a time),
        // then stored as whole 128-byte lines. A staged row's 16-byte unit c
        // sits at unit c ^ (row % 16 or 32), which spreads both the writes (32
        // rows, one unit) and the 16-byte reads (one row) over every bank.
        char* stg = slots + (kASlots + 1) * kOpBytes;
        // the lane index through an opaque copy, so that the epilogue's
        // per-lane offsets are computed here, not hoisted out of the unit
        // loop where they would stay live across the K loop
        int ln, wv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
        asm volatile("s_mov_b32 %0, %1" : "=s"(wv) : "s"(wave));
        const int er = ln & 31, eh = ln >> 5, ewm = wv >> 1, ewn = wv & 1;
        if constexpr (!SPLIT) {
            // whole tile (the down tile in two halves of 128 rows)
            if (MODE == kGateUp) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = ewm * 128 + i * 32 + er;
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            float hv[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                hv[q] = fast_silu(acc[i][j][g4 * 4 + q]) * acc[i][j + 2][g4 * 4 + q];
                            uint2 pk;
                            pk.x = moe::pack_bf16x2(hv[0], hv[1]);
                            pk.y = moe::pack_bf16x2(hv[2], hv[3]);
                            const int c = ewn * 8 + j * 4 + g4;
                            *reinterpret_cast<uint2*>(stg + row * 256 + ((c ^ (row & 15)) << 4) + eh * 8) = pk;
                            const int col = u.n0 + c * 8 + eh * 4;
                            if (gu_out && row < u.rows && col < F)  // training: keep g | u
                                store_gu(gu_out, u.hrow0 + row, F, col, acc[i][j], acc[i][j + 2], g4);
                        }
                }
                wait_vm_lgkm<63>();
                slot_barrier();
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int row = 4 * (4 * q + wv) + (ln >> 4), c = ln & 15;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * 256 + ((c ^ (row & 15)) << 4));
                    const int col = u.n0 + c * 8;
                    if (row < u.rows && col < F)
                        *reinterpret_cast<u32x4*>(out + (size_t)(u.hrow0 + row) * F + col) = v;
                }
                wait_vm_lgkm<63>();
                slot_barrier();
            } else {
                // output rows of the staged half, in A slot 1
                int32_t* orows = reinterpret_cast<int32_t*>(slots + kOpBytes);
#pragma unroll
                for (int p = 0; p < 2; ++p) {
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int i = 2 * p + ii, lr = ewm * 64 + ii * 32 + er;
                        if (eh == 0) orows[lr] = rw[i];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int g4 = 0; g4 < 4; ++g4) {
                                uint2 pk;
                                pk.x = moe::pack_bf16x2(acc[i][j][g4 * 4 + 0], acc[i][j][g4 * 4 + 1]);
                                pk.y = moe::pack_bf16x2(acc[i][j][g4 * 4 + 2], acc[i][j][g4 * 4 + 3]);
                                const int c = ewn * 16 + j * 4 + g4;
                                *reinterpret_cast<uint2*>(stg + lr * 512 + ((c ^ (lr & 31)) << 4) + eh * 8) = pk;
                            }
                    }
                    wait_vm_lgkm<63>();
                    slot_barrier();
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int lr = 2 * (4 * q + wv) + (ln >> 5), c = ln & 31;
                        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + lr * 512 + ((c ^ (lr & 31)) << 4));
                        const int row = (lr >> 6) * 128 + (2 * p + ((lr >> 5) & 1)) * 32 + (lr & 31);
                        const int col = u.n0 + c * 8;
                        if (row < u.rows && col < H)
                            *reinterpret_cast<u32x4*>(out + (size_t)orows[lr] * H + col) = v;
                    }
                    wait_vm_lgkm<63>();
                    slot_barrier();
                }
            }
        } else {
            // K-part of a split tile: the fp32 partial tile [row][B-row] that
            // fixup_kernel sums, staged 64 rows (64 KB) at a time and stored
            // as whole rows; its padding rows are stored too (fixup reads
            // only the tile's rows)
            float* dst = part + (size_t)u.pidx * kTM * kTN;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int lr = ewm * 32 + er;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int c = ((MODE == kGateUp ? (j >> 1) * 128 + ewn * 64 + (j & 1) * 32
                                                        : ewn * 128 + j * 32) + g4 * 8) / 4 + eh;
                        *reinterpret_cast<float4*>(stg + lr * 1024 + ((c ^ (lr & 15)) << 4)) =
                            make_float4(acc[p][j][g4 * 4 + 0], acc[p][j][g4 * 4 + 1],
                                        acc[p][j][g4 * 4 + 2], acc[p][j][g4 * 4 + 3]);
                    }
                wait_vm_lgkm<63>();
                slot_barrier();
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int r = 4 * q + wv;
                    const float4 v = *reinterpret_cast<const float4*>(stg + r * 1024 + ((ln ^ (r & 15)) << 4));
                    const int row = (r >> 5) * 128 + p * 32 + (r & 31);
                    *reinterpret_cast<float4*>(dst + (size_t)row * kTN + ln * 4) = v;
                }
                wait_vm_lgkm<63>();
                slot_barrier();
            }
        }
        if (has_next) prologue_tail(un);
        if (!has_next) break;
        if (Ln >= end) {  // the next unit is the K-part loop's first
            carry_Lu = Ln;
            carry_u = un;
#pragma unroll
            for (int i = 0; i < kRowLoads; ++i) carry_rw[i] = nrw[i];
            break;
        }
        Lu = Ln;
        u = un;
        for (int i = 0; i < kRowLoads; ++i) rw[i] = nrw[i];
    }
    };
    run(No{});
    run(Yes{});
}

// ------------------------------------------------------- bf16, skinny ----
// Experts with at most 64 rows (decode-like batches, cold experts under
// skew) get one SKM-row tile per N-tile (SKM = 32 or 64) instead of a mostly
// empty 256-row M-tile; when the schedule takes tails, so do the last 1..64
// rows of a larger expert, past its whole 256-row M-tiles. Such a tile is
// bound by streaming the expert's weights, so its LDS stage holds only SKM
// rows of activations next to the 32 KB weight tile and the ring is deeper:
// 4 stages (three stages of weight copies in flight per CU; 160 KB for
// SKM = 64), 3 for down's SKM = 64. Same N-tiles, K stages, swizzle, copy
// wrappers and epilogues as the 256-row tiles; 4 waves, each SKM rows x 64
// B-rows (gate/up: 32 gate and the same 32 up columns).
//
// Balance: whole rounds of tiles go to the workgroups in turn (slot w takes
// tiles w, w + P, ...); the n tiles left over (n < P), each KT stages deep,
// form one run of n*KT stages that is cut into equal contiguous pieces, one
// per workgroup (stream-K; at least kSkMinStages stages each, so a few
// tiles use fewer workgroups). A piece that covers a whole tile finishes it;
// a tile cut by a piece boundary is finished by the fixup kernel, which sums
// its parts in order. A piece is cut at most twice, so it writes at most two
// fp32 partial tiles: its first segment to slot 2q, its last (when the first
// is not also the last) to slot 2q + 1 (q: its piece).
template <int SKM>
struct Skinny {
    static constexpr int kSlots = 4;
    static constexpr int kA = SKM * kTK * 2;                  // 4 or 8 KB of A per stage
    static constexpr int kSlot = kA + kOpBytes;               // 36 or 40 KB per stage
    static constexpr int kACopies = SKM / 32;                 // A copies per wave per stage
    static constexpr int kPerStage = kACopies + kCopiesWave;  // copies per wave per stage
    static constexpr int kBlocks = SKM / 32;                  // 32-row blocks per wave
    static constexpr int kSchedOff = SKM == 32 ? 2 : 3;       // tile_start prefix (x (E+1))
};
constexpr int kSkMinStages = 8;
// parts of one cut tile: pieces hold at least KT / 32 stages (sk_cut), so a
// tile meets at most 33 of them
constexpr int kSkMaxParts = 34;

// The stream-K cut of n tiles of KT stages over P workgroups: workgroup
// piece q covers stages [first(q), first(q + 1)); pieces >= Pe are empty.
struct SkCut {
    int64_t W;  // n * KT
    int Pe;     // pieces in use
    __host__ __device__ int64_t first(int q) const { return q >= Pe ? W : (int64_t)q * W / Pe; }
    // the piece holding stage g (0 <= g < W)
    __host__ __device__ int piece_of(int64_t g) const { return (int)(((g + 1) * Pe - 1) / W); }
};
__host__ __device__ inline SkCut sk_cut(int n, int KT, int P)
{
    SkCut c;
    c.W = (int64_t)n * KT;
    // pieces of at least kSkMinStages stages and at least KT / 32, so that
    // no tile is cut into more than kSkMaxParts parts
    const int minlen = max(kSkMinStages, (KT + 31) / 32);
    const int64_t by_min = c.W / minlen;
    c.Pe = (int)(by_min < P ? (by_min > 1 ? by_min : 1) : P);
    return c;
}
// Tiles done whole, in rounds: all of them when the last round would keep at
// least half the workgroups busy (cutting its tiles then saves less than the
// partial tiles cost), else the full rounds only.
__host__ __device__ inline int sk_full_tiles(int total, int P)
{
    const int full = total / P * P;
    return total - full > P / 2 ? total : full;
}
// partial slot of the segment of piece q that starts at stage g
__host__ __device__ inline int sk_slot(const SkCut& c, int q, int64_t g)
{
    return g == c.first(q) ? 2 * q : 2 * q + 1;
}

// the SKM-row tiles of one launch (a phase of the skinny kernel below); the
// ring is the kernel's whole LDS, shared by its phases. The schedule is read
// with scalar loads and each lane keeps the gathered rows it needs in
// registers, so that all four slots fit for both tile heights. Piece q of
// the phase goes to workgroup slot (q + qofs) mod P, so a phase that uses
// fewer than P workgroups leaves the next phase the ones it did not use.
template <int MODE, int SKM>
__device__ __forceinline__ int skinny_phase(
    int G, int ntiles_n, int H, int F, const uint16_t* __restrict__ a_src,
    const int32_t* __restrict__ sched, const int32_t* __restrict__ vrow,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1,
    const uint64_t* __restrict__ wtab, uint16_t* __restrict__ out, uint16_t* __restrict__ gu_out,
    float* __restrict__ part, char* ring, int qofs, int P, int bid)
{
    using SK = Skinny<SKM>;
    // down's 64-row tiles keep three slots (measured 1-5 % faster than four
    // on the decode and dsv3 shapes, where gate/up gains 3-6 % from four)
    constexpr int kSkSlots = SKM == 64 && MODE == kDown ? 3 : SK::kSlots;
    constexpr int kSkA = SK::kA, kSkSlot = SK::kSlot;
    constexpr int kSkPerStage = SK::kPerStage, kNB = SK::kBlocks;

    // entry i of (this height's tile_start[G+1], row_start[G+1])
    auto ssched = [&](int i) {
        return i <= G ? ldc(sched, SK::kSchedOff * (G + 1) + i) : ldc(sched, i);
    };
    const int KT = (MODE == kGateUp ? H : F) / kTK;
    const int total = ssched(G) * ntiles_n;
    if (total == 0) return 0;
    // whole rounds of tiles first (workgroup slot w takes tiles w, w + P, ...),
    // then the stream-K pieces of the tiles left over
    const int nfull = sk_full_tiles(total, P);
    const SkCut cut = sk_cut(total - nfull, KT, P);
    const int per_xcd = P / 8;
    const int my_slot = (bid % 8) * per_xcd + bid / 8;
    const int q = (my_slot - qofs % P + P) % P;  // this workgroup's piece of the leftover
    int t_full = my_slot;
    int64_t g = cut.first(q);
    const int64_t g_end = cut.first(q + 1);
    // the workgroup's segments in order: (tile, first stage, end stage, partial slot or -1)
    struct Seg {
        int t, k0, k1, pslot;
    };
    auto next_seg = [&](Seg& sg) {
        if (t_full < nfull) {
            sg = Seg{t_full, 0, KT, -1};
            t_full += P;
            return true;
        }
        if (g < g_end) {
            const int tl = (int)(g / KT);
            const int k0 = (int)(g - (int64_t)tl * KT);
            const int k1 = (int)min<int64_t>((int64_t)KT, k0 + (g_end - g));
            sg = Seg{nfull + tl, k0, k1, (k0 == 0 && k1 == KT) ? -1 : sk_slot(cut, q, g)};
            g += k1 - k0;
            return true;
        }
        return false;
    };
    Seg cur;
    if (!next_seg(cur)) return cut.Pe;

    const int tid = threadIdx.x;
    const int wave = uni(tid >> 6), lane = tid & 63;
    const int fr = lane & 31, fh = lane >> 5;
    const uint32_t ring_u = (uint32_t)(uintptr_t)ring;
    // fragment byte offsets in a stage, k-steps 0..3: A rows 0..31 (row block
    // i at 32 i); B block 0 rows (gate/up) 32 wave + fr, block 1 the up rows
    // 128 further; (down) 64 wave + fr, block 1 32 further
    uint32_t fa[4], fb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint32_t ch = (uint32_t)(((2 * kk + fh) ^ swz(fr)) * 16);
        fa[kk] = (uint32_t)fr * 128u + ch;
        fb[kk] = (uint32_t)kSkA + (uint32_t)((MODE == kGateUp ? 32 : 64) * wave + fr) * 128u + ch;
    }
    constexpr int kB1 = MODE == kGateUp ? 128 * 128 : 32 * 128;  // block 1 offset

    // the next segment's tile is looked up while this one's copies fly
    TileRef rn = tile_of<MODE, true>(cur.t, G, ntiles_n, ssched);
    for (;;) {
        const int k0 = uni(cur.k0), nst = uni(cur.k1 - cur.k0), pslot = uni(cur.pslot);
        const bool whole = pslot < 0;
        const TileRef r0 = rn;
        const int e = uni(r0.e), n0 = uni(r0.n0), rows = uni(r0.rows), hrow0 = uni(r0.hrow0);
        // gathered rows: gate/up, the activation row of each A copy (needed
        // for the copies); down, the output row of each accumulator block,
        // read after the first copies go out (rows past the tile's repeat its
        // last; their A copies land zeros)
        int grow[kNB > SK::kACopies ? kNB : SK::kACopies];
        auto load_grow = [&]() {
#pragma unroll
            for (int i = 0; i < (MODE == kGateUp ? SK::kACopies : kNB); ++i) {
                const int r = MODE == kGateUp ? 8 * (wave + 4 * i) + (lane >> 3) : 32 * i + fr;
                grow[i] = vrow[hrow0 + (r < rows ? r : rows - 1)];
            }
        };
        if (MODE == kGateUp) load_grow();

        // copy sources: A row 8 wave + lane/8 (one instruction per wave), B as
        // in the 256-row kernel (8 instructions per wave); both start at
        // stage k0
        const size_t kofs = (size_t)k0 * kTK;
        const char *abase, *bbase0, *bbase1;
        if (MODE == kGateUp) {
            abase = uni_ptr(reinterpret_cast<const char*>(a_src + kofs));
            bbase0 = uni_ptr(reinterpret_cast<const char*>(group_w(wtab, w0, e, 0, F, H) + kofs));
            bbase1 = uni_ptr(reinterpret_cast<const char*>(group_w(wtab, w1, e, 1, F, H) + kofs));
        } else {
            abase = uni_ptr(reinterpret_cast<const char*>(a_src + (size_t)hrow0 * F + kofs));
            bbase0 = uni_ptr(reinterpret_cast<const char*>(group_w(wtab, w0, e, 2, F, H) + kofs));
            bbase1 = bbase0;
        }
        // A copy instruction q = wave + 4 i fills rows 8q .. 8q+7
        uint32_t aoff[SK::kACopies], boff[kCopiesWave];
#pragma unroll
        for (int i = 0; i < SK::kACopies; ++i) {
            const int ra = 8 * (wave + 4 * i) + (lane >> 3);
            const uint32_t ch = (uint32_t)(((lane & 7) ^ swz(ra)) * 16);
            aoff[i] = ra >= rows ? kZeroRow
                      : MODE == kGateUp ? (uint32_t)grow[i] * (uint32_t)H * 2u + ch
                                        : (uint32_t)ra * (uint32_t)F * 2u + ch;
        }
#pragma unroll
        for (int i = 0; i < kCopiesWave; ++i) {
            const int rb = 8 * (wave + 4 * i) + (lane >> 3);
            const uint32_t ch = (uint32_t)(((lane & 7) ^ swz(rb)) * 16);
            boff[i] = MODE == kGateUp ? (uint32_t)min(n0 + (rb & 127), F - 1) * (uint32_t)H * 2u + ch
                                      : (uint32_t)min(n0 + rb, H - 1) * (uint32_t)F * 2u + ch;
        }
        // stage st of the segment covers its K-stage (st + rot) mod nst with
        // rot = tile mod nst: as in the 256-row tiles' down projection,
        // neighbouring tiles (each streaming its own weight tile) copy
        // different 128-byte columns at once, so rows a power of two bytes
        // apart do not crowd a few memory channels. Measured against the
        // unstaggered build: decode64 @ 1 gate/up (all skinny, 8 KB rows)
        // 8 % faster, decode256 1-2 %, no change elsewhere.
        const int rot = uni(cur.t % nst);
        auto copy_stage = [&](int st) {
            const uint32_t slot = ring_u + (uint32_t)(st % kSkSlots) * kSkSlot;
            const int x = st + rot;
            const int kb = (x >= nst ? x - nst : x) * (kTK * 2);
#pragma unroll
            for (int i = 0; i < SK::kACopies; ++i)
                copy16_or_zero(abase + kb, aoff[i], slot + wave * 1024 + i * 4096);
#pragma unroll
            for (int i = 0; i < kCopiesWave; ++i)
                copy16((i < 4 ? bbase0 : bbase1) + kb, boff[i], slot + kSkA + wave * 1024 + i * 4096);
        };
        f32x16 acc[kNB][2];
#pragma unroll
        for (int b = 0; b < kNB; ++b)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int qq = 0; qq < 16; ++qq) acc[b][j][qq] = 0.0f;
        constexpr int kAhead = kSkSlots - 1;  // stages in flight beyond the current one
        for (int st = 0; st < kAhead && st < nst; ++st) copy_stage(st);
        if (MODE == kDown) load_grow();
        Seg nxt;
        const bool more = next_seg(nxt);
        if (more) rn = tile_of<MODE, true>(nxt.t, G, ntiles_n, ssched);

        for (int s = 0; s < nst; ++s) {
            // stage s landed: this wave's copies of later stages issued so far
            const int after = min(nst - 1, s + kAhead - 1) - s;
            if (after >= 2) wait_vm_lgkm<2 * kSkPerStage>();
            else if (after == 1) wait_vm_lgkm<kSkPerStage>();
            else wait_vm_lgkm<0>();
            slot_barrier();  // ... in every wave; and stage s-1's slot is free
            if (s + kAhead < nst) copy_stage(s + kAhead);
            const char* slot = ring + (s % kSkSlots) * kSkSlot;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 af[kNB];
#pragma unroll
                for (int b = 0; b < kNB; ++b) af[b] = lds_frag(slot + fa[kk] + b * 4096);
                const bf16x8 bf0 = lds_frag(slot + fb[kk]);
                const bf16x8 bf1 = lds_frag(slot + fb[kk] + kB1);
#pragma unroll
                for (int b = 0; b < kNB; ++b) {
                    acc[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf0, af[b], acc[b][0], 0, 0, 0);
                    acc[b][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf1, af[b], acc[b][1], 0, 0, 0);
                }
            }
        }

        // epilogue: acc[b][j][4 g4 + qq] is row 32 b + (lane & 31), B-row block
        // j column 8 g4 + 4 (lane >> 5) + qq
        if (whole) {
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                const int row = 32 * b + fr;
                if (row >= rows) continue;
                if (MODE == kGateUp) {
                    uint16_t* dst = out + (size_t)(hrow0 + row) * F;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int col = n0 + 32 * wave + g4 * 8 + fh * 4;
                        if (col >= F) continue;
                        float hv[4];
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq)
                            hv[qq] = fast_silu(acc[b][0][g4 * 4 + qq]) * acc[b][1][g4 * 4 + qq];
                        uint2 pk;
                        pk.x = moe::pack_bf16x2(hv[0], hv[1]);
                        pk.y = moe::pack_bf16x2(hv[2], hv[3]);
                        *reinterpret_cast<uint2*>(dst + col) = pk;
                        if (gu_out) store_gu(gu_out, hrow0 + row, F, col, acc[b][0], acc[b][1], g4);
                    }
                } else {
                    uint16_t* dst = out + (size_t)grow[b] * H;
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const int col = n0 + 64 * wave + 32 * j + g4 * 8 + fh * 4;
                            if (col >= H) continue;
                            uint2 pk;
                            pk.x = moe::pack_bf16x2(acc[b][j][g4 * 4 + 0], acc[b][j][g4 * 4 + 1]);
                            pk.y = moe::pack_bf16x2(acc[b][j][g4 * 4 + 2], acc[b][j][g4 * 4 + 3]);
                            *reinterpret_cast<uint2*>(dst + col) = pk;
                        }
                }
            }
        } else {
            // a cut tile: its fp32 partial [SKM][256] in B-row order (gate/up:
            // gate columns 0..127, up columns 128..255); padding rows too
            float* dst = part + (size_t)pslot * SKM * kTN;
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                const int row = 32 * b + fr;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int c = (MODE == kGateUp ? j * 128 + 32 * wave : 64 * wave + 32 * j) +
                                      g4 * 8 + fh * 4;
                        *reinterpret_cast<float4*>(dst + (size_t)row * kTN + c) =
                            make_float4(acc[b][j][g4 * 4 + 0], acc[b][j][g4 * 4 + 1],
                                        acc[b][j][g4 * 4 + 2], acc[b][j][g4 * 4 + 3]);
                    }
            }
        }
        // everyone is done with the ring before the next segment
        wait_vm_lgkm<63>();
        slot_barrier();
        if (!more) break;
        cur = nxt;
    }
    return cut.Pe;
}

constexpr int kSkinnyRing = Skinny<32>::kSlots * Skinny<32>::kSlot > Skinny<64>::kSlots * Skinny<64>::kSlot
                                ? Skinny<32>::kSlots * Skinny<32>::kSlot
                                : Skinny<64>::kSlots * Skinny<64>::kSlot;
constexpr int kGemmLds = kSkinnyRing > (kASlots + kBSlots) * kOpBytes ? kSkinnyRing
                                                                      : (kASlots + kBSlots) * kOpBytes;

// How a launch of P workgroups splits between the two kinds of tile: the
// first ps take the skinny tiles and the other pm the 256-row tiles, at the
// same time. A skinny tile streams its weights and a 256-row one is bound by
// its MFMAs, so running both side by side overlaps the two. The split
// follows the estimated work: a multiple of 8 (as many on every XCD), at
// least 8 for either kind that has tiles. Below 16 workgroups both kinds
// cannot have 8: then every workgroup takes the skinny tiles and then the
// 256-row ones (serial; ps = pm = P). Every workgroup and the fixup kernel
// compute the same split from the schedule.
struct Split {
    int ps, pm;
    bool serial;
};
__device__ __forceinline__ Split gemm_split(int G, int ntiles_n, int P, const int32_t* sched)
{
    const int tm = ldc(sched, G) * ntiles_n;
    const int t32 = ldc(sched, Skinny<32>::kSchedOff * (G + 1) + G) * ntiles_n;
    const int t64 = ldc(sched, Skinny<64>::kSchedOff * (G + 1) + G) * ntiles_n;
    if (t32 + t64 == 0) return Split{0, P, false};
    if (tm == 0) return Split{P, 0, false};
    if (P < 16) return Split{P, P, true};
    const float sk = kCostSk32 * (float)t32 + kCostSk64 * (float)t64;
    const float mn = kCostMain * (float)tm;
    const int ps = min(max(((int)((float)P * sk / (sk + mn)) + 4) / 8 * 8, 8), P - 8);
    return Split{ps, P - ps, false};
}

// The grouped GEMM of one projection: workgroups [0, Ps) take the skinny
// tiles (32-row ones, then 64-row ones on the workgroups the first phase left
// idle first), the rest the 256-row tiles.
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(
    int G, int ntiles_n, int H, int F, const uint16_t* __restrict__ a_src,
    const int32_t* __restrict__ sched, const int32_t* __restrict__ vrow,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1,
    const uint64_t* __restrict__ wtab, uint16_t* __restrict__ out, uint16_t* __restrict__ gu_out,
    float* __restrict__ part, float* __restrict__ part32, float* __restrict__ part64)
{
    __shared__ __attribute__((aligned(1024))) char lds[kGemmLds];
    const int P = gridDim.x, b = blockIdx.x;
    const Split sp = gemm_split(G, ntiles_n, P, sched);
    if (b < sp.ps) {
        const int used = skinny_phase<MODE, 32>(G, ntiles_n, H, F, a_src, sched, vrow, w0, w1, wtab,
                                                out, gu_out, part32, lds, 0, sp.ps, b);
        skinny_phase<MODE, 64>(G, ntiles_n, H, F, a_src, sched, vrow, w0, w1, wtab, out, gu_out,
                               part64, lds, used, sp.ps, b);
        if (!sp.serial) return;
    }
    // (the skinny phases end with every copy landed and a barrier, so the
    // LDS is free here in the serial case)
    const int mb = sp.serial ? b : b - sp.ps;
    main_tiles<MODE>(sp.pm, mb, lds, G, ntiles_n, H, F, a_src, sched, vrow, w0, w1, wtab, out, part,
                     gu_out);
}

// Finishes the skinny tiles cut by the stream-K split of the leftover
// tiles: workgroup b takes the piece boundary q = b / 2 + 1 (phase 32 first,
// then phase 64) and, if that boundary is the first one inside a tile, sums
// the tile's parts (pieces in order) for 32 of its rows (half b % 2) and
// applies the whole-tile epilogue.
constexpr int kSkFixupHalves = 2;

template <int MODE, int SKM>
__device__ __forceinline__ void skinny_fixup(int G, int ntiles_n, int H, int F, int P, int b,
                                             const int32_t* __restrict__ sched,
                                             const int32_t* __restrict__ vrow,
                                             const float* __restrict__ part,
                                             uint16_t* __restrict__ out,
                                             uint16_t* __restrict__ gu_out)
{
    using SK = Skinny<SKM>;
    auto ssched = [&](int i) { return i <= G ? sched[SK::kSchedOff * (G + 1) + i] : sched[i]; };
    const int KT = (MODE == kGateUp ? H : F) / kTK;
    const int total = ssched(G) * ntiles_n;
    if (total == 0) return;
    const int nfull = sk_full_tiles(total, P);  // tiles done whole, in rounds
    const SkCut cut = sk_cut(total - nfull, KT, P);
    const int qb = b / kSkFixupHalves + 1;    // boundary between pieces qb - 1 and qb
    const int half = b % kSkFixupHalves;
    if (qb >= cut.Pe || half * 32 >= SKM) return;
    const int64_t gb = cut.first(qb);
    const int t = (int)(gb / KT);
    const int64_t t0 = (int64_t)t * KT, t1 = t0 + KT;
    if (gb == t0) return;                          // the boundary is between tiles
    if (cut.first(qb - 1) > t0) return;            // an earlier boundary cuts this tile
    const TileRef r = tile_of_wg<MODE, true>(nfull + t, G, ntiles_n, [&](int i) { return ssched(i); });
    const int q_lo = cut.piece_of(t0), q_hi = cut.piece_of(t1 - 1);
    constexpr int kQuads = MODE == kGateUp ? kTN / 2 / 4 : kTN / 4;  // 4-column groups per row
    constexpr int kRowsPerPass = kThreads / kQuads;
    const int c = (threadIdx.x % kQuads) * 4;
    const int row_end = min(r.rows, half * 32 + 32);
    // the parts' slots, in piece order (at most kSkMaxParts)
    __shared__ int slot[kSkMaxParts];
    const int np = q_hi - q_lo + 1;
    if ((int)threadIdx.x < np) {
        const int qq = q_lo + (int)threadIdx.x;
        slot[threadIdx.x] = sk_slot(cut, qq, max(cut.first(qq), t0));
    }
    __syncthreads();
    for (int row = half * 32 + threadIdx.x / kQuads; row < row_end; row += kRowsPerPass) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), u = a;
        // eight parts' loads in flight at a time, summed in piece order
        for (int i0 = 0; i0 < np; i0 += 8) {
            float4 va[8], vu[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i0 + i < np) {
                    const float* src = part + ((size_t)slot[i0 + i] * SKM + row) * kTN + c;
                    va[i] = *reinterpret_cast<const float4*>(src);
                    if (MODE == kGateUp) vu[i] = *reinterpret_cast<const float4*>(src + kTN / 2);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i0 + i < np) {
                    a.x += va[i].x; a.y += va[i].y; a.z += va[i].z; a.w += va[i].w;
                    if (MODE == kGateUp) {
                        u.x += vu[i].x; u.y += vu[i].y; u.z += vu[i].z; u.w += vu[i].w;
                    }
                }
            }
        }
        uint2 pk;
        if (MODE == kGateUp) {
            if (r.n0 + c >= F) continue;
            pk.x = moe::pack_bf16x2(fast_silu(a.x) * u.x, fast_silu(a.y) * u.y);
            pk.y = moe::pack_bf16x2(fast_silu(a.z) * u.z, fast_silu(a.w) * u.w);
            *reinterpret_cast<uint2*>(out + (size_t)(r.hrow0 + row) * F + r.n0 + c) = pk;
            if (gu_out) {
                uint16_t* d = gu_out + (size_t)(r.hrow0 + row) * 2 * F + r.n0 + c;
                pk.x = moe::pack_bf16x2(a.x, a.y);
                pk.y = moe::pack_bf16x2(a.z, a.w);
                *reinterpret_cast<uint2*>(d) = pk;
                pk.x = moe::pack_bf16x2(u.x, u.y);
                pk.y = moe::pack_bf16x2(u.z, u.w);
                *reinterpret_cast<uint2*>(d + F) = pk;
            }
        } else {
            if (r.n0 + c >= H) continue;
            pk.x = moe::pack_bf16x2(a.x, a.y);
            pk.y = moe::pack_bf16x2(a.z, a.w);
            *reinterpret_cast<uint2*>(out + (size_t)vrow[r.hrow0 + row] * H + r.n0 + c) = pk;
        }
    }
}

// Finishes the K-split leftover tiles of a bf16 GEMM launch: sums the fp32
// partial tiles of each leftover tile in part order and writes the result
// the whole-tile epilogue would have written (gate/up: bf16 silu(g) * u into
// h; down: bf16 y rows at their buffer rows). Main item b takes leftover
// tile b / 16, rows 16 (b % 16) .. +15; a thread owns one 4-column group.
constexpr int kFixupRows = 16;
constexpr int kFixupSlabs = kTM / kFixupRows;
// split leftover tiles: at most half the persistent grid (each gets >= 2 parts)
constexpr int kFixupGrid = moe::kGemmMaxGrid / 2 * kFixupSlabs;

// The first 2 P kSkFixupHalves workgroups finish the skinny kernel's cut
// tiles (P * kSkFixupHalves per tile height), the next kFixupGrid (main
// items) the K-split leftover tiles.
template <int MODE>
__global__ __launch_bounds__(kThreads) void fixup_kernel(int G, int ntiles_n, int H, int F, int P,
                                                         const int32_t* __restrict__ sched,
                                                         const int32_t* __restrict__ vrow,
                                                         const float* __restrict__ part,
                                                         const float* __restrict__ part32,
                                                         const float* __restrict__ part64,
                                                         uint16_t* __restrict__ out,
                                                         uint16_t* __restrict__ gu_out)
{
    const Split sp = gemm_split(G, ntiles_n, P, sched);
    // the skinny items first, so that they are not dispatched behind the
    // main items' (mostly idle) workgroups (measured: decode T = 256 at
    // maxvio 15, -3.5 us over its two fixups)
    const int nsk = 2 * P * kSkFixupHalves;
    const int mbx = (int)blockIdx.x - nsk;  // main item, if >= 0
    if (mbx < 0) {
        const int b = (int)blockIdx.x, nb = sp.ps * kSkFixupHalves;
        if (b < nb)
            skinny_fixup<MODE, 32>(G, ntiles_n, H, F, sp.ps, b, sched, vrow, part32, out, gu_out);
        else
            skinny_fixup<MODE, 64>(G, ntiles_n, H, F, sp.ps, b - nb, sched, vrow, part64, out,
                                   gu_out);
        return;
    }
    const int KT_all = (MODE == kGateUp ? H : F) / kTK;
    const Balance bal = balance_of(sched[G] * ntiles_n, sp.pm, KT_all);
    const int lt = mbx / kFixupSlabs;
    if (bal.S == 1 || lt >= bal.L) return;
    const TileRef r = tile_of_wg<MODE>(bal.full + lt, G, ntiles_n, [&](int i) { return sched[i]; });
    constexpr int kQuads = MODE == kGateUp ? kTN / 2 / 4 : kTN / 4;  // 4-column groups per row
    constexpr int kRowsPerPass = kThreads / kQuads;
    const int c = (threadIdx.x % kQuads) * 4;
    const int row0 = (int)(mbx % kFixupSlabs) * kFixupRows;
    const int row_end = min(r.rows, row0 + kFixupRows);
    for (int row = row0 + threadIdx.x / kQuads; row < row_end;
         row += kRowsPerPass) {
        if (MODE == kGateUp) {
            if (r.n0 + c >= F) continue;
            float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
#pragma unroll 4
            for (int p = 0; p < bal.S; ++p) {
                const float* src = part + ((size_t)(p * bal.L + lt) * kTM + row) * kTN + c;
                const float4 a = *reinterpret_cast<const float4*>(src);
                const float4 b = *reinterpret_cast<const float4*>(src + kTN / 2);
                g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
                u.x += b.x; u.y += b.y; u.z += b.z; u.w += b.w;
            }
            uint2 pk;
            pk.x = moe::pack_bf16x2(fast_silu(g.x) * u.x, fast_silu(g.y) * u.y);
            pk.y = moe::pack_bf16x2(fast_silu(g.z) * u.z, fast_silu(g.w) * u.w);
            *reinterpret_cast<uint2*>(out + (size_t)(r.hrow0 + row) * F + r.n0 + c) = pk;
            if (gu_out) {
                uint16_t* d = gu_out + (size_t)(r.hrow0 + row) * 2 * F + r.n0 + c;
                pk.x = moe::pack_bf16x2(g.x, g.y);
                pk.y = moe::pack_bf16x2(g.z, g.w);
                *reinterpret_cast<uint2*>(d) = pk;
                pk.x = moe::pack_bf16x2(u.x, u.y);
                pk.y = moe::pack_bf16x2(u.z, u.w);
                *reinterpret_cast<uint2*>(d + F) = pk;
            }
        } else {
            if (r.n0 + c >= H) continue;
            float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
            for (int p = 0; p < bal.S; ++p) {
                const float4 a = *reinterpret_cast<const float4*>(
                    part + ((size_t)(p * bal.L + lt) * kTM + row) * kTN + c);
                y.x += a.x; y.y += a.y; y.z += a.z; y.w += a.w;
            }
            uint2 pk;
            pk.x = moe::pack_bf16x2(y.x, y.y);
            pk.y = moe::pack_bf16x2(y.z, y.w);
            *reinterpret_cast<uint2*>(out + (size_t)vrow[r.hrow0 + row] * H + r.n0 + c) = pk;
        }
    }
}

// ---------------------------------------------------------------- fp32 ----
// Plain LDS-tiled VALU kernels for the fp32 dtype (small shapes): 32-row x
// 32-column tiles, K in chunks of 32, each thread 2 x 2 outputs.
constexpr int kFM = 32;

// Buffer row of row v of group g (by expert: through its pieces; by segment:
// the segment's first row + v).
__device__ __forceinline__ int group_buf_row(int g, int v, int R, bool seg, const int32_t* plan,
                                             const moe::PlanLayout& L)
{
    return seg ? plan[L.seg_row + g] + v : buf_row_of(g, v, R, plan, L);
}

__global__ __launch_bounds__(kThreads) void gateup_f32_kernel(
    int G, int E, int R, int seg, int H, int F, int mtiles, const float* __restrict__ a,
    const int32_t* __restrict__ plan, const int32_t* __restrict__ sched,
    const float* __restrict__ wg_all, const float* __restrict__ wu_all,
    const uint64_t* __restrict__ wtab, float* __restrict__ h)
{
    __shared__ float As[kFM][33], Gs[kFM][33], Us[kFM][33];
    __shared__ int32_t rowmap[kFM];
    const int mt = blockIdx.x % mtiles;
    const int nt = blockIdx.x / mtiles;
    const Tile tile = find_tile(mt, G, kFM, sched);
    if (tile.rows <= 0) return;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int tid = threadIdx.x;
    if (tid < kFM)
        rowmap[tid] = group_buf_row(tile.e, tile.v0 + (tid < tile.rows ? tid : 0), R, seg != 0, plan, L);
    const float* wg = group_w(wtab, wg_all, tile.e, 0, F, H);
    const float* wu = group_w(wtab, wu_all, tile.e, 1, F, H);
    __syncthreads();
    const int n0 = nt * kFM;
    const int ty = tid / 16, tx = tid % 16;
    float g[2][2] = {}, u[2][2] = {};
    for (int k0 = 0; k0 < H; k0 += 32) {
        for (int i = tid; i < kFM * 32; i += kThreads) {
            const int r = i / 32, c = i % 32;
            const int kc = k0 + c;
            const bool kin = kc < H;
            As[r][c] = kin ? a[(size_t)rowmap[r] * H + kc] : 0.f;
            const int f = min(n0 + r, F - 1);
            Gs[r][c] = kin ? wg[(size_t)f * H + kc] : 0.f;
            Us[r][c] = kin ? wu[(size_t)f * H + kc] : 0.f;
        }
        __syncthreads();
        for (int c = 0; c < 32; ++c)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    g[i][j] = fmaf(As[ty * 2 + i][c], Gs[tx * 2 + j][c], g[i][j]);
                    u[i][j] = fmaf(As[ty * 2 + i][c], Us[tx * 2 + j][c], u[i][j]);
                }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = ty * 2 + i, col = n0 + tx * 2 + j;
            if (row < tile.rows && col < F)
                h[(size_t)(tile.hrow0 + row) * F + col] = moe::silu(g[i][j]) * u[i][j];
        }
}

__global__ __launch_bounds__(kThreads) void down_f32_kernel(
    int G, int E, int R, int seg, int H, int F, int mtiles, const float* __restrict__ h,
    const int32_t* __restrict__ plan, const int32_t* __restrict__ sched,
    const float* __restrict__ wd_all, const uint64_t* __restrict__ wtab, float* __restrict__ y)
{
    __shared__ float As[kFM][33], Bs[kFM][33];
    __shared__ int32_t rowmap[kFM];
    const int mt = blockIdx.x % mtiles;
    const int nt = blockIdx.x / mtiles;
    const Tile tile = find_tile(mt, G, kFM, sched);
    if (tile.rows <= 0) return;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int tid = threadIdx.x;
    if (tid < kFM)
        rowmap[tid] = tid < tile.rows ? group_buf_row(tile.e, tile.v0 + tid, R, seg != 0, plan, L) : -1;
    const float* wd = group_w(wtab, wd_all, tile.e, 2, F, H);
    __syncthreads();
    const int n0 = nt * kFM;
    const int ty = tid / 16, tx = tid % 16;
    float acc[2][2] = {};
    for (int k0 = 0; k0 < F; k0 += 32) {
        for (int i = tid; i < kFM * 32; i += kThreads) {
            const int r = i / 32, c = i % 32;
            const int kc = k0 + c;
            const bool kin = kc < F;
            const int ar = r < tile.rows ? r : 0;
            As[r][c] = kin ? h[(size_t)(tile.hrow0 + ar) * F + kc] : 0.f;
            const int o = min(n0 + r, H - 1);
            Bs[r][c] = kin ? wd[(size_t)o * F + kc] : 0.f;
        }
        __syncthreads();
        for (int c = 0; c < 32; ++c)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = fmaf(As[ty * 2 + i][c], Bs[tx * 2 + j][c], acc[i][j]);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = ty * 2 + i, col = n0 + tx * 2 + j;
            if (row < tile.rows && col < H) y[(size_t)rowmap[row] * H + col] = acc[i][j];
        }
}

// Workgroups of the persistent bf16 kernels: one per CU, a multiple of 8 so
// that every XCD gets the same number, at most kGemmMaxGrid (the partial-tile
// workspace is sized for that many).
int persistent_grid()
{
    static int grid = 0;
    if (grid == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = moe::kGemmMaxGrid;
        grid = cus >= 8 ? (cus / 8) * 8 : 8;
        if (grid > moe::kGemmMaxGrid) grid = moe::kGemmMaxGrid;
    }
    return grid;
}


int max_mtiles(const moe_shape_t& s, int bm, int G)
{
    const int64_t N = (int64_t)s.T * s.k;
    return (int)((N + bm - 1) / bm + G);
}

}  // namespace

hipError_t moe_launch_gemm_schedule(const moe_shape_t& s, const int32_t* plan, char* ws,
                                    hipStream_t st, const moe::GemmGroups& g)
{
    const moe::WsLayout W = moe::ws_layout(s);
    int32_t* sched = reinterpret_cast<int32_t*>(ws + W.sched);
    const bool bf = s.dtype == MOE_BF16;
    const int N = s.T * s.k;
    int32_t* vrow = bf && N > 0 ? reinterpret_cast<int32_t*>(ws + W.vrow) : nullptr;
    const int grid = vrow ? (N + kThreads - 1) / kThreads : 1;
    schedule_kernel<<<grid, kThreads, 0, st>>>(g.G, s.E, s.R, g.seg ? 1 : 0, bf ? kTM : kFM,
                                               bf ? 32 : 0, bf ? 64 : 0, N, plan, sched, vrow);
    return hipGetLastError();
}

hipError_t moe_launch_gemm_schedule_bm(const moe_shape_t& s, const int32_t* plan, int32_t* sched,
                                       int32_t* vrow, hipStream_t st)
{
    const int N = s.T * s.k;
    const int grid = N > 0 ? (N + kThreads - 1) / kThreads : 1;
    schedule_kernel<<<grid, kThreads, 0, st>>>(s.E, s.E, s.R, 0, kTM, 0, 0, N, plan, sched,
                                               N > 0 ? vrow : nullptr);
    return hipGetLastError();
}

hipError_t moe_launch_gemm_gateup(const moe_shape_t& s, const void* a, const int32_t* plan,
                                  const void* w_gate, const void* w_up, char* ws,
                                  hipStream_t st, const moe::GemmGroups& g, void* gu_out_v)
{
    uint16_t* gu_out = static_cast<uint16_t*>(gu_out_v);
    if (s.T == 0) return hipSuccess;
    const moe::WsLayout W = moe::ws_layout(s);
    const int32_t* sched = reinterpret_cast<const int32_t*>(ws + W.sched);
    if (s.dtype == MOE_BF16) {
        const int ntn = (s.F + kTN / 2 - 1) / (kTN / 2);
        const int P = persistent_grid();
        const int32_t* vrow = reinterpret_cast<const int32_t*>(ws + W.vrow);
        float* part = reinterpret_cast<float*>(ws + W.part);
        uint16_t* h = reinterpret_cast<uint16_t*>(ws + W.h);
        const uint16_t* av = static_cast<const uint16_t*>(a);
        const uint16_t* wg = static_cast<const uint16_t*>(w_gate);
        const uint16_t* wu = static_cast<const uint16_t*>(w_up);
        float* sk32 = reinterpret_cast<float*>(ws + W.skpart);
        float* sk64 = sk32 + (size_t)2 * moe::kGemmMaxGrid * 32 * kTN;
        gemm_bf16_kernel<kGateUp><<<P, kThreads, 0, st>>>(g.G, ntn, s.H, s.F, av, sched, vrow, wg,
                                                           wu, g.wtab, h, gu_out, part, sk32, sk64);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        fixup_kernel<kGateUp><<<kFixupGrid + 2 * P * kSkFixupHalves, kThreads, 0, st>>>(
            g.G, ntn, s.H, s.F, P, sched, vrow, part, sk32, sk64, h, gu_out);
    } else {
        const int mtiles = max_mtiles(s, kFM, g.G);
        const int nt = (s.F + kFM - 1) / kFM;
        gateup_f32_kernel<<<mtiles * nt, kThreads, 0, st>>>(
            g.G, s.E, s.R, g.seg ? 1 : 0, s.H, s.F, mtiles, static_cast<const float*>(a), plan,
            sched, static_cast<const float*>(w_gate), static_cast<const float*>(w_up), g.wtab,
            reinterpret_cast<float*>(ws + W.h));
    }
    return hipGetLastError();
}

hipError_t moe_launch_gemm_down(const moe_shape_t& s, const int32_t* plan, const void* w_down,
                                void* y, char* ws, hipStream_t st, const moe::GemmGroups& g)
{
    if (s.T == 0) return hipSuccess;
    const moe::WsLayout W = moe::ws_layout(s);
    const int32_t* sched = reinterpret_cast<const int32_t*>(ws + W.sched);
    if (s.dtype == MOE_BF16) {
        const int ntn = (s.H + kTN - 1) / kTN;
        const int P = persistent_grid();
        const int32_t* vrow = reinterpret_cast<const int32_t*>(ws + W.vrow);
        float* part = reinterpret_cast<float*>(ws + W.part);
        const uint16_t* hv = reinterpret_cast<const uint16_t*>(ws + W.h);
        const uint16_t* wd = static_cast<const uint16_t*>(w_down);
        uint16_t* yv = static_cast<uint16_t*>(y);
        float* sk32 = reinterpret_cast<float*>(ws + W.skpart);
        float* sk64 = sk32 + (size_t)2 * moe::kGemmMaxGrid * 32 * kTN;
        gemm_bf16_kernel<kDown><<<P, kThreads, 0, st>>>(g.G, ntn, s.H, s.F, hv, sched, vrow, wd,
                                                         nullptr, g.wtab, yv, nullptr, part, sk32, sk64);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        fixup_kernel<kDown><<<kFixupGrid + 2 * P * kSkFixupHalves, kThreads, 0, st>>>(
            g.G, ntn, s.H, s.F, P, sched, vrow, part, sk32, sk64, yv, nullptr);
    } else {
        const int mtiles = max_mtiles(s, kFM, g.G);
        const int nt = (s.H + kFM - 1) / kFM;
        down_f32_kernel<<<mtiles * nt, kThreads, 0, st>>>(
            g.G, s.E, s.R, g.seg ? 1 : 0, s.H, s.F, mtiles, reinterpret_cast<const float*>(ws + W.h),
            plan, sched, static_cast<const float*>(w_down), g.wtab, static_cast<float*>(y));
    }
    return hipGetLastError();
}
