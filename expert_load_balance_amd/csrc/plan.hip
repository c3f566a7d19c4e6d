// plan.hip -- the equal-load replica plan, computed on the device from the
// demand vector (no host round trip).
//
// "Moonshot AI drops MoonEP ..." paragraph 3: every rank receives exactly the
// same number of tokens however skewed the routing, by planning a few
// redundant expert copies directly from the router output; paragraph 4:
// with as many prefetch slots as experts per rank, every expert a rank's
// GEMM touches is local.
//
// The pages fix the invariant, not the rule; the rule implemented here is:
//   quota C_r = floor(N/R) + [r < N mod R]; windows are the prefix of quotas.
//   While an unfilled rank is below quota: take the rank s with the largest
//   deficit (ties: lower rank) and the rank l with the largest excess (ties:
//   lower rank); move C_s - L_s assignments from l's home experts to s,
//   draining l's experts in (count desc, id asc) order; s is now filled.
//   What remains of each expert stays home.
// A receiving rank gets pieces from one donor only, so it holds at most n
// replica experts: with S = n slots everything is local.
//
// One workgroup of sixteen wavefronts (E <= 256, R <= 64). Threads sweep
// the experts for the counts and the donor orders. The transfer loop runs
// on the first wavefront, lane r owning rank r: its argmaxes are a DPP /
// permlane max, then the lowest lane holding it (by ballot); the donor walk
// is a prefix sum over the donor's remaining counts, kept in donor order,
// lane i taking its i-th (a serial walk on one lane past 64 experts a
// rank). The windows and the pieces are laid out by groups of lanes, one
// rank's 2n candidate segments or one expert's R candidate pieces a group,
// several groups a wavefront; ballots place the non-empty entries and a
// wavefront permute packs them to the front, so that every table is written
// with whole-wavefront stores. Every entry of the plan block is written.
#include <climits>

#include "common.h"
#include "count_fused.h"

namespace {

template <int CTRL>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int opaque(int v)
{
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}
// Two maxes over lanes 0 .. W-1 at once (W = 16, 32 or 64; W-lane groups
// reduce alike), without LDS: DPP moves inside rows of 16 lanes (xor 1,
// xor 2, then the half-row and row mirrors, which for a commutative op pair
// each lane with the other half of its reduced group), then, past 16 lanes,
// the gfx950 permlane swaps across rows of 16 and of 32; the steps of the
// two interleave, each hiding the other's latency. Each swap gets an
// opaque copy as its second operand (with the same value twice the
// compiler was seen to drop the second half of a swap).
template <int W>
__device__ __forceinline__ void wave_max2(int& a, int& b)
{
    a = max(a, dpp<0xB1>(a));
    b = max(b, dpp<0xB1>(b));
    a = max(a, dpp<0x4E>(a));
    b = max(b, dpp<0x4E>(b));
    a = max(a, dpp<0x141>(a));
    b = max(b, dpp<0x141>(b));
    a = max(a, dpp<0x140>(a));
    b = max(b, dpp<0x140>(b));
    if constexpr (W > 16) {
        const auto a1 = __builtin_amdgcn_permlane16_swap(a, opaque(a), false, false);
        const auto b1 = __builtin_amdgcn_permlane16_swap(b, opaque(b), false, false);
        a = max((int)a1[0], (int)a1[1]);
        b = max((int)b1[0], (int)b1[1]);
    }
    if constexpr (W > 32) {
        const auto a2 = __builtin_amdgcn_permlane32_swap(a, opaque(a), false, false);
        const auto b2 = __builtin_amdgcn_permlane32_swap(b, opaque(b), false, false);
        a = max((int)a2[0], (int)a2[1]);
        b = max((int)b2[0], (int)b2[1]);
    }
}

// Lanes below this one, as a ballot mask.
__device__ __forceinline__ uint64_t lanes_below(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Bits [g * w, g * w + w) of a ballot (w <= 64).
__device__ __forceinline__ uint64_t group_bits(int g, int w)
{
    return (w == 64 ? ~0ull : ((1ull << w) - 1)) << (g * w);
}

// Forward permute inside the wavefront: the value of every lane lands in
// lane `to` (a permutation of the lanes).
__device__ __forceinline__ int send_to(int to, int v) { return __builtin_amdgcn_ds_permute(to * 4, v); }

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}


// The transfer loop, on one wavefront, lane r holding rank r's quota and
// load: at most R - 1 fills (the LDS writes of a wavefront reach its own
// later reads in order, so no barrier inside). A fill takes s, the unfilled
// rank of largest deficit d, and l, the rank of largest excess (ties to the
// lower rank both; d <= 0 ends the loop), moves d assignments from l's home
// experts in donor order to s and marks s filled. The next fill's choice
// depends only on the loads, so it is made while this fill's walk reads
// l's remaining counts. W: lanes the argmaxes span (R <= W). SCAN: the
// walk over l's n experts as a prefix sum, by DPP shifts inside the first
// row (16: n <= 16) or by shuffles (64: n <= 64), the i-th expert giving
// min(rem_i, d - (rem of the ones before it)), at least 0; 0: one lane
// walks them in turn (n > 64). donor[r] ends as r's donor, -1 if none.
constexpr int kZeroEntry = 256;  // E <= 256

template <int W, int SCAN>
__device__ __forceinline__ void transfer_loop(int R, int n, int lane, int my_q, int my_load,
                                              int2* ro, int32_t* take, int32_t* ptr,
                                              int32_t* donor)
{
    bool my_filled = false;
    int my_donor = -1;
    // argmaxes: the max over the lanes (lane 0's copy, a scalar), then the
    // lowest lane holding it
    auto pick = [&](int& d, int& s, int& l) {
        int def = -1, exc = INT_MIN;
        if (lane < R) {
            const int dd = my_q - my_load;
            def = (!my_filled && dd > 0) ? dd : -1;
            exc = -dd;
        }
        int bd = def, be = exc;
        wave_max2<W>(bd, be);
        d = __builtin_amdgcn_readfirstlane(bd);
        be = __builtin_amdgcn_readfirstlane(be);
        s = __ffsll((unsigned long long)__ballot(lane < R && def == d)) - 1;
        l = __ffsll((unsigned long long)__ballot(lane < R && exc == be)) - 1;
    };
    int d, s, l;
    pick(d, s, l);
    for (int it = 0; it < R && d > 0; ++it) {
        if (lane == l) my_load -= d;
        if (lane == s) {
            my_load = my_q;
            my_filled = true;
            my_donor = l;
        }
        if constexpr (SCAN == 0) {
            if (lane == 0) {
                int left = d;
                int p = ptr[l];
                while (left > 0 && p < n) {
                    const int e = ro[l * n + p].y;
                    const int r = ro[l * n + p].x;
                    const int t = r < left ? r : left;
                    if (t > 0) {
                        take[s * n + (e - l * n)] = t;
                        ro[l * n + p].x = r - t;
                        left -= t;
                    }
                    if (r - t == 0) ++p;
                }
                ptr[l] = p;
            }
            pick(d, s, l);
        } else {
            // lanes past n read the zero entry (they take nothing); the
            // next choice is made while the read is in flight (kept apart
            // from the walk's arithmetic by a scheduling barrier)
            const int2 v = ro[lane < n ? l * n + lane : kZeroEntry];
            int d2, s2, l2;
            pick(d2, s2, l2);
            __builtin_amdgcn_sched_barrier(0);
            const int r = v.x, e = v.y;
            int incl = r;
            if constexpr (SCAN == 16) {
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);
            } else {
                for (int off = 1; off < n; off <<= 1) {  // n is uniform
                    const int v = __shfl_up(incl, off, 64);
                    if (lane >= off) incl += v;
                }
            }
            const int room = d - (incl - r);
            const int t = room <= 0 ? 0 : (room < r ? room : r);
            if (t > 0) {
                take[s * n + (e - l * n)] = t;
                ro[l * n + lane].x = r - t;
            }
            d = d2;
            s = s2;
            l = l2;
        }
    }
    if (lane < R) donor[lane] = my_donor;
}

constexpr int kPlanThreads = 1024;

// The plan from the counts (global memory, or the fused count's LDS copy).
// Every thread of the workgroup calls it.
__device__ __forceinline__ void plan_body(int E, int R, const int32_t* __restrict__ counts,
                                          int32_t* __restrict__ plan)
{
    __shared__ int32_t cnt[256], rem[256], take[256], home_row[256], rep_row[256];
    // the experts in donor order inside every home block, with what remains
    // of each (the transfer loop's view): (remaining count, expert id); one
    // more entry of zeros
    __shared__ int2 ro[kZeroEntry + 1];
    __shared__ int32_t quota[64], load[64], donor[64], ptr[64], win[65];
    __shared__ int32_t wsum[kPlanThreads / 64];

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int n = E / R;
    const moe::PlanLayout L = moe::plan_layout(E, R);

    int part = 0;
    for (int e = tid; e < E; e += kPlanThreads) {
        const int c = counts[e];
        cnt[e] = c;
        rem[e] = c;
        take[e] = 0;
        part += c;
    }
    part = wave_sum(part);
    if (lane == 0) wsum[wave] = part;
    __syncthreads();
    int N = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / 64; ++w) N += wsum[w];

    // quotas, home loads, windows (first wavefront)
    const int q = N / R, extra = N % R;
    int my_quota = 0;
    if (wave == 0 && lane < R) {
        my_quota = q + (lane < extra ? 1 : 0);
        int s = 0;
        for (int e = lane * n; e < (lane + 1) * n; ++e) s += cnt[e];
        quota[lane] = my_quota;
        load[lane] = s;
        donor[lane] = -1;
        ptr[lane] = 0;
    }
    int incl = my_quota;  // inclusive scan of quotas over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (wave == 0 && lane < R) win[lane + 1] = incl;
    if (tid == 0) {
        win[0] = 0;
        ro[kZeroEntry] = make_int2(0, 0);
    }

    // donor order inside every rank's home block: (count desc, id asc)
    if (R > 1) {
        for (int e = tid; e < E; e += kPlanThreads) {
            const int r0 = (e / n) * n;
            int pos = 0;
            for (int x = r0; x < r0 + n; ++x)
                pos += (cnt[x] > cnt[e] || (cnt[x] == cnt[e] && x < e)) ? 1 : 0;
            ro[r0 + pos] = make_int2(cnt[e], e);
        }
    }
    __syncthreads();

    // transfer loop (E <= 256 and R | E: past 16 ranks a rank has at most 15
    // experts, past 32 at most 7)
    if (wave == 0) {
        const int my_q = lane < R ? quota[lane] : 0;
        const int my_load = lane < R ? load[lane] : 0;
        if (R > 32)
            transfer_loop<64, 16>(R, n, lane, my_q, my_load, ro, take, ptr, donor);
        else if (R > 16)
            transfer_loop<32, 16>(R, n, lane, my_q, my_load, ro, take, ptr, donor);
        else if (n <= 16)
            transfer_loop<16, 16>(R, n, lane, my_q, my_load, ro, take, ptr, donor);
        else if (n <= 64)
            transfer_loop<16, 64>(R, n, lane, my_q, my_load, ro, take, ptr, donor);
        else
            transfer_loop<16, 0>(R, n, lane, my_q, my_load, ro, take, ptr, donor);
    }
    __syncthreads();
    // back to expert order for the layout below
    if (R > 1)
        for (int i = tid; i < E; i += kPlanThreads) rem[ro[i].y] = ro[i].x;
    __syncthreads();

    // Per-rank windows: segments in expert id order (the lower id block
    // first), replica slots. Rank r's 2n candidate segments (pass 0: its
    // first block, pass 1: the other) sit in 2n consecutive lanes; ballots
    // place the non-empty ones, a prefix sum gives their rows, and a
    // wavefront permute packs them to the front so that every table is
    // written by one coalesced store (the rest -1). More than 32 experts a
    // rank: one lane per rank.
    if (2 * n <= 64) {
        const int gs = 2 * n, gpw = 64 / gs;
        const int g = lane / gs, j = lane % gs;
        const int pass = j / n, i = j % n;
        for (int base = wave * gpw; base < R; base += (kPlanThreads / 64) * gpw) {
            const int r = base + g;
            const bool act = g < gpw && r < R;  // uniform over the group
            const int l = act ? donor[r] : -1;
            int c = 0, e = -1, home = 0;
            if (act) {
                int blk;
                if (l < 0) blk = pass == 0 ? r : -1;
                else blk = (pass == 0) == (l < r) ? l : r;
                if (blk >= 0) {
                    e = blk * n + i;
                    home = blk == r;
                    c = home ? rem[e] : take[r * n + i];
                }
            }
            const uint64_t gm = act ? group_bits(g, gs) : 0ull, below = lanes_below(lane);
            const uint64_t has = __ballot(act && c > 0), rep = __ballot(act && c > 0 && !home);
            const int pos = __popcll(has & gm & below), ns = __popcll(has & gm);
            const int spos = __popcll(rep & gm & below), nslot = __popcll(rep & gm);
            int incl = c;  // prefix sum of the counts inside the group
            for (int off = 1; off < gs; off <<= 1) {
                const int v = __shfl_up(incl, off, 64);
                if (j >= off) incl += v;
            }
            const int row = act ? win[r] + incl - c : 0;
            if (act && c > 0) {
                if (home) home_row[e] = row;
                else rep_row[r * n + i] = row;
            }
            // segment k of rank r comes from the k-th non-empty lane; the
            // empty ones follow in order (a permutation of the group)
            const int to = act ? g * gs + (c > 0 ? pos : ns + (j - pos)) : lane;
            const int se = send_to(to, e), sr = send_to(to, row), scn = send_to(to, c);
            if (act) {
                const int64_t o = (int64_t)r * gs + j;  // j is now the segment index
                plan[L.seg_expert + o] = j < ns ? se : -1;
                plan[L.seg_row + o] = j < ns ? sr : -1;
                plan[L.seg_cnt + o] = j < ns ? scn : -1;
            }
            const int sto = act ? g * gs + (c > 0 && !home ? spos : nslot + (j - spos)) : lane;
            const int sl = send_to(sto, e);
            if (act && j < n) plan[L.slot_expert + (int64_t)r * n + j] = j < nslot ? sl : -1;
            if (act && j == 0) {
                plan[L.seg_num + r] = ns;
                plan[L.slots_needed + r] = nslot;
                plan[L.quota + r] = quota[r];
                plan[L.donor + r] = l;
                plan[L.win_off + r + 1] = win[r + 1];
                if (r == 0) plan[L.win_off] = 0;
            }
        }
    } else if (wave == 0 && lane < R) {
        const int r = lane;
        const int l = donor[r];
        int row = win[r];
        int ns = 0, nslot = 0;
        int32_t* seg_e = plan + L.seg_expert + (size_t)r * 2 * n;
        int32_t* seg_r = plan + L.seg_row + (size_t)r * 2 * n;
        int32_t* seg_c = plan + L.seg_cnt + (size_t)r * 2 * n;
        int32_t* slot = plan + L.slot_expert + (size_t)r * n;
        for (int pass = 0; pass < 2; ++pass) {
            // lower id block first
            int blk;
            if (l < 0) blk = pass == 0 ? r : -1;
            else blk = (pass == 0) == (l < r) ? l : r;
            if (blk < 0) continue;
            for (int i = 0; i < n; ++i) {
                const int e = blk * n + i;
                const int c = (blk == r) ? rem[e] : take[r * n + i];
                if (c <= 0) continue;
                seg_e[ns] = e;
                seg_r[ns] = row;
                seg_c[ns] = c;
                if (blk == r) home_row[e] = row;
                else {
                    rep_row[r * n + i] = row;
                    slot[nslot++] = e;
                }
                row += c;
                ++ns;
            }
        }
        for (int i = ns; i < 2 * n; ++i) seg_e[i] = seg_r[i] = seg_c[i] = -1;
        for (int i = nslot; i < n; ++i) slot[i] = -1;
        plan[L.seg_num + r] = ns;
        plan[L.slots_needed + r] = nslot;
        plan[L.quota + r] = quota[r];
        plan[L.donor + r] = l;
        plan[L.win_off + r + 1] = win[r + 1];
        if (r == 0) plan[L.win_off] = 0;
    }
    __syncthreads();

    // Per-expert pieces in rank order: an expert's R candidate pieces (rank
    // r: its home remainder when r is its home rank, what r took from it
    // when r is a receiver of its home rank) sit in R consecutive lanes, 64 / R
    // experts a wavefront; packed to the front by a permute as above.
    {
        const int gpw = 64 / R;
        const int g = lane / R, r = lane % R;
        for (int base = wave * gpw; base < E; base += (kPlanThreads / 64) * gpw) {
            const int e = base + g;
            const bool act = g < gpw && e < E;  // uniform over the group
            int c = 0, row = -1;
            if (act) {
                const int h = e / n;
                if (r == h) {
                    c = rem[e];
                    row = home_row[e];
                } else if (donor[r] == h) {
                    c = take[r * n + (e - h * n)];
                    row = rep_row[r * n + (e - h * n)];
                }
            }
            const uint64_t gm = act ? group_bits(g, R) : 0ull;
            const uint64_t has = __ballot(act && c > 0);
            const int pos = __popcll(has & gm & lanes_below(lane)), np = __popcll(has & gm);
            const int to = act ? g * R + (c > 0 ? pos : np + (r - pos)) : lane;
            const int sk = send_to(to, r), sw = send_to(to, row), sc = send_to(to, c);
            if (act) {
                const int64_t o = (int64_t)e * R + r;  // r is now the piece index
                plan[L.piece_rank + o] = r < np ? sk : -1;
                plan[L.piece_row + o] = r < np ? sw : -1;
                plan[L.piece_cnt + o] = r < np ? sc : -1;
                if (r == 0) plan[L.piece_num + e] = np;
            }
        }
    }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(int E, int R, const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ plan)
{
    plan_body(E, R, counts, plan);
}

// Count and plan in one launch (up to 16384 assignments, where the count is
// one workgroup of the same size): the plan reads the counts from the
// count's LDS copy. Results are those of the two launches, bit for bit.
static_assert(kPlanThreads == moe::cnt::kFusedThreads, "one workgroup runs both");
__global__ __launch_bounds__(kPlanThreads) void count_plan_kernel(
    int N, int k, int E, int R, const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ eidx, int32_t* __restrict__ rank_load,
    int32_t* err, int32_t* __restrict__ plan)
{
    __shared__ int32_t hist[256];
    moe::cnt::count_fused_body(N, k, E, R, ids, counts, offsets, eidx, rank_load, err, hist);
    __syncthreads();
    plan_body(E, R, hist, plan);
}

}  // namespace

hipError_t moe_launch_plan(const moe_shape_t& s, const int32_t* counts, int32_t* plan,
                           hipStream_t st)
{
    plan_kernel<<<1, kPlanThreads, 0, st>>>(s.E, s.R, counts, plan);
    return hipGetLastError();
}

hipError_t moe_launch_count_plan(const moe_shape_t& s, const int32_t* ids, int32_t* counts,
                                 int32_t* offsets, int32_t* eidx, int32_t* rank_load,
                                 int32_t* err, char* ws, int32_t* plan, hipStream_t st)
{
    const int64_t N = (int64_t)s.T * s.k;
    if (N > moe::cnt::kFusedMax) {
        const hipError_t e = moe_launch_count(s, ids, counts, offsets, eidx, rank_load, err, ws, st);
        if (e != hipSuccess) return e;
        return moe_launch_plan(s, counts, plan, st);
    }
    count_plan_kernel<<<1, kPlanThreads, 0, st>>>((int)N, s.k, s.E, s.R, ids, counts, offsets,
                                                   eidx, rank_load, err, plan);
    return hipGetLastError();
}
