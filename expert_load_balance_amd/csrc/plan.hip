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
// is a prefix sum over the donor's experts, lane i taking its i-th in donor
// order (a serial walk on one lane past 64 experts a rank). Lane r of the
// first wavefront lays out rank r's window; then the wavefronts take
// experts in turn, lane r the piece on rank r, compacted in rank order with
// a ballot. Every entry of the plan block is written.
#include <climits>

#include "common.h"

namespace {

// Wavefront max without LDS: DPP moves inside rows of 16 lanes (xor 1,
// xor 2, then the half-row and row mirrors, which for a commutative op pair
// each lane with the other half of its reduced group), then the gfx950
// permlane swaps across rows of 16 and of 32. Each swap gets an opaque copy
// as its second operand (with the same value twice the compiler was seen to
// drop the second half of a swap).
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
__device__ __forceinline__ int wave_max(int v)
{
    v = max(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max(v, dpp<0x141>(v));  // lane i <-> 7-i in each 8
    v = max(v, dpp<0x140>(v));  // lane i <-> 15-i in each 16
    const auto a = __builtin_amdgcn_permlane16_swap(v, opaque(v), false, false);
    v = max((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, opaque(v), false, false);
    return max((int)b[0], (int)b[1]);
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}


constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(int E, int R, const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ plan)
{
    __shared__ int32_t cnt[256], rem[256], order[256], take[256], home_row[256], rep_row[256];
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
    if (tid == 0) win[0] = 0;

    // donor order inside every rank's home block: (count desc, id asc)
    if (R > 1) {
        for (int e = tid; e < E; e += kPlanThreads) {
            const int r0 = (e / n) * n;
            int pos = 0;
            for (int x = r0; x < r0 + n; ++x)
                pos += (cnt[x] > cnt[e] || (cnt[x] == cnt[e] && x < e)) ? 1 : 0;
            order[r0 + pos] = e;
        }
    }
    __syncthreads();

    // transfer loop: at most R - 1 fills, on the first wavefront alone (its
    // LDS writes reach its own later reads in order, so no barrier inside)
    if (wave == 0) {
        // lane r's rank: quota, load and whether it has been filled
        const int my_q = lane < R ? quota[lane] : 0;
        int my_load = lane < R ? load[lane] : 0;
        bool my_filled = false;
        for (int it = 0; it < R; ++it) {
            int def = -1, exc = -1;
            if (lane < R) {
                const int d = my_q - my_load;
                def = (!my_filled && d > 0) ? d : -1;
                exc = -d;
            }
            // argmaxes, ties to the lower rank: the wavefront max, then the
            // lowest lane holding it
            const int best_def = wave_max(lane < R ? def : -1);
            if (best_def <= 0) break;  // uniform
            const int s = __ffsll((unsigned long long)__ballot(lane < R && def == best_def)) - 1;
            const int best_exc = wave_max(lane < R ? exc : INT_MIN);
            const int l = __ffsll((unsigned long long)__ballot(lane < R && exc == best_exc)) - 1;
            if (n <= 64) {
                // the walk over l's experts in donor order as a prefix sum: the
                // i-th takes min(rem_i, d - (rem of the ones before it)), at least 0
                const int e = lane < n ? order[l * n + lane] : 0;
                const int r = lane < n ? rem[e] : 0;
                int incl = r;
                if (n <= 16) {  // inside the first row of 16 lanes: DPP shifts
                    if (n > 1) incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);
                    if (n > 2) incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);
                    if (n > 4) incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);
                    if (n > 8) incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);
                } else {
                    for (int off = 1; off < n; off <<= 1) {  // n is uniform
                        const int v = __shfl_up(incl, off, 64);
                        if (lane >= off) incl += v;
                    }
                }
                const int room = best_def - (incl - r);
                const int t = room <= 0 ? 0 : (room < r ? room : r);
                if (t > 0) {
                    take[s * n + (e - l * n)] = t;
                    rem[e] = r - t;
                }
            } else if (lane == 0) {  // more than 64 experts a rank: one step at a time
                int d = best_def;
                int p = ptr[l];
                while (d > 0 && p < n) {
                    const int e = order[l * n + p];
                    const int t = rem[e] < d ? rem[e] : d;
                    if (t > 0) {
                        take[s * n + (e - l * n)] = t;
                        rem[e] -= t;
                        d -= t;
                    }
                    if (rem[e] == 0) ++p;
                }
                ptr[l] = p;
            }
            if (lane == l) my_load -= best_def;
            if (lane == s) {
                my_load = my_q;
                my_filled = true;
            }
            if (lane == 0) donor[s] = l;
        }
    }
    __syncthreads();

    // per-rank windows: segments in expert id order, replica slots
    if (wave == 0 && lane < R) {
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

    // per-expert pieces in rank order: lane r of the expert's wavefront
    // holds its piece on rank r (if any) and writes it at its rank among the
    // non-empty pieces; lanes from the piece count on fill with -1
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int e = wave; e < E; e += kPlanThreads / 64) {
        const int h = e / n;
        int c = 0, row = -1;
        if (lane < R) {
            if (lane == h) {
                c = rem[e];
                row = home_row[e];
            } else if (donor[lane] == h) {
                c = take[lane * n + (e - h * n)];
                row = rep_row[lane * n + (e - h * n)];
            }
        }
        const uint64_t has = __ballot(c > 0);
        const int np = __popcll(has);
        int32_t* pr = plan + L.piece_rank + (size_t)e * R;
        int32_t* pw = plan + L.piece_row + (size_t)e * R;
        int32_t* pc = plan + L.piece_cnt + (size_t)e * R;
        if (c > 0) {
            const int pos = __popcll(has & lt_mask);
            pr[pos] = lane;
            pw[pos] = row;
            pc[pos] = c;
        }
        if (lane < R && lane >= np) pr[lane] = pw[lane] = pc[lane] = -1;
        if (lane == 0) plan[L.piece_num + e] = np;
    }
}

}  // namespace

hipError_t moe_launch_plan(const moe_shape_t& s, const int32_t* counts, int32_t* plan,
                           hipStream_t st)
{
    plan_kernel<<<1, kPlanThreads, 0, st>>>(s.E, s.R, counts, plan);
    return hipGetLastError();
}
