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
// One wavefront does it all (E <= 256, R <= 64): lane r owns rank r in the
// transfer loop, whose two argmaxes are xor-shuffle reductions of a packed
// (value, rank) key; the donor walk is a few serial steps on lane 0; then
// lane r lays out rank r's window and lanes sweep experts to build the piece
// tables. Every entry of the plan block is written.
#include "common.h"

namespace {

__device__ __forceinline__ long long wave_max_ll(long long v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const long long o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// key orders by value, then by lower rank
__device__ __forceinline__ long long argmax_key(int value, int r)
{
    return ((long long)value << 8) | (long long)(255 - r);
}

__global__ __launch_bounds__(64) void plan_kernel(int E, int R, const int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ plan)
{
    __shared__ int32_t cnt[256], rem[256], order[256], take[256], home_row[256], rep_row[256];
    __shared__ int32_t quota[64], load[64], filled[64], donor[64], ptr[64], win[65];

    const int lane = threadIdx.x;
    const int n = E / R;
    const moe::PlanLayout L = moe::plan_layout(E, R);

    int part = 0;
    for (int e = lane; e < E; e += 64) {
        const int c = counts[e];
        cnt[e] = c;
        rem[e] = c;
        take[e] = 0;
        part += c;
    }
    const int N = wave_sum(part);
    __syncthreads();

    // quotas, home loads, windows
    const int q = N / R, extra = N % R;
    int my_quota = 0;
    if (lane < R) {
        my_quota = q + (lane < extra ? 1 : 0);
        int s = 0;
        for (int e = lane * n; e < (lane + 1) * n; ++e) s += cnt[e];
        quota[lane] = my_quota;
        load[lane] = s;
        filled[lane] = 0;
        donor[lane] = -1;
        ptr[lane] = 0;
    }
    int incl = my_quota;  // inclusive scan of quotas over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane < R) win[lane + 1] = incl;
    if (lane == 0) win[0] = 0;

    // donor order inside every rank's home block: (count desc, id asc)
    if (R > 1) {
        for (int e = lane; e < E; e += 64) {
            const int r0 = (e / n) * n;
            int pos = 0;
            for (int x = r0; x < r0 + n; ++x)
                pos += (cnt[x] > cnt[e] || (cnt[x] == cnt[e] && x < e)) ? 1 : 0;
            order[r0 + pos] = e;
        }
    }
    __syncthreads();

    // transfer loop: at most R - 1 fills
    for (int it = 0; it < R; ++it) {
        int def = -1, exc = -1;
        if (lane < R) {
            const int d = quota[lane] - load[lane];
            def = (!filled[lane] && d > 0) ? d : -1;
            exc = -d;
        }
        const long long ks = wave_max_ll(lane < R ? argmax_key(def, lane) : argmax_key(-1, 255));
        const int best_def = (int)(ks >> 8);
        if (best_def <= 0) break;  // uniform
        const int s = 255 - (int)(ks & 255);
        const long long kl = wave_max_ll(lane < R ? argmax_key(exc, lane) : argmax_key(-1, 255));
        const int l = 255 - (int)(kl & 255);
        if (lane == 0) {
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
            donor[s] = l;
            load[l] -= best_def;
            load[s] = quota[s];
            filled[s] = 1;
        }
        __syncthreads();
    }

    // per-rank windows: segments in expert id order, replica slots
    if (lane < R) {
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

    // per-expert pieces in rank order
    for (int e = lane; e < E; e += 64) {
        const int h = e / n;
        int np = 0;
        int32_t* pr = plan + L.piece_rank + (size_t)e * R;
        int32_t* pw = plan + L.piece_row + (size_t)e * R;
        int32_t* pc = plan + L.piece_cnt + (size_t)e * R;
        for (int r = 0; r < R; ++r) {
            int c = 0, row = -1;
            if (r == h) {
                c = rem[e];
                row = home_row[e];
            } else if (donor[r] == h) {
                c = take[r * n + (e - h * n)];
                row = rep_row[r * n + (e - h * n)];
            }
            if (c > 0) {
                pr[np] = r;
                pw[np] = row;
                pc[np] = c;
                ++np;
            }
        }
        for (int i = np; i < R; ++i) pr[i] = pw[i] = pc[i] = -1;
        plan[L.piece_num + e] = np;
    }
}

}  // namespace

hipError_t moe_launch_plan(const moe_shape_t& s, const int32_t* counts, int32_t* plan,
                           hipStream_t st)
{
    plan_kernel<<<1, 64, 0, st>>>(s.E, s.R, counts, plan);
    return hipGetLastError();
}
