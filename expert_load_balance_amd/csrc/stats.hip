// stats.hip -- device reductions behind moe_stats.
//
// "MoE Load Balancing: Find Expert Hotspots": expert demand and rank demand
// under a mapping ("Separate expert demand from rank placement"), the
// fixed-capacity ledger from raw demand ("Make expert capacity, overflow, and
// padding explicit"), remote routes where the token's origin rank differs from
// the destination rank ("Count remote routes before celebrating balance").
// "Moonshot AI drops MoonEP ..." paragraph 4: slots per rank (locality).
//
// One workgroup reduces everything into int64 slots; the host turns them into
// ratios. Off the timed path.
#include "common.h"

namespace {

constexpr int kThreads = 256;

__device__ long long block_sum(long long v, long long* red)
{
    red[threadIdx.x] = v;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    const long long r = red[0];
    __syncthreads();
    return r;
}

__device__ long long block_max(long long v, long long* red)
{
    red[threadIdx.x] = v;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + off]);
        __syncthreads();
    }
    const long long r = red[0];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void stats_kernel(
    int T, int k, int E, int R, int S, int cap, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ plan,
    const int32_t* __restrict__ dest_row, const int32_t* __restrict__ mapping,
    const int32_t* __restrict__ origin, const int32_t* __restrict__ err, long long* out)
{
    __shared__ long long red[kThreads];
    __shared__ int32_t win[65];
    const int tid = threadIdx.x;
    const int n = E / R;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int N = T * k;

    long long c = 0, proc = 0, over = 0, pad = 0, act = 0, mn = 0x7fffffffffffffffll;
    if (tid < E) {
        c = counts[tid];
        proc = c < cap ? c : cap;
        over = c > cap ? c - cap : 0;
        pad = cap > c ? cap - c : 0;
        act = c > 0;
        mn = c;
    }
    const long long total = block_sum(c, red);
    const long long mx = block_max(c, red);
    const long long mnv = -block_max(-mn, red);
    const long long sp = block_sum(proc, red), so = block_sum(over, red), spd = block_sum(pad, red);
    const long long sa = block_sum(act, red);

    if (tid <= R) win[tid] = plan[L.win_off + tid];
    __syncthreads();

    long long rh = 0, rm = 0, rp = 0;
    for (int a = tid; a < N; a += kThreads) {
        const int t = a / k;
        const int o = origin ? origin[t] : t % R;
        const int e = ids[a];
        if (e < 0 || e >= E) continue;
        rh += (e / n) != o;
        if (mapping) rm += mapping[e] != o;
        if (dest_row) {
            const int d = dest_row[a];
            int lo = 0, hi = R - 1;  // window holding row d
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (win[mid] <= d) lo = mid;
                else hi = mid - 1;
            }
            rp += lo != o;
        }
    }
    const long long srh = block_sum(rh, red), srm = block_sum(rm, red), srp = block_sum(rp, red);

    long long reps = 0, maxslots = 0, over_s = 0, nonlocal = 0;
    if (tid < R) {
        const int sn = plan[L.slots_needed + tid];
        reps = sn;
        maxslots = sn;
        over_s = sn > S;
        const int ns = plan[L.seg_num + tid];
        for (int i = S; i < sn && i < n; ++i) {
            const int e = plan[L.slot_expert + (size_t)tid * n + i];
            for (int q = 0; q < ns && q < 2 * n; ++q)
                if (plan[L.seg_expert + (size_t)tid * 2 * n + q] == e)
                    nonlocal += plan[L.seg_cnt + (size_t)tid * 2 * n + q];
        }
    }
    const long long sreps = block_sum(reps, red), smax = block_max(maxslots, red);
    const long long sover = block_sum(over_s, red), snl = block_sum(nonlocal, red);

    // rank load vectors: home, mapped, planned
    for (int r = tid; r < R; r += kThreads) {
        long long hsum = 0, msum = 0, psum = 0;
        for (int e = r * n; e < (r + 1) * n; ++e) hsum += counts[e];
        if (mapping)
            for (int e = 0; e < E; ++e) msum += mapping[e] == r ? counts[e] : 0;
        const int ns = plan[L.seg_num + r];
        for (int q = 0; q < ns && q < 2 * n; ++q) psum += plan[L.seg_cnt + (size_t)r * 2 * n + q];
        out[moe::kStScalars + r] = hsum;
        out[moe::kStScalars + R + r] = msum;
        out[moe::kStScalars + 2 * R + r] = psum;
    }
    if (tid == 0) {
        out[moe::kStN] = total;
        out[moe::kStMax] = mx;
        out[moe::kStMin] = E > 0 ? mnv : 0;
        out[moe::kStActive] = sa;
        out[moe::kStProcessed] = sp;
        out[moe::kStOverflow] = so;
        out[moe::kStPadding] = spd;
        out[moe::kStRemoteHome] = srh;
        out[moe::kStRemoteMapped] = srm;
        out[moe::kStRemotePlanned] = srp;
        out[moe::kStReplicas] = sreps;
        out[moe::kStMaxSlots] = smax;
        out[moe::kStOverSlots] = sover;
        out[moe::kStNonlocal] = snl;
        out[moe::kStErr] = err ? *err : 0;
    }
}

}  // namespace

hipError_t moe_launch_stats(const moe_shape_t& s, const int32_t* counts, const int32_t* ids,
                            const int32_t* plan, const int32_t* dest_row, const int32_t* mapping,
                            const int32_t* origin, const int32_t* err, int32_t capacity,
                            int64_t* d_out, hipStream_t st)
{
    stats_kernel<<<1, kThreads, 0, st>>>(s.T, s.k, s.E, s.R, s.S, capacity, counts, ids, plan,
                                         dest_row, mapping, origin, err,
                                         reinterpret_cast<long long*>(d_out));
    return hipGetLastError();
}
