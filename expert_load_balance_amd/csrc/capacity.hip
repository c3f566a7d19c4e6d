// capacity.hip -- the two baselines the equal-load plan is measured against:
// fixed-capacity dispatch (drop and pad) and greedy repacking of experts onto
// ranks.
//
// "MoE Load Balancing: Find Expert Hotspots", "Make expert capacity,
// overflow, and padding explicit": every expert has the same capacity cap;
// demand above it overflows and unused slots below it are padding. Here an
// expert keeps its first cap assignments in stable order (eidx < cap), in a
// static [E][cap] buffer whose padding rows are zero.
// Same page, "Separate expert demand from rank placement": a mapping that
// pairs hot and cold experts evens out rank demand ({0,7},{1,6},{2,5},{3,4}
// for the fixture). Here: experts by decreasing demand (equal: lower id) each
// go to the least-loaded rank that holds fewer than n = E/R experts (equal:
// lower rank).
#include "common.h"

namespace {

constexpr int kThreads = 256;

// One wavefront per (token, 1 KB row chunk), as in dispatch: lanes 0..k-1
// resolve the k destinations (-1: dropped or out of range).
__global__ __launch_bounds__(kThreads) void capacity_dispatch_kernel(
    int T, int k, int E, int cap, int row_vecs, int nchunks, const uint4* __restrict__ x,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ eidx, uint4* __restrict__ buf,
    int32_t* __restrict__ dest_row)
{
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= (int64_t)T * nchunks) return;
    const int t = (int)(wid / nchunks), ch = (int)(wid % nchunks);
    const int c = ch * 64 + lane;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (c < row_vecs) v = x[(size_t)t * row_vecs + c];
    int d = -1;
    if (lane < k) {
        const int a = t * k + lane;
        const int e = ids[a], r = eidx[a];
        if (e >= 0 && e < E && r >= 0 && r < cap) d = e * cap + r;
        if (ch == 0) dest_row[a] = d;
    }
    for (int j = 0; j < k; ++j) {
        const int dj = __builtin_amdgcn_readlane(d, j);
        if (dj >= 0 && c < row_vecs) buf[(size_t)dj * row_vecs + c] = v;
    }
}

// Zeroes the padding rows: row e*cap + r with r >= min(counts[e], cap).
__global__ __launch_bounds__(kThreads) void capacity_pad_kernel(int E, int cap, int row_vecs,
                                                                int nchunks,
                                                                const int32_t* __restrict__ counts,
                                                                uint4* __restrict__ buf)
{
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= (int64_t)E * cap * nchunks) return;
    const int64_t row = wid / nchunks;
    const int ch = (int)(wid % nchunks);
    const int e = (int)(row / cap), r = (int)(row % cap);
    if (r < counts[e]) return;  // a kept row (counts >= cap: no padding)
    const int c = ch * 64 + lane;
    if (c < row_vecs) buf[row * row_vecs + c] = make_uint4(0, 0, 0, 0);
}

// The plan block of the capacity layout: every expert is home on rank e / n
// with one piece of cap rows at row e * cap; no replicas.
__global__ __launch_bounds__(kThreads) void capacity_plan_kernel(int E, int R, int cap,
                                                                 int32_t* __restrict__ plan)
{
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int n = E / R;
    for (int i = threadIdx.x; i < R; i += kThreads) {
        plan[L.quota + i] = n * cap;
        plan[L.seg_num + i] = n;
        plan[L.slots_needed + i] = 0;
        plan[L.donor + i] = -1;
    }
    for (int i = threadIdx.x; i <= R; i += kThreads) plan[L.win_off + i] = i * n * cap;
    for (int i = threadIdx.x; i < R * 2 * n; i += kThreads) {
        const int r = i / (2 * n), q = i % (2 * n);
        const int e = r * n + q;
        plan[L.seg_expert + i] = q < n ? e : -1;
        plan[L.seg_row + i] = q < n ? e * cap : -1;
        plan[L.seg_cnt + i] = q < n ? cap : 0;
    }
    for (int i = threadIdx.x; i < R * n; i += kThreads) plan[L.slot_expert + i] = -1;
    for (int i = threadIdx.x; i < E; i += kThreads) plan[L.piece_num + i] = 1;
    for (int i = threadIdx.x; i < E * R; i += kThreads) {
        const int e = i / R, p = i % R;
        plan[L.piece_rank + i] = p == 0 ? e / n : -1;
        plan[L.piece_row + i] = p == 0 ? e * cap : -1;
        plan[L.piece_cnt + i] = p == 0 ? cap : 0;
    }
}

// Greedy balanced packing in one workgroup: the experts' order by (count
// desc, id asc) is a rank count per expert; one wavefront then places them in
// that order, lane r holding rank r's load and number of experts.
__global__ __launch_bounds__(kThreads) void repack_kernel(int E, int R,
                                                          const int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ mapping)
{
    __shared__ int32_t sc[256], order[256];
    const int tid = threadIdx.x;
    if (tid < E) sc[tid] = counts[tid];
    __syncthreads();
    if (tid < E) {
        const int c = sc[tid];
        int pos = 0;
        for (int e = 0; e < E; ++e) pos += (sc[e] > c || (sc[e] == c && e < tid)) ? 1 : 0;
        order[pos] = tid;
    }
    __syncthreads();
    if (tid >= 64) return;
    const int n = E / R;
    int64_t load = 0;
    int held = 0;
    for (int i = 0; i < E; ++i) {
        const int e = order[i];
        // least-loaded rank with room; equal loads -> lower rank
        int64_t key = (tid < R && held < n) ? load * 64 + tid : INT64_MAX;
        for (int off = 32; off > 0; off >>= 1) {
            const int64_t o = __shfl_xor(key, off);
            key = o < key ? o : key;
        }
        const int r = (int)(key % 64);
        if (tid == r) {
            load += sc[e];
            held += 1;
        }
        if (tid == 0) mapping[e] = r;
    }
}

}  // namespace

hipError_t moe_launch_capacity_dispatch(const moe_shape_t& s, int cap, const int32_t* counts,
                                        const void* x, const int32_t* ids, const int32_t* eidx,
                                        void* buf, int32_t* dest_row, hipStream_t st)
{
    const int bytes = s.dtype == MOE_BF16 ? 2 : 4;
    const int row_vecs = s.H * bytes / 16;
    const int nchunks = (row_vecs + 63) / 64;
    uint4* bv = static_cast<uint4*>(buf);
    if (s.T > 0) {
        const int64_t waves = (int64_t)s.T * nchunks;
        capacity_dispatch_kernel<<<(unsigned)((waves + 3) / 4), kThreads, 0, st>>>(
            s.T, s.k, s.E, cap, row_vecs, nchunks, static_cast<const uint4*>(x), ids, eidx, bv,
            dest_row);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t waves = (int64_t)s.E * cap * nchunks;
    capacity_pad_kernel<<<(unsigned)((waves + 3) / 4), kThreads, 0, st>>>(s.E, cap, row_vecs,
                                                                           nchunks, counts, bv);
    return hipGetLastError();
}

hipError_t moe_launch_capacity_plan(const moe_shape_t& s, int cap, int32_t* plan, hipStream_t st)
{
    capacity_plan_kernel<<<1, kThreads, 0, st>>>(s.E, s.R, cap, plan);
    return hipGetLastError();
}

hipError_t moe_launch_repack(const moe_shape_t& s, const int32_t* counts, int32_t* mapping,
                             hipStream_t st)
{
    repack_kernel<<<1, kThreads, 0, st>>>(s.E, s.R, counts, mapping);
    return hipGetLastError();
}
