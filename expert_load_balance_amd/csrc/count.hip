// count.hip -- per-expert demand, exclusive offsets, stable within-expert
// index and home rank loads.
//
// "MoE Load Balancing: Find Expert Hotspots", sections "Separate expert
// demand from rank placement" (count assignments by expert first, then sum
// under the expert -> rank mapping) and "Work the 16-token hotspot fixture"
// (an unknown id or a token repeating an expert stops the count).
//
// Up to 16384 assignments, one workgroup of 1024 threads does it all in one
// launch (count_fused_kernel: each wavefront ranks a contiguous chunk, then
// the chunk bases). Above that, three launches, none of whose results
// depend on thread timing:
//   1. hist: workgroup b histograms assignments [b*C, (b+1)*C) in LDS (the
//      adds are order-free), writes blk_hist[b][E], and checks ids.
//   2. scan: one workgroup; thread e scans blk_hist[.][e] over workgroups
//      (blk_base), giving counts[e]; then offsets and home rank loads.
//   3. rank: workgroup b walks its chunk again in 256-assignment rounds.
//      Within a wavefront, lanes holding the same expert are found with
//      eight ballots over the bits of the id (a multisplit match); a lane's
//      rank among them is the popcount of the lower matching lanes. The
//      per-wave match counts, prefixed over the four wavefronts in LDS, and
//      the running per-expert base give eidx in flat (t*k+j) order.
#include <mutex>

#include "common.h"
#include "count_fused.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / moe::kWave;

__global__ __launch_bounds__(kThreads) void count_hist_kernel(int N, int k, int E,
                                                              const int32_t* __restrict__ ids,
                                                              int32_t* __restrict__ blk_hist,
                                                              int32_t* err)
{
    __shared__ int32_t hist[256];
    for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * moe::kCountChunk;
    int bad = 0;
    // lane l holds assignment base + 256 m + 64 w + l: with k dividing 64 a
    // token's earlier assignments are in the lanes below (shuffles)
    const bool by_lanes = 64 % k == 0;
    const int lane = threadIdx.x % moe::kWave;
    for (int i = threadIdx.x; i < moe::kCountChunk; i += kThreads) {
        const int64_t a = base + i;
        const int32_t e = a < N ? ids[a] : -1;
        if (by_lanes) {
            const int j = lane % k;  // = a % k
            for (int jj = 1; jj < k; ++jj) {
                const int32_t o = __shfl(e, lane - jj);
                if (jj <= j && a < N && o == e) bad |= MOE_ERR_REPEAT;
            }
        } else if (a < N) {
            const int j = (int)(a % k);
            for (int jj = 1; jj <= j; ++jj)
                if (ids[a - jj] == e) bad |= MOE_ERR_REPEAT;
        }
        if (a >= N) continue;
        if (e < 0 || e >= E) {
            bad |= MOE_ERR_RANGE;
            continue;
        }
        atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) blk_hist[(size_t)blockIdx.x * E + e] = hist[e];
    if (bad) atomicOr(err, bad);
}

__global__ __launch_bounds__(kThreads) void count_scan_kernel(int B, int E, int R,
                                                              const int32_t* __restrict__ blk_hist,
                                                              int32_t* __restrict__ blk_base,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ rank_load)
{
    __shared__ int32_t sc[256];
    const int e = threadIdx.x;
    int32_t run = 0;
    if (e < E) {
        // 16 loads in flight at a time, then their running sum
        for (int b0 = 0; b0 < B; b0 += 16) {
            int32_t h[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) h[j] = b0 + j < B ? blk_hist[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (b0 + j >= B) break;
                blk_base[(size_t)(b0 + j) * E + e] = run;
                run += h[j];
            }
        }
        counts[e] = run;
    }
    sc[e] = (e < E) ? run : 0;
    __syncthreads();
    // inclusive Hillis-Steele scan over 256 entries
    for (int off = 1; off < kThreads; off <<= 1) {
        const int32_t v = (e >= off) ? sc[e - off] : 0;
        __syncthreads();
        sc[e] += v;
        __syncthreads();
    }
    if (e < E) offsets[e + 1] = sc[e];
    if (e == 0) offsets[0] = 0;
    if (e < R) {
        const int n = E / R;
        rank_load[e] = sc[(e + 1) * n - 1] - (e > 0 ? sc[e * n - 1] : 0);
    }
}

__global__ __launch_bounds__(kThreads) void count_rank_kernel(int N, int E,
                                                              const int32_t* __restrict__ ids,
                                                              const int32_t* __restrict__ blk_base,
                                                              int32_t* __restrict__ eidx)
{
    __shared__ int32_t base[256];
    __shared__ int32_t wcnt[kWaves][256];
    const int tid = threadIdx.x;
    const int wave = tid / moe::kWave;
    const int lane = tid % moe::kWave;
    for (int e = tid; e < 256; e += kThreads) {
        base[e] = (e < E) ? blk_base[(size_t)blockIdx.x * E + e] : 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) wcnt[w][e] = 0;
    }
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    __syncthreads();

    const int64_t chunk0 = (int64_t)blockIdx.x * moe::kCountChunk;
    for (int r0 = 0; r0 < moe::kCountChunk; r0 += kThreads) {
        if (chunk0 + r0 >= N) break;  // uniform across the workgroup
        const int64_t a = chunk0 + r0 + tid;
        const bool valid = a < N;
        const int32_t e = valid ? ids[a] : -1;
        const bool ok = valid && e >= 0 && e < E;
        uint64_t match = __ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = ok && ((e >> b) & 1);
            const uint64_t bal = __ballot(bit);
            match &= bit ? bal : ~bal;
        }
        const int rank = __popcll(match & lt_mask);
        if (ok && rank == 0) wcnt[wave][e] = __popcll(match);
        __syncthreads();
        if (ok) {
            int32_t pre = base[e];
            for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
            eidx[a] = pre + rank;
        } else if (valid) {
            eidx[a] = -1;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kThreads) {
            int32_t s = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                s += wcnt[w][x];
                wcnt[w][x] = 0;
            }
            base[x] += s;
        }
        __syncthreads();
    }
}

// The one-workgroup count as its own launch.
__global__ __launch_bounds__(moe::cnt::kFusedThreads) void count_fused_kernel(
    int N, int k, int E, int R, const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ eidx, int32_t* __restrict__ rank_load,
    int32_t* err)
{
    __shared__ int32_t hist[256];
    moe::cnt::count_fused_body(N, k, E, R, ids, counts, offsets, eidx, rank_load, err, hist);
}

}  // namespace

namespace {

// The count proper, with the multi-launch path's per-workgroup tables at
// blk_hist and blk_base (int32[B][E] each; unused up to 16384 assignments).
// Every entry of both tables is written before it is read, so they need no
// clearing between calls.
hipError_t launch_count(const moe_shape_t& s, const int32_t* ids, int32_t* counts,
                        int32_t* offsets, int32_t* eidx, int32_t* rank_load, int32_t* err,
                        int32_t* blk_hist, int32_t* blk_base, hipStream_t st)
{
    const int64_t N = (int64_t)s.T * s.k;
    const int B = moe::count_blocks(N);
    if (N <= moe::cnt::kFusedMax) {
        count_fused_kernel<<<1, moe::cnt::kFusedThreads, 0, st>>>((int)N, s.k, s.E, s.R, ids, counts, offsets,
                                                         eidx, rank_load, err);
        return hipGetLastError();
    }
    if (B > 0) {
        count_hist_kernel<<<B, kThreads, 0, st>>>((int)N, s.k, s.E, ids, blk_hist, err);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    count_scan_kernel<<<1, kThreads, 0, st>>>(B, s.E, s.R, blk_hist, blk_base, counts, offsets,
                                              rank_load);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || B == 0) return e;
    count_rank_kernel<<<B, kThreads, 0, st>>>((int)N, s.E, ids, blk_base, eidx);
    return hipGetLastError();
}

}  // namespace

hipError_t moe_launch_count(const moe_shape_t& s, const int32_t* ids, int32_t* counts,
                            int32_t* offsets, int32_t* eidx, int32_t* rank_load, int32_t* err,
                            char* ws, hipStream_t st)
{
    const moe::WsLayout L = moe::ws_layout(s);
    return launch_count(s, ids, counts, offsets, eidx, rank_load, err,
                        reinterpret_cast<int32_t*>(ws + L.blk_hist),
                        reinterpret_cast<int32_t*>(ws + L.blk_base), st);
}

// ---- the count without a caller workspace --------------------------------
// For callers that cannot allocate (graph capture, allocation-free loops):
// the multi-launch path's two tables live in this fixed device array instead
// of the workspace. Each GPU the library runs on holds its own copy until the
// process ends; every call on a GPU shares it, so calls that overlap on one
// GPU (other streams, other host threads) race on it.
static __device__ __align__(256) char scratch[moe::kCountScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // the array's device address on each GPU, once known

// The device address of `scratch` on the current GPU, looked up once per
// device (host code must not use the array's name as a device address).
hipError_t scratch_on_current_device(char** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = static_cast<char*>(g_scratch[dev]);
    return hipSuccess;
}

}  // namespace

hipError_t moe_launch_count_noalloc(const moe_shape_t& s, const int32_t* ids, int32_t* counts,
                                    int32_t* offsets, int32_t* eidx, int32_t* rank_load,
                                    int32_t* err, hipStream_t st)
{
    char* p = nullptr;
    const hipError_t e = scratch_on_current_device(&p);
    if (e != hipSuccess) return e;
    const int64_t N = (int64_t)s.T * s.k;
    const size_t table = moe::count_table_bytes(N, s.E);
    return launch_count(s, ids, counts, offsets, eidx, rank_load, err,
                        reinterpret_cast<int32_t*>(p), reinterpret_cast<int32_t*>(p + table), st);
}
