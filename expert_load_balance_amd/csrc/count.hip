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
#include "common.h"

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
    for (int i = threadIdx.x; i < moe::kCountChunk; i += kThreads) {
        const int64_t a = base + i;
        if (a >= N) break;
        const int32_t e = ids[a];
        const int j = (int)(a % k);
        for (int jj = 1; jj <= j; ++jj)
            if (ids[a - jj] == e) bad |= MOE_ERR_REPEAT;
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

constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / moe::kWave;
constexpr int kFusedMax = 16384;  // assignments handled by the one-workgroup path
constexpr int kFusedRounds = kFusedMax / kFusedThreads;  // ids per thread

// The one-workgroup path. Wavefront w takes the contiguous assignments
// [w C, (w + 1) C), C = 64 ceil(N / 1024), 64 at a time in order: lanes
// holding the same expert are found with ballots over the id bits, and a
// lane's index within the wavefront's chunk is the chunk's running count of
// that expert (a per-wavefront LDS row, no barrier) plus its rank among the
// matching lower lanes. After one barrier, the exclusive prefix over the
// wavefronts of each expert's chunk counts gives the chunk bases, and their
// sum the counts.
__global__ __launch_bounds__(kFusedThreads) void count_fused_kernel(int N, int k, int E, int R,
                                                                     const int32_t* __restrict__ ids,
                                                                     int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ eidx,
                                                                     int32_t* __restrict__ rank_load,
                                                                     int32_t* err)
{
    __shared__ int32_t hist[256];
    __shared__ int32_t sc[256];
    __shared__ int32_t wcnt[kFusedWaves][256];
    __shared__ int32_t wsum[4];
    const int tid = threadIdx.x;
    const int wave = tid / moe::kWave;
    const int lane = tid % moe::kWave;
    for (int x = tid; x < kFusedWaves * 256; x += kFusedThreads) (&wcnt[0][0])[x] = 0;
    const int C = 64 * ((N + kFusedThreads - 1) / kFusedThreads);
    const int a0 = wave * C + lane;
    // the lane's ids, assignments a0 + 64 i, and their checks
    int32_t ev[kFusedRounds];
    int bad = 0;
#pragma unroll
    for (int i = 0; i < kFusedRounds; ++i) {
        const int a = a0 + 64 * i;
        ev[i] = 64 * i < C && a < N ? ids[a] : -1;
    }
#pragma unroll
    for (int i = 0; i < kFusedRounds; ++i) {
        const int a = a0 + 64 * i;
        if (64 * i >= C || a >= N) break;
        const int32_t e = ev[i];
        const int j = a % k;
        for (int jj = 1; jj <= j; ++jj)
            if (ids[a - jj] == e) bad |= MOE_ERR_REPEAT;
        if (e < 0 || e >= E) bad |= MOE_ERR_RANGE;
    }
    __syncthreads();

    // index within the wavefront's chunk
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int32_t loc[kFusedRounds];
#pragma unroll
    for (int i = 0; i < kFusedRounds; ++i) {
        loc[i] = -1;
        if (64 * i >= C) break;
        const int32_t e = ev[i];
        const bool ok = a0 + 64 * i < N && e >= 0 && e < E;
        uint64_t match = __ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = ok && ((e >> b) & 1);
            const uint64_t bal = __ballot(bit);
            match &= bit ? bal : ~bal;
        }
        const int rank = __popcll(match & lt_mask);
        // every matching lane reads the running count before the first of
        // them (rank 0) advances it: one wavefront's LDS operations execute
        // in order
        const int32_t prev = ok ? wcnt[wave][e] : 0;
        if (ok) loc[i] = prev + rank;
        if (ok && rank == 0) wcnt[wave][e] = prev + __popcll(match);
    }
    __syncthreads();

    // chunk bases (exclusive prefix over the wavefronts) and counts
    if (tid < 256) {
        int32_t run = 0;
        if (tid < E) {
#pragma unroll
            for (int w = 0; w < kFusedWaves; ++w) {
                const int32_t c = wcnt[w][tid];
                wcnt[w][tid] = run;
                run += c;
            }
        }
        hist[tid] = run;
        // inclusive scan of the 256 counts: wavefronts 0..3 scan 64 each
        // with shuffles, then add the totals of the wavefronts before them
        int32_t inc = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        if (lane == 63) wsum[wave] = inc;
        sc[tid] = inc;
    }
    __syncthreads();
    if (tid < 256) {
        for (int w = 0; w < wave; ++w) sc[tid] += wsum[w];
    }
    // eidx: index within the chunk + the chunk's base
#pragma unroll
    for (int i = 0; i < kFusedRounds; ++i) {
        const int a = a0 + 64 * i;
        if (64 * i >= C || a >= N) break;
        eidx[a] = loc[i] >= 0 ? loc[i] + wcnt[wave][ev[i]] : -1;
    }
    __syncthreads();
    if (tid < E) {
        counts[tid] = hist[tid];
        offsets[tid + 1] = sc[tid];
    }
    if (tid == 0) offsets[0] = 0;
    if (tid < R) {
        const int n = E / R;
        rank_load[tid] = sc[(tid + 1) * n - 1] - (tid > 0 ? sc[tid * n - 1] : 0);
    }
    if (bad) atomicOr(err, bad);
}

}  // namespace

hipError_t moe_launch_count(const moe_shape_t& s, const int32_t* ids, int32_t* counts,
                            int32_t* offsets, int32_t* eidx, int32_t* rank_load, int32_t* err,
                            char* ws, hipStream_t st)
{
    const moe::WsLayout L = moe::ws_layout(s);
    const int64_t N = (int64_t)s.T * s.k;
    int32_t* blk_hist = reinterpret_cast<int32_t*>(ws + L.blk_hist);
    int32_t* blk_base = reinterpret_cast<int32_t*>(ws + L.blk_base);
    const int B = L.count_blocks;
    if (N <= kFusedMax) {
        count_fused_kernel<<<1, kFusedThreads, 0, st>>>((int)N, s.k, s.E, s.R, ids, counts, offsets,
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
