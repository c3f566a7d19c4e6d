// count_fused.h -- the one-workgroup count (up to 16384 assignments) as a
// device function, for the count kernel and for the fused count + plan.
//
// "MoE Load Balancing: Find Expert Hotspots", sections "Separate expert
// demand from rank placement" and "Work the 16-token hotspot fixture".
#pragma once

#include "common.h"

namespace moe {
namespace cnt {

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
// hist: 256 ints of LDS that end holding the counts (entries past E are 0).
// Every thread of the workgroup calls it.
__device__ __forceinline__ void count_fused_body(int N, int k, int E, int R,
                                                 const int32_t* __restrict__ ids,
                                                 int32_t* __restrict__ counts,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ eidx,
                                                 int32_t* __restrict__ rank_load, int32_t* err,
                                                 int32_t* hist)
{
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
    // a token's k assignments: when k divides 64 they sit in k adjacent
    // lanes of one round (chunks start at multiples of 64). Then a repeat
    // of an in-range id shows in the same-expert lane mask of the ranking
    // below, and only a round holding an out-of-range id compares the raw
    // ids here, the earlier ones from the lanes below by shuffles.
    // Otherwise the earlier ids come from memory.
    const bool by_lanes = 64 % k == 0;
#pragma unroll
    for (int i = 0; i < kFusedRounds; ++i) {
        if (64 * i >= C) break;
        const int a = a0 + 64 * i;
        const int32_t e = ev[i];
        const bool out = a < N && (e < 0 || e >= E);
        if (out) bad |= MOE_ERR_RANGE;
        if (by_lanes) {
            if (__ballot(out)) {
                const int j = lane % k;  // = a % k
                for (int jj = 1; jj < k; ++jj) {
                    const int32_t o = __shfl(e, lane - jj);
                    if (jj <= j && a < N && o == e) bad |= MOE_ERR_REPEAT;
                }
            }
        } else if (a < N) {
            const int j = a % k;
            for (int jj = 1; jj <= j; ++jj)
                if (ids[a - jj] == e) bad |= MOE_ERR_REPEAT;
        }
    }
    __syncthreads();

    // index within the wavefront's chunk
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // the lanes of this lane's token (k divides 64)
    const uint64_t tok_mask = k >= 64 ? ~0ull : (((1ull << k) - 1) << (lane - lane % k));
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
        if (by_lanes && ok && __popcll(match & tok_mask) > 1) bad |= MOE_ERR_REPEAT;
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

}  // namespace cnt
}  // namespace moe
