// slots.hip -- replica weight slots: the pool copy and the per-segment weight
// table of the slot-reading grouped GEMM.
//
// "Moonshot AI drops MoonEP ..." paragraph 3: the planner's redundant expert
// copies are prefetched into weight slots on the ranks that serve them;
// paragraph 4: as many slots as experts per rank make every expert the
// grouped GEMM touches local, and a few slots usually suffice. On one GPU the
// prefetch is an HBM -> HBM copy of each replica expert's three projections
// into pool[r][j] (rank r's j-th replica expert, in slot_expert order, for
// j < min(S, n)); a replica segment then reads its slot, a home segment (or
// a replica beyond the S slots: a non-local read) the home weights.
//
// The copy is a persistent grid-stride loop over 16 KB chunks (256 threads x
// 4 x 16-byte vectors, the four loads issued before the four stores) of the
// filled slots only.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kVecs = 4;                           // 16-byte vectors per thread per chunk
constexpr int kChunkVecs = kThreads * kVecs;       // 16 KB
constexpr int kPrefetchGrid = 2048;

// Expert held by slot j of rank r, or -1.
__device__ __forceinline__ int slot_expert_of(int r, int j, int E, int R, const int32_t* plan,
                                              const moe::PlanLayout& L)
{
    const int n = E / R;
    const int e = plan[L.slot_expert + (size_t)r * n + j];
    return (e >= 0 && e < E) ? e : -1;
}

// Every workgroup first lists the filled slots (at most E = R*n <= 256 slots,
// one per thread, compacted with a workgroup scan in slot order), then takes
// chunks (filled slot, projection, 16 KB piece) in a grid-stride loop, so
// empty slots cost nothing.
__global__ __launch_bounds__(kThreads) void prefetch_kernel(int E, int R, int Sm, int64_t slice_vecs,
                                                            int64_t chunks_per_slice,
                                                            const int32_t* __restrict__ plan,
                                                            const uint4* __restrict__ wg,
                                                            const uint4* __restrict__ wu,
                                                            const uint4* __restrict__ wd,
                                                            uint4* __restrict__ pool)
{
    __shared__ int32_t scan[kThreads];
    __shared__ int32_t list_slot[kThreads], list_expert[kThreads];
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int tid = threadIdx.x;
    const int nslots = R * Sm;  // <= E <= 256
    const int e_t = tid < nslots ? slot_expert_of(tid / Sm, tid % Sm, E, R, plan, L) : -1;
    scan[tid] = e_t >= 0 ? 1 : 0;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int a = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += a;
        __syncthreads();
    }
    if (e_t >= 0) {
        list_slot[scan[tid] - 1] = tid;
        list_expert[scan[tid] - 1] = e_t;
    }
    const int filled = scan[kThreads - 1];
    __syncthreads();

    const int64_t per_slot = 3 * chunks_per_slice;
    const int64_t total = (int64_t)filled * per_slot;
    for (int64_t i = blockIdx.x; i < total; i += gridDim.x) {
        const int f = (int)(i / per_slot);
        const int64_t rem = i % per_slot;
        const int q = (int)(rem / chunks_per_slice);
        const int64_t c0 = (rem % chunks_per_slice) * kChunkVecs;
        const int slot = list_slot[f], e = list_expert[f];
        const uint4* src = (q == 0 ? wg : q == 1 ? wu : wd) + (size_t)e * slice_vecs;
        uint4* dst = pool + ((size_t)slot * 3 + q) * slice_vecs;
        uint4 v[kVecs];
#pragma unroll
        for (int u = 0; u < kVecs; ++u) {
            const int64_t x = c0 + u * kThreads + tid;
            if (x < slice_vecs) v[u] = src[x];
        }
#pragma unroll
        for (int u = 0; u < kVecs; ++u) {
            const int64_t x = c0 + u * kThreads + tid;
            if (x < slice_vecs) dst[x] = v[u];
        }
    }
}

// wtab[g][q] for group g = r*2n + i (segment i of rank r): slot (r, j) of the
// pool when the segment's expert is rank r's j-th replica and j < Sm, else
// the home expert's slice. Groups past seg_num[r] get expert 0's (unread).
__global__ __launch_bounds__(kThreads) void slot_table_kernel(int E, int R, int Sm, int64_t slice_bytes,
                                                              const int32_t* __restrict__ plan,
                                                              const char* wg, const char* wu,
                                                              const char* wd, const char* pool,
                                                              uint64_t* __restrict__ wtab)
{
    const int g = blockIdx.x * kThreads + threadIdx.x;
    const int n = E / R;
    if (g >= 2 * E) return;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int r = g / (2 * n), i = g % (2 * n);
    int e = i < plan[L.seg_num + r] ? plan[L.seg_expert + g] : 0;
    if (e < 0 || e >= E) e = 0;
    const char* src[3] = {wg + e * slice_bytes, wu + e * slice_bytes, wd + e * slice_bytes};
    if (e / n != r) {
        for (int j = 0; j < Sm; ++j) {
            if (slot_expert_of(r, j, E, R, plan, L) == e) {
                const char* s0 = pool + (size_t)(r * Sm + j) * 3 * slice_bytes;
                src[0] = s0;
                src[1] = s0 + slice_bytes;
                src[2] = s0 + 2 * slice_bytes;
                break;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) wtab[3 * g + q] = reinterpret_cast<uint64_t>(src[q]);
}

}  // namespace

hipError_t moe_launch_prefetch(const moe_shape_t& s, const int32_t* plan, const void* w_gate,
                               const void* w_up, const void* w_down, void* pool, hipStream_t st)
{
    const int Sm = moe::pool_slots(s);
    if (Sm == 0) return hipSuccess;
    const int64_t slice_vecs = (int64_t)s.F * s.H * (s.dtype == MOE_BF16 ? 2 : 4) / 16;
    const int64_t cps = (slice_vecs + kChunkVecs - 1) / kChunkVecs;
    // the filled-slot count is on the device: size the grid for all slots
    const int64_t total = (int64_t)s.R * Sm * 3 * cps;
    const int grid = (int)(total < kPrefetchGrid ? total : kPrefetchGrid);
    prefetch_kernel<<<grid, kThreads, 0, st>>>(s.E, s.R, Sm, slice_vecs, cps, plan,
                                               static_cast<const uint4*>(w_gate),
                                               static_cast<const uint4*>(w_up),
                                               static_cast<const uint4*>(w_down),
                                               static_cast<uint4*>(pool));
    return hipGetLastError();
}

hipError_t moe_launch_slot_table(const moe_shape_t& s, const int32_t* plan, const void* w_gate,
                                 const void* w_up, const void* w_down, const void* pool,
                                 uint64_t* wtab, hipStream_t st)
{
    const int64_t slice_bytes = (int64_t)s.F * s.H * (s.dtype == MOE_BF16 ? 2 : 4);
    const int G = 2 * s.E;
    slot_table_kernel<<<(G + kThreads - 1) / kThreads, kThreads, 0, st>>>(
        s.E, s.R, moe::pool_slots(s), slice_bytes, plan, static_cast<const char*>(w_gate),
        static_cast<const char*>(w_up), static_cast<const char*>(w_down),
        static_cast<const char*>(pool), wtab);
    return hipGetLastError();
}
