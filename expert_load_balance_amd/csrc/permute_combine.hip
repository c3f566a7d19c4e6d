// permute_combine.hip -- dispatch into the static-shape buffer and the
// gate-weighted combine. Both are HBM-bound row moves.
//
// "DeepEP-on-EFA Guidance, section 1": dispatch (phase b) sends a token only
// to its k experts; combine (phase d) brings expert outputs back and sums them
// with the gate weights, the transpose of dispatch.
// "Moonshot AI drops MoonEP ..." paragraph 3: zero-copy placement -- each
// assignment is written once, straight into its final row of a buffer whose
// shape does not depend on the routing.
//
// Dispatch reads x[t] once (16-byte vector loads,
// fully coalesced) and writes it to its k destination rows, so HBM sees the
// algorithmic (T + N) * H * bytes. Combine reads the k rows it needs and
// writes out[t] once: (N + T) * H * bytes (+ T * H * bytes with a shared
// expert). Rows are contiguous in both source and destination, so staging
// through registers already gives whole-line transactions; there is no
// transpose or reuse that an LDS stage would serve. Measured on MI355X: the
// dispatch of the DeepSeek-V3 shape (1.06 GB) runs at 5.6 TB/s of kernel
// time, faster than the runtime's own device-to-device copy (5.3 TB/s on
// 1 GiB), and its HBM counter bytes equal the algorithmic bytes (1.01x).
#include "common.h"

namespace {

constexpr int kThreads = 256;

// Assignment (e, v) -> destination row: it lands in the piece of expert e
// whose running count range holds v, at that piece's row + (v - rows before
// it); -1 if the inputs are out of range. One lane walks the pieces.
__device__ __forceinline__ int dest_of(int e, int v, int E, int R, int N, const int32_t* plan,
                                       const moe::PlanLayout& L)
{
    if (e < 0 || e >= E || v < 0) return -1;
    const int np = plan[L.piece_num + e];
    const int32_t* pr = plan + L.piece_row + (size_t)e * R;
    const int32_t* pc = plan + L.piece_cnt + (size_t)e * R;
    int cum = 0;
    for (int p = 0; p < np && p < R; ++p) {
        const int c = pc[p];
        if (v < cum + c) {
            const int d = pr[p] + (v - cum);
            return (d >= 0 && d < N) ? d : -1;
        }
        cum += c;
    }
    return -1;
}

// Destination rows of token t's k assignments; lane j < k returns
// assignment j's row. When the k experts' pieces fit one wavefront (k * G <=
// 64, G = R rounded up to a power of two), lane j * G + p reads piece p of
// assignment j's expert, all pieces at once: one round trip to memory after
// the ids instead of one per piece; a prefix sum over the group's lanes
// gives the ranges and a ballot the matching piece. Otherwise each lane
// j < k walks its expert's pieces (measured faster than several passes of
// the wavefront-wide lookup).
__device__ __forceinline__ int resolve_dests(int t, int k, int E, int R, int N,
                                             const int32_t* __restrict__ ids,
                                             const int32_t* __restrict__ eidx,
                                             const int32_t* __restrict__ plan)
{
    const int lane = threadIdx.x & 63;
    int e = -1, v = -1;
    if (lane < k) {
        e = ids[t * k + lane];
        v = eidx[t * k + lane];
    }
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int G = R <= 1 ? 1 : 1 << (32 - __builtin_clz(R - 1));
    if (k * G > 64) return lane < k ? dest_of(e, v, E, R, N, plan, L) : -1;
    const int j = lane / G, p = lane % G;
    int d = -1;
    {
        const int ej = __shfl(e, j < k ? j : 0), vj = __shfl(v, j < k ? j : 0);
        const bool ok = j < k && ej >= 0 && ej < E && vj >= 0 && p < R;
        int np = 0, c = 0, r = 0;
        if (ok) {
            np = plan[L.piece_num + ej];
            c = plan[L.piece_cnt + (size_t)ej * R + p];
            r = plan[L.piece_row + (size_t)ej * R + p];
        }
        if (p >= np) c = 0;
        int s = c;
        for (int off = 1; off < G; off <<= 1) {
            const int y = __shfl_up(s, off, G);
            if (p >= off) s += y;
        }
        const int before = s - c;
        const bool hit = ok && p < np && vj >= before && vj < s;
        const int row = r + (vj - before);
        const uint64_t m = __ballot(hit);
        for (int jj = 0; jj < k; ++jj) {
            const uint64_t gm = (m >> (jj * G)) & (G == 64 ? ~0ull : ((1ull << G) - 1));
            if (gm == 0) continue;
            const int src = jj * G + __ffsll((unsigned long long)gm) - 1;
            const int dj = __builtin_amdgcn_readlane(row, src);
            if (lane == jj) d = (dj >= 0 && dj < N) ? dj : -1;
        }
    }
    return d;
}

// Work split: one wavefront per (token, row chunk); a chunk is 64 lanes x VPL
// 16-byte vectors. Each wavefront resolves the token's k destinations itself
// (lanes 0..k-1, broadcast with readlane), so there is no LDS and no barrier.
// Measured on MI355X over the 2 KB .. 14 KB rows of the workloads here,
// dispatch is fastest with 1 KB chunks (one vector per lane: the most
// wavefronts in flight) and combine with 2 KB chunks.
constexpr int kPermuteVpl = 1;
constexpr int kVpl = 2;  // combine
constexpr int kChunkVecs = 64 * kVpl;

template <int VPL>
__global__ __launch_bounds__(kThreads) void permute_kernel(int T, int k, int E, int R, int row_vecs,
                                                           int nchunks,
                                                           const uint4* __restrict__ x,
                                                           const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ eidx,
                                                           const int32_t* __restrict__ plan,
                                                           uint4* __restrict__ buf,
                                                           int32_t* __restrict__ dest_row,
                                                           int32_t* __restrict__ row_src)
{
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= (int64_t)T * nchunks) return;
    const int t = (int)(wid / nchunks), ch = (int)(wid % nchunks);
    const int N = T * k;
    const int c0 = ch * 64 * VPL + lane;
    const uint4* src = x + (size_t)t * row_vecs;
    // the row does not depend on the routing: start reading it first
    uint4 v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (c0 + 64 * i < row_vecs) v[i] = src[c0 + 64 * i];
    const int d = resolve_dests(t, k, E, R, N, ids, eidx, plan);
    if (lane < k && ch == 0) {
        dest_row[t * k + lane] = d;
        if (d >= 0) row_src[d] = t;
    }
    for (int j = 0; j < k; ++j) {
        const int dj = __builtin_amdgcn_readlane(d, j);
        if (dj < 0) continue;
        uint4* dst = buf + (size_t)dj * row_vecs;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (c0 + 64 * i < row_vecs) dst[c0 + 64 * i] = v[i];
    }
}

// fp32 accumulate of 16-byte vectors: 8 bf16 or 4 f32 lanes
template <bool BF16>
struct Vec;

template <>
struct Vec<true> {
    static constexpr int kN = 8;
    __device__ static void load(const uint4& u, float* f)
    {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static uint4 store(const float* f)
    {
        uint4 u;
        u.x = moe::pack_bf16x2(f[0], f[1]);
        u.y = moe::pack_bf16x2(f[2], f[3]);
        u.z = moe::pack_bf16x2(f[4], f[5]);
        u.w = moe::pack_bf16x2(f[6], f[7]);
        return u;
    }
};

template <>
struct Vec<false> {
    static constexpr int kN = 4;
    __device__ static void load(const uint4& u, float* f)
    {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
    __device__ static uint4 store(const float* f)
    {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
};

// One wavefront per (token, row chunk) as in permute; lanes 0..k-1 hold the
// k destination rows and weights (broadcast with readlane). The k source rows
// are read four at a time before they are accumulated (fp32, in j order);
// then the shared row is added.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(int T, int k, int64_t nrows, int row_vecs,
                                                           int nchunks,
                                                           const uint4* __restrict__ y,
                                                           const int32_t* __restrict__ dest_row,
                                                           const float* __restrict__ w,
                                                           const uint4* __restrict__ shared_y,
                                                           uint4* __restrict__ out)
{
    using V = Vec<BF16>;
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= (int64_t)T * nchunks) return;
    const int t = (int)(wid / nchunks), ch = (int)(wid % nchunks);
    const int c0 = ch * kChunkVecs + lane;
    int d = -1;
    float wl = 0.0f;
    if (lane < k) {
        const int a = t * k + lane;
        const int dd = dest_row[a];
        d = (dd >= 0 && dd < nrows) ? dd : -1;
        wl = w ? w[a] : 1.0f;  // no weights: the plain sum (dispatch's backward)
    }
    float acc[kVpl][V::kN];
#pragma unroll
    for (int i = 0; i < kVpl; ++i)
#pragma unroll
        for (int q = 0; q < V::kN; ++q) acc[i][q] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 4) {
        uint4 u[4][kVpl];
        int dj[4];
        float wj[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = j0 + jj < k ? j0 + jj : k - 1;
            dj[jj] = j0 + jj < k ? __builtin_amdgcn_readlane(d, j) : -1;
            wj[jj] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), j));
            if (dj[jj] < 0) continue;
            const uint4* src = y + (size_t)dj[jj] * row_vecs;
#pragma unroll
            for (int i = 0; i < kVpl; ++i)
                if (c0 + 64 * i < row_vecs) u[jj][i] = src[c0 + 64 * i];
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            if (dj[jj] < 0) continue;
#pragma unroll
            for (int i = 0; i < kVpl; ++i) {
                float f[V::kN];
                V::load(u[jj][i], f);
#pragma unroll
                for (int q = 0; q < V::kN; ++q) acc[i][q] = fmaf(wj[jj], f[q], acc[i][q]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
        const int c = c0 + 64 * i;
        if (c >= row_vecs) continue;
        if (shared_y) {
            float f[V::kN];
            V::load(shared_y[(size_t)t * row_vecs + c], f);
#pragma unroll
            for (int q = 0; q < V::kN; ++q) acc[i][q] += f[q];
        }
        out[(size_t)t * row_vecs + c] = V::store(acc[i]);
    }
}

}  // namespace

hipError_t moe_launch_permute(const moe_shape_t& s, const void* x, const int32_t* ids,
                              const int32_t* eidx, const int32_t* plan, void* buf,
                              int32_t* dest_row, int32_t* row_src, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    const int bytes = s.dtype == MOE_BF16 ? 2 : 4;
    const int row_vecs = s.H * bytes / 16;
    const int vpl = kPermuteVpl;
    const int nchunks = (row_vecs + 64 * vpl - 1) / (64 * vpl);
    const int64_t waves = (int64_t)s.T * nchunks;
    const int grid = (int)((waves + kThreads / 64 - 1) / (kThreads / 64));
    const uint4* xv = static_cast<const uint4*>(x);
    uint4* bv = static_cast<uint4*>(buf);
    switch (vpl) {
#define MOE_PERMUTE(V)                                                                           \
    case V:                                                                                      \
        permute_kernel<V><<<grid, kThreads, 0, st>>>(s.T, s.k, s.E, s.R, row_vecs, nchunks, xv, ids, \
                                                      eidx, plan, bv, dest_row, row_src);        \
        break;
        MOE_PERMUTE(1) MOE_PERMUTE(2) MOE_PERMUTE(4) MOE_PERMUTE(8)
#undef MOE_PERMUTE
    }
    return hipGetLastError();
}

hipError_t moe_launch_combine_rows(const moe_shape_t& s, int64_t nrows, const void* y,
                                   const int32_t* dest_row, const float* w, const void* shared_y,
                                   void* out, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    const int bytes = s.dtype == MOE_BF16 ? 2 : 4;
    const int row_vecs = s.H * bytes / 16;
    const int nchunks = (row_vecs + kChunkVecs - 1) / kChunkVecs;
    const int64_t waves = (int64_t)s.T * nchunks;
    const int grid = (int)((waves + kThreads / 64 - 1) / (kThreads / 64));
    const uint4* yv = static_cast<const uint4*>(y);
    const uint4* sv = static_cast<const uint4*>(shared_y);
    uint4* ov = static_cast<uint4*>(out);
    if (s.dtype == MOE_BF16)
        combine_kernel<true><<<grid, kThreads, 0, st>>>(s.T, s.k, nrows, row_vecs, nchunks, yv,
                                                        dest_row, w, sv, ov);
    else
        combine_kernel<false><<<grid, kThreads, 0, st>>>(s.T, s.k, nrows, row_vecs, nchunks, yv,
                                                         dest_row, w, sv, ov);
    return hipGetLastError();
}

hipError_t moe_launch_combine(const moe_shape_t& s, const void* y, const int32_t* dest_row,
                              const float* w, const void* shared_y, void* out, hipStream_t st)
{
    return moe_launch_combine_rows(s, (int64_t)s.T * s.k, y, dest_row, w, shared_y, out, st);
}
