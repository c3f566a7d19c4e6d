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
// One workgroup per token. Dispatch reads x[t] once (16-byte vector loads,
// fully coalesced) and writes it to its k destination rows, so HBM sees the
// algorithmic (T + N) * H * bytes. Combine reads the k rows it needs and
// writes out[t] once: (N + T) * H * bytes (+ T * H * bytes with a shared
// expert). Rows are contiguous, so register staging already gives whole
// 64-byte-segment transactions; there is no transpose that LDS would help.
#include "common.h"

namespace {

constexpr int kThreads = 256;

// Assignment (t,j) -> destination row; -1 if the inputs are out of range.
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

template <int VPT>  // 16-byte vectors per thread held in registers
__global__ __launch_bounds__(kThreads) void permute_kernel(int T, int k, int E, int R,
                                                           int row_vecs,
                                                           const uint4* __restrict__ x,
                                                           const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ eidx,
                                                           const int32_t* __restrict__ plan,
                                                           uint4* __restrict__ buf,
                                                           int32_t* __restrict__ dest_row,
                                                           int32_t* __restrict__ row_src)
{
    __shared__ int sdest[64];
    const int t = blockIdx.x;
    const int N = T * k;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const uint4* src = x + (size_t)t * row_vecs;
    // the row does not depend on the routing: start reading it first
    uint4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = i * kThreads + threadIdx.x;
        if (c < row_vecs) v[i] = src[c];
    }
    if (threadIdx.x < k) {
        const int a = t * k + threadIdx.x;
        const int d = dest_of(ids[a], eidx[a], E, R, N, plan, L);
        sdest[threadIdx.x] = d;
        dest_row[a] = d;
        if (d >= 0) row_src[d] = t;
    }
    __syncthreads();
    for (int base = 0; base < row_vecs; base += VPT * kThreads) {
        if (base > 0) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int c = base + i * kThreads + threadIdx.x;
                if (c < row_vecs) v[i] = src[c];
            }
        }
        for (int j = 0; j < k; ++j) {
            const int d = sdest[j];
            if (d < 0) continue;
            uint4* dst = buf + (size_t)d * row_vecs;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int c = base + i * kThreads + threadIdx.x;
                if (c < row_vecs) dst[c] = v[i];
            }
        }
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

template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(int T, int k, int row_vecs,
                                                           const uint4* __restrict__ y,
                                                           const int32_t* __restrict__ dest_row,
                                                           const float* __restrict__ w,
                                                           const uint4* __restrict__ shared_y,
                                                           uint4* __restrict__ out)
{
    using V = Vec<BF16>;
    __shared__ int sdest[64];
    __shared__ float sw[64];
    const int t = blockIdx.x;
    const int N = T * k;
    if (threadIdx.x < k) {
        const int a = t * k + threadIdx.x;
        const int d = dest_row[a];
        sdest[threadIdx.x] = (d >= 0 && d < N) ? d : -1;
        sw[threadIdx.x] = w[a];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < row_vecs; c += kThreads) {
        float acc[V::kN];
#pragma unroll
        for (int i = 0; i < V::kN; ++i) acc[i] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int d = sdest[j];
            if (d < 0) continue;
            float f[V::kN];
            V::load(y[(size_t)d * row_vecs + c], f);
            const float wj = sw[j];
#pragma unroll
            for (int i = 0; i < V::kN; ++i) acc[i] = fmaf(wj, f[i], acc[i]);
        }
        if (shared_y) {
            float f[V::kN];
            V::load(shared_y[(size_t)t * row_vecs + c], f);
#pragma unroll
            for (int i = 0; i < V::kN; ++i) acc[i] += f[i];
        }
        out[(size_t)t * row_vecs + c] = V::store(acc);
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
    const uint4* xv = static_cast<const uint4*>(x);
    uint4* bv = static_cast<uint4*>(buf);
    if (row_vecs <= 2 * kThreads)
        permute_kernel<2><<<s.T, kThreads, 0, st>>>(s.T, s.k, s.E, s.R, row_vecs, xv, ids, eidx,
                                                    plan, bv, dest_row, row_src);
    else
        permute_kernel<4><<<s.T, kThreads, 0, st>>>(s.T, s.k, s.E, s.R, row_vecs, xv, ids, eidx,
                                                    plan, bv, dest_row, row_src);
    return hipGetLastError();
}

hipError_t moe_launch_combine(const moe_shape_t& s, const void* y, const int32_t* dest_row,
                              const float* w, const void* shared_y, void* out, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    const int bytes = s.dtype == MOE_BF16 ? 2 : 4;
    const int row_vecs = s.H * bytes / 16;
    if (s.dtype == MOE_BF16)
        combine_kernel<true><<<s.T, kThreads, 0, st>>>(
            s.T, s.k, row_vecs, static_cast<const uint4*>(y), dest_row, w,
            static_cast<const uint4*>(shared_y), static_cast<uint4*>(out));
    else
        combine_kernel<false><<<s.T, kThreads, 0, st>>>(
            s.T, s.k, row_vecs, static_cast<const uint4*>(y), dest_row, w,
            static_cast<const uint4*>(shared_y), static_cast<uint4*>(out));
    return hipGetLastError();
}
