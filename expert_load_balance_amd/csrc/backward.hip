// backward.hip -- the row-move and gate steps of the layer's backward.
//
// "DeepEP-on-EFA Guidance, section 1", phases (d), (b) and (a) in reverse:
//   combine   out[t] = sum_j w[t][j] y[dest[t][j]]
//             -> dy[dest[t][j]] = w[t][j] dout[t]  (bf16, one RNE rounding)
//                dw[t][j] = <dout[t], y[dest[t][j]]>  (fp32)
//   dispatch  buf[dest[t][j]] = x[t]  -> dx[t] = sum_j dbuf[dest[t][j]]
//             (the combine kernel with unit weights, permute_combine.hip)
//   gate      w = softmax over the selected raw logits
//             -> dlogits[t][ids[t][j]] = w_j (dw_j - sum_j' w_j' dw_j'), 0 for
//                the experts not selected (the balancing bias only selects and
//                gets no gradient: "MoE load balancing: 90/10 routing in
//                production", editor's note).
#include "common.h"

namespace {

constexpr int kThreads = 256;

// One wavefront per token: the wave walks the row in 1 KB chunks (one
// 16-byte vector per lane: 8 bf16 or 4 fp32), writes the k scaled rows of dy
// and accumulates the k dot products per lane; a butterfly adds the lanes at
// the end, so dw does not depend on timing.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_backward_kernel(int T, int k, int64_t nrows,
                                                                    int row_vecs,
                                                                    const uint4* __restrict__ dout,
                                                                    const uint4* __restrict__ y,
                                                                    const int32_t* __restrict__ dest_row,
                                                                    const float* __restrict__ w,
                                                                    uint4* __restrict__ dy,
                                                                    float* __restrict__ dw)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (t >= T) return;
    int d = -1;
    float wl = 0.0f;
    if (lane < k) {
        const int dd = dest_row[(size_t)t * k + lane];
        d = (dd >= 0 && dd < nrows) ? dd : -1;
        wl = w[(size_t)t * k + lane];
    }
    float my_dw = 0.0f;  // lane j ends with dw[t][j]
    for (int j = 0; j < k; ++j) {
        const int dj = __builtin_amdgcn_readlane(d, j);
        const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), j));
        float acc = 0.0f;
        if (dj >= 0) {
            for (int c = lane; c < row_vecs; c += 64) {
                const uint4 g = dout[(size_t)t * row_vecs + c];
                const uint4 v = y[(size_t)dj * row_vecs + c];
                const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, vw[4] = {v.x, v.y, v.z, v.w};
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (BF16) {
                        const float g0 = __uint_as_float(gw[q] << 16), g1 = __uint_as_float(gw[q] & 0xffff0000u);
                        const float v0 = __uint_as_float(vw[q] << 16), v1 = __uint_as_float(vw[q] & 0xffff0000u);
                        acc = fmaf(g0, v0, acc);
                        acc = fmaf(g1, v1, acc);
                        o[q] = moe::pack_bf16x2(wj * g0, wj * g1);
                    } else {
                        const float g0 = __uint_as_float(gw[q]), v0 = __uint_as_float(vw[q]);
                        acc = fmaf(g0, v0, acc);
                        o[q] = __float_as_uint(wj * g0);
                    }
                }
                dy[(size_t)dj * row_vecs + c] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        // wave sum of the lanes' partial dot products (fixed order)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == j) my_dw = acc;
    }
    if (lane < k) dw[(size_t)t * k + lane] = my_dw;
}

// One thread per (token, expert).
__global__ __launch_bounds__(kThreads) void route_backward_kernel(int T, int E, int k,
                                                                  const int32_t* __restrict__ ids,
                                                                  const float* __restrict__ w,
                                                                  const float* __restrict__ dw,
                                                                  float* __restrict__ dlogits)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)T * E) return;
    const int t = (int)(i / E), e = (int)(i % E);
    const int32_t* it = ids + (size_t)t * k;
    const float* wt = w + (size_t)t * k;
    const float* dt = dw + (size_t)t * k;
    float dot = 0.0f, v = 0.0f;
    for (int j = 0; j < k; ++j) dot = fmaf(wt[j], dt[j], dot);
    for (int j = 0; j < k; ++j)
        if (it[j] == e) v = wt[j] * (dt[j] - dot);
    dlogits[i] = v;
}

}  // namespace

hipError_t moe_launch_combine_backward(const moe_shape_t& s, const void* dout, const void* y,
                                       const int32_t* dest_row, const float* w, void* dy,
                                       float* dw, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    const bool bf = s.dtype == MOE_BF16;
    const int row_vecs = s.H * (bf ? 2 : 4) / 16;
    const int grid = (s.T + kThreads / 64 - 1) / (kThreads / 64);
    const uint4* dv = static_cast<const uint4*>(dout);
    const uint4* yv = static_cast<const uint4*>(y);
    uint4* dyv = static_cast<uint4*>(dy);
    const int64_t nrows = (int64_t)s.T * s.k;
    if (bf)
        combine_backward_kernel<true><<<grid, kThreads, 0, st>>>(s.T, s.k, nrows, row_vecs, dv, yv,
                                                                 dest_row, w, dyv, dw);
    else
        combine_backward_kernel<false><<<grid, kThreads, 0, st>>>(s.T, s.k, nrows, row_vecs, dv, yv,
                                                                  dest_row, w, dyv, dw);
    return hipGetLastError();
}

hipError_t moe_launch_route_backward(const moe_shape_t& s, const int32_t* ids, const float* w,
                                     const float* dw, float* dlogits, hipStream_t st)
{
    const int64_t n = (int64_t)s.T * s.E;
    if (n == 0) return hipSuccess;
    route_backward_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        s.T, s.E, s.k, ids, w, dw, dlogits);
    return hipGetLastError();
}
