// route.hip -- router top-k gating on gfx950.
//
// "DeepEP-on-EFA Guidance, section 1", phase (a): each token scores every
// expert, keeps the k best and gets per-expert combine weights.
// "MoE load balancing: 90/10 routing in production", editor's note: the
// balancing bias steers selection only; the gate weights come from the raw
// logits.
//
// Mapping: a group of G lanes (G = the next power of two >= E, at most one
// wavefront) owns one token; lane l holds experts l, l+G, l+2G, ... in
// registers, so the row is read with unit-stride coalesced loads. Each of
// the k rounds takes a per-lane best among untaken experts and a butterfly
// (xor-shuffle) argmax over the group under the total order
// (score desc, id asc), so every lane agrees on the winner. After k rounds
// lane j of the group holds the j-th winner; the softmax over the selected
// raw logits is a second pair of group reductions. Scores compare by IEEE
// value (-0 == +0); a NaN never wins over a number.
#include <math.h>

#include "common.h"

namespace {

template <int G>
__device__ __forceinline__ void group_argmax(float& v, int& id)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
        const float ov = __shfl_xor(v, off, G);
        const int oi = __shfl_xor(id, off, G);
        if (ov > v || (ov == v && oi < id)) {
            v = ov;
            id = oi;
        }
    }
}

template <int G>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, G));
    return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, G);
    return v;
}

template <int G, int P>
__global__ __launch_bounds__(256) void route_kernel(int T, int E, int k,
                                                     const float* __restrict__ logits,
                                                     const float* __restrict__ bias,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ w, int32_t* err)
{
    const int lane = threadIdx.x & (G - 1);
    const int tok = blockIdx.x * (blockDim.x / G) + threadIdx.x / G;
    const bool active = tok < T;
    const float* row = logits + (size_t)(active ? tok : 0) * E;

    float lg[P], sc[P];
    bool taken[P];
    bool bad = false;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int e = lane + p * G;
        if (active && e < E) {
            const float l = row[e];
            const float b = bias ? bias[e] : 0.0f;
            bad |= !isfinite(l) || !isfinite(b);
            lg[p] = l;
            const float s = l + b;  // one fp32 add, round to nearest even
            sc[p] = isnan(s) ? -INFINITY : s;
            taken[p] = false;
        } else {
            lg[p] = 0.0f;
            sc[p] = -INFINITY;
            taken[p] = true;
        }
    }

    int my_id = 0;
    float my_lg = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        float bl = 0.0f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int e = lane + p * G;
            if (!taken[p] && (sc[p] > bv || (sc[p] == bv && e < bi))) {
                bv = sc[p];
                bi = e;
                bl = lg[p];
            }
        }
        const int cand = bi;
        group_argmax<G>(bv, bi);
        // the owner lane of the winner supplies its raw logit
        const float wl = __shfl(bl, bi & (G - 1), G);
        if (cand == bi) {
#pragma unroll
            for (int p = 0; p < P; ++p)
                if (lane + p * G == bi) taken[p] = true;
        }
        if (lane == j) {
            my_id = bi;
            my_lg = wl;
        }
    }

    const bool sel = lane < k;
    const float m = group_max<G>(sel ? my_lg : -INFINITY);
    const float ex = sel ? expf(my_lg - m) : 0.0f;
    const float den = group_sum<G>(ex);
    if (active && sel) {
        ids[(size_t)tok * k + lane] = my_id;
        w[(size_t)tok * k + lane] = ex / den;
    }
    // one atomic per wavefront that saw a non-finite input
    if (__any(bad) && (threadIdx.x & (moe::kWave - 1)) == 0) atomicOr(err, MOE_ERR_NONFINITE);
}

template <int G, int P>
hipError_t launch(const moe_shape_t& s, const float* logits, const float* bias, int32_t* ids,
                  float* w, int32_t* err, hipStream_t st)
{
    const int per_block = 256 / G;
    const int blocks = (s.T + per_block - 1) / per_block;
    route_kernel<G, P><<<blocks, 256, 0, st>>>(s.T, s.E, s.k, logits, bias, ids, w, err);
    return hipGetLastError();
}

}  // namespace

hipError_t moe_launch_route(const moe_shape_t& s, const float* logits, const float* bias,
                            int32_t* ids, float* w, int32_t* err, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    const int E = s.E;
    if (E <= 1) return launch<1, 1>(s, logits, bias, ids, w, err, st);
    if (E <= 2) return launch<2, 1>(s, logits, bias, ids, w, err, st);
    if (E <= 4) return launch<4, 1>(s, logits, bias, ids, w, err, st);
    if (E <= 8) return launch<8, 1>(s, logits, bias, ids, w, err, st);
    if (E <= 16) return launch<16, 1>(s, logits, bias, ids, w, err, st);
    if (E <= 32) return launch<32, 1>(s, logits, bias, ids, w, err, st);
    if (E <= 64) return launch<64, 1>(s, logits, bias, ids, w, err, st);
    if (E <= 128) return launch<64, 2>(s, logits, bias, ids, w, err, st);
    if (E <= 192) return launch<64, 3>(s, logits, bias, ids, w, err, st);
    return launch<64, 4>(s, logits, bias, ids, w, err, st);
}
