// route.hip -- router top-k gating on gfx950.
//
// "DeepEP-on-EFA Guidance, section 1", phase (a): each token scores every
// expert, keeps the k best and gets per-expert combine weights.
// "MoE load balancing: 90/10 routing in production", editor's note: the
// balancing bias steers selection only; the gate weights come from the raw
// logits.
//
// Mapping: a group of G lanes (G = the next power of two >= E, at most one
// wavefront; 32 above 64 experts with 4096 tokens or more and k <= 32) owns
// one token; lane l holds experts l, l+G, l+2G, ... in registers, so the row
// is read with unit-stride coalesced loads. Each of
// the k rounds takes a per-lane best among untaken experts and an all-reduce
// over the group (DPP moves and permlane swaps, no LDS) under the total order
// (score desc, id asc), so every lane agrees on the winner and its logit. After k rounds
// lane j of the group holds the j-th winner; the softmax over the selected
// raw logits is two more group reductions (max, sum). Scores compare by IEEE
// value (-0 == +0); a NaN never wins over a number.
#include <math.h>

#include "common.h"

namespace {

// Cross-lane steps without LDS: DPP moves inside rows of 16 lanes and the
// gfx950 permlane swaps across rows. For an all-reduce of a commutative op a
// partner from the other half of the current group is enough, so the
// mirrors stand in for xor 4 and xor 8 once the smaller groups are reduced.
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i in each 8
constexpr int kMirror = 0x140;      // lane i <-> 15-i in each 16

template <int CTRL>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, v)));
}

// a candidate: score, expert id, raw logit
struct Cand {
    float v;
    int id;
    float lg;
};

// the better of two under (score desc, id asc); equal keys are one expert
__device__ __forceinline__ Cand better(const Cand& a, const Cand& b)
{
    return (b.v > a.v || (b.v == a.v && b.id < a.id)) ? b : a;
}

template <int CTRL>
__device__ __forceinline__ Cand dpp(const Cand& c)
{
    return Cand{dpp<CTRL>(c.v), dpp<CTRL>(c.id), dpp<CTRL>(c.lg)};
}

// A copy the optimiser cannot see through. The permlane swaps below take the
// same value as both operands; the compiler was seen to treat the second
// half of such a swap as equal to the first and drop it, so each swap gets
// an opaque copy as its second operand.
__device__ __forceinline__ int opaque(int v)
{
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// the rows of 16 (ROWS32 false) or 32 lanes paired by a permlane swap: every
// lane gets {its own row's value, the paired row's value} in row order
template <bool ROWS32>
__device__ __forceinline__ void swap_halves(int v, int& lo, int& hi)
{
    if constexpr (ROWS32) {
        const auto s = __builtin_amdgcn_permlane32_swap(v, opaque(v), false, false);
        lo = (int)s[0];
        hi = (int)s[1];
    } else {
        const auto s = __builtin_amdgcn_permlane16_swap(v, opaque(v), false, false);
        lo = (int)s[0];
        hi = (int)s[1];
    }
}

template <bool ROWS32>
__device__ __forceinline__ Cand swap_best(const Cand& c)
{
    int v0, v1, i0, i1, l0, l1;
    swap_halves<ROWS32>(__builtin_bit_cast(int, c.v), v0, v1);
    swap_halves<ROWS32>(c.id, i0, i1);
    swap_halves<ROWS32>(__builtin_bit_cast(int, c.lg), l0, l1);
    return better(Cand{__builtin_bit_cast(float, v0), i0, __builtin_bit_cast(float, l0)},
                  Cand{__builtin_bit_cast(float, v1), i1, __builtin_bit_cast(float, l1)});
}

// every lane of a group of G (aligned) lanes gets the group's best candidate
template <int G>
__device__ __forceinline__ Cand group_best(Cand c)
{
    if constexpr (G >= 2) c = better(c, dpp<kQuadXor1>(c));
    if constexpr (G >= 4) c = better(c, dpp<kQuadXor2>(c));
    if constexpr (G >= 8) c = better(c, dpp<kHalfMirror>(c));
    if constexpr (G >= 16) c = better(c, dpp<kMirror>(c));
    if constexpr (G >= 32) c = swap_best<false>(c);
    if constexpr (G >= 64) c = swap_best<true>(c);
    return c;
}

template <bool SUM>
__device__ __forceinline__ float op(float a, float b)
{
    return SUM ? a + b : fmaxf(a, b);
}

template <bool SUM, bool ROWS32>
__device__ __forceinline__ float swap_op(float x)
{
    int lo, hi;
    swap_halves<ROWS32>(__builtin_bit_cast(int, x), lo, hi);
    return op<SUM>(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

// max or sum over a group; every lane gets the same value (each step is commutative)
template <int G, bool SUM>
__device__ __forceinline__ float group_reduce(float v)
{
    if constexpr (G >= 2) v = op<SUM>(v, dpp<kQuadXor1>(v));
    if constexpr (G >= 4) v = op<SUM>(v, dpp<kQuadXor2>(v));
    if constexpr (G >= 8) v = op<SUM>(v, dpp<kHalfMirror>(v));
    if constexpr (G >= 16) v = op<SUM>(v, dpp<kMirror>(v));
    if constexpr (G >= 32) v = swap_op<SUM, false>(v);
    if constexpr (G >= 64) v = swap_op<SUM, true>(v);
    return v;
}

// partial logit planes summed in plane order; the loads are issued together
constexpr int kMaxPlanes = 16;

__device__ __forceinline__ float plane_sum(const float* p, int nplanes, int64_t plane)
{
    float v[kMaxPlanes];
#pragma unroll
    for (int q = 0; q < kMaxPlanes; ++q) v[q] = q < nplanes ? p[q * plane] : 0.0f;
    float l = v[0];
#pragma unroll
    for (int q = 1; q < kMaxPlanes; ++q)
        if (q < nplanes) l += v[q];
    return l;
}

template <int G, int P>
__global__ __launch_bounds__(256) void route_kernel(int T, int E, int k,
                                                     const float* __restrict__ logits,
                                                     const float* __restrict__ bias,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ w, int32_t* err,
                                                     int nplanes, int64_t plane,
                                                     float* __restrict__ logits_out)
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
            // the router's K-range partials, summed in range order
            const float l = nplanes == 1 ? row[e] : plane_sum(row + e, nplanes, plane);
            if (logits_out) logits_out[(size_t)tok * E + e] = l;
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
        Cand c{-INFINITY, 0x7fffffff, 0.0f};
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int e = lane + p * G;
            if (!taken[p] && (sc[p] > c.v || (sc[p] == c.v && e < c.id))) c = Cand{sc[p], e, lg[p]};
        }
        const Cand b = group_best<G>(c);
        // the owner lane of the winner marks it taken
        if (c.id == b.id) {
#pragma unroll
            for (int p = 0; p < P; ++p)
                if (lane + p * G == b.id) taken[p] = true;
        }
        if (lane == j) {
            my_id = b.id;
            my_lg = b.lg;
        }
    }

    const bool sel = lane < k;
    const float m = group_reduce<G, false>(sel ? my_lg : -INFINITY);
    const float ex = sel ? expf(my_lg - m) : 0.0f;
    const float den = group_reduce<G, true>(ex);
    if (active && sel) {
        ids[(size_t)tok * k + lane] = my_id;
        w[(size_t)tok * k + lane] = ex / den;
    }
    // one atomic per wavefront that saw a non-finite input
    if (__any(bad) && (threadIdx.x & (moe::kWave - 1)) == 0) atomicOr(err, MOE_ERR_NONFINITE);
}

struct Planes {
    int n;
    int64_t stride;
    float* out;
};

template <int G, int P>
hipError_t launch(const moe_shape_t& s, const float* logits, const float* bias, int32_t* ids,
                  float* w, int32_t* err, hipStream_t st, const Planes& pl)
{
    const int per_block = 256 / G;
    const int blocks = (s.T + per_block - 1) / per_block;
    route_kernel<G, P><<<blocks, 256, 0, st>>>(s.T, s.E, s.k, logits, bias, ids, w, err, pl.n,
                                                pl.stride, pl.out);
    return hipGetLastError();
}

}  // namespace

hipError_t moe_launch_route(const moe_shape_t& s, const float* logits, const float* bias,
                            int32_t* ids, float* w, int32_t* err, hipStream_t st, int nplanes,
                            int64_t plane, float* logits_out)
{
    if (s.T == 0) return hipSuccess;
    const int E = s.E;
    const Planes pl{nplanes, plane, logits_out};
    if (E <= 1) return launch<1, 1>(s, logits, bias, ids, w, err, st, pl);
    if (E <= 2) return launch<2, 1>(s, logits, bias, ids, w, err, st, pl);
    if (E <= 4) return launch<4, 1>(s, logits, bias, ids, w, err, st, pl);
    if (E <= 8) return launch<8, 1>(s, logits, bias, ids, w, err, st, pl);
    if (E <= 16) return launch<16, 1>(s, logits, bias, ids, w, err, st, pl);
    if (E <= 32) return launch<32, 1>(s, logits, bias, ids, w, err, st, pl);
    if (E <= 64) return launch<64, 1>(s, logits, bias, ids, w, err, st, pl);
    // above 64 experts, many tokens: two tokens a wavefront, 32 lanes each
    // (measured 8-14 % faster at 4096 and 8192 tokens; at 1024 tokens a token
    // a wavefront is faster). Lane j of a group holds the j-th winner, so a
    // 32-lane group serves k <= 32 only; larger k keeps 64 lanes a token.
    if (s.T >= 4096 && s.k <= 32) {
        if (E <= 128) return launch<32, 4>(s, logits, bias, ids, w, err, st, pl);
        if (E <= 192) return launch<32, 6>(s, logits, bias, ids, w, err, st, pl);
        return launch<32, 8>(s, logits, bias, ids, w, err, st, pl);
    }
    if (E <= 128) return launch<64, 2>(s, logits, bias, ids, w, err, st, pl);
    if (E <= 192) return launch<64, 3>(s, logits, bias, ids, w, err, st, pl);
    return launch<64, 4>(s, logits, bias, ids, w, err, st, pl);
}
