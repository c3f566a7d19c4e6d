// router.hip -- the router's scores and the bias update.
//
// "DeepEP-on-EFA Guidance, section 1", phase (a): the router scores every
// expert for every token, then the top-k step (route.hip) keeps the k best.
// The pages do not print the router itself; the plain reading is a linear
// layer: logits[t][e] = sum_h x[t][h] * W_r[e][h], accumulated in fp32.
// Bias update: NOT ON THE PAGES (an assumption). "MoE load balancing: 90/10
// routing in production" keeps a per-expert balancing bias out of the gate
// but prints no update rule; the sign rule of auxiliary-loss-free balancing is
// used: above-mean experts lose gamma, below-mean ones gain gamma.
//
// bf16 router GEMM: one 256-thread workgroup per 32 tokens; all E (<= 256)
// experts in one tile of EB = E rounded up to 32/64/128/256 rows; K in
// 64-deep stages of whole 128-byte row lines through an LDS ring of up to
// 120 KB (global -> LDS copies, the same swizzle and waits as the expert
// GEMM): a stage is 8 KB for EB = 32, so 15 stages can be in flight -- the
// few workgroups of a small router are bound by copy latency, not bytes;
// v_mfma_f32_32x32x16_bf16 with wave w owning experts 64w .. 64w+63. The
// fp32 logits are written once and read by the top-k kernel.
#include "common.h"
#include "lds_pipe.h"

namespace {

using namespace moe::lds;

constexpr int kThreads = 256;
constexpr int kRM = 32;              // tokens per tile
constexpr int kRK = 64;              // K per stage
constexpr int kRA = kRM * kRK * 2;   // 4 KB of x per stage
constexpr int kRRing = 120 * 1024;   // LDS for the ring

template <int EB>
__global__ __launch_bounds__(kThreads, 1) void router_gemm_kernel(int T, int E, int H,
                                                                  const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr,
                                                                  float* __restrict__ logits)
{
    constexpr int kSlot = kRA + EB * kRK * 2;
    constexpr int kRSlots = kRRing / kSlot < 16 ? kRRing / kSlot : 16;
    constexpr int kBCopies = EB / 32;          // B copy instructions per wave per stage
    constexpr int kPerStage = 1 + kBCopies;    // copies per wave per stage
    static_assert((kRSlots - 2) * kPerStage < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char ring[kRSlots * kSlot];

    const int KT = H / kRK;
    const int t0 = blockIdx.x * kRM;
    const int tid = threadIdx.x;
    const int wave = uni(tid >> 6), lane = tid & 63;
    const int fr = lane & 31, fh = lane >> 5;
    const uint32_t ring_u = (uint32_t)(uintptr_t)ring;
    const char* xb = uni_ptr(reinterpret_cast<const char*>(x));
    const char* wb = uni_ptr(reinterpret_cast<const char*>(wr));

    // copy sources: x rows 8 wave + lane / 8 of the tile (token clamped to
    // T-1); W_r rows 8q + lane / 8 for q = wave + 4 i (expert clamped to E-1)
    uint32_t aoff, boff[kBCopies];
    {
        const int r = 8 * wave + (lane >> 3);
        const uint32_t ch = (uint32_t)(((lane & 7) ^ swz(r)) * 16);
        aoff = (uint32_t)min(t0 + r, T - 1) * (uint32_t)H * 2u + ch;
    }
#pragma unroll
    for (int i = 0; i < kBCopies; ++i) {
        const int r = 8 * (wave + 4 * i) + (lane >> 3);
        const uint32_t ch = (uint32_t)(((lane & 7) ^ swz(r)) * 16);
        boff[i] = (uint32_t)min(r, E - 1) * (uint32_t)H * 2u + ch;
    }
    auto copy_stage = [&](int st) {
        const uint32_t slot = ring_u + (uint32_t)(st % kRSlots) * kSlot;
        copy16(xb + st * (kRK * 2), aoff, slot + wave * 1024);
#pragma unroll
        for (int i = 0; i < kBCopies; ++i)
            copy16(wb + st * (kRK * 2), boff[i], slot + kRA + wave * 1024 + i * 4096);
    };
    // fragments: x rows fr; W_r rows 64 wave + 32 j + fr
    uint32_t fa[4], fb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint32_t ch = (uint32_t)(((2 * kk + fh) ^ swz(fr)) * 16);
        fa[kk] = (uint32_t)fr * 128u + ch;
        fb[kk] = (uint32_t)kRA + (uint32_t)(64 * wave + fr) * 128u + ch;
    }
    const int nb = min(2, max(0, (EB - 64 * wave) / 32));  // this wave's 32-expert blocks

    f32x16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;
    constexpr int kAhead = kRSlots - 1;
    for (int st = 0; st < kAhead && st < KT; ++st) copy_stage(st);
    for (int s = 0; s < KT; ++s) {
        // stage s landed: the copies of stages s+1 .. s+kAhead-1 may stay in
        // flight (all of them exist away from the end of K; near it, wait for all)
        if (s + kAhead - 1 < KT) wait_vm_lgkm<(kAhead - 1) * kPerStage>();
        else wait_vm_lgkm<0>();
        slot_barrier();  // ... in every wave; and stage s-1's slot is free
        if (s + kAhead < KT) copy_stage(s + kAhead);
        const char* slot = ring + (s % kRSlots) * kSlot;
        if (nb > 0) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 af = lds_frag(slot + fa[kk]);
                const bf16x8 b0 = lds_frag(slot + fb[kk]);
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, af, acc[0], 0, 0, 0);
                if (nb > 1) {
                    const bf16x8 b1 = lds_frag(slot + fb[kk] + 32 * 128);
                    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, af, acc[1], 0, 0, 0);
                }
            }
        }
    }
    // acc[j][4 g4 + q]: token t0 + (lane & 31), expert 64 wave + 32 j + 8 g4 + 4 (lane >> 5) + q
    const int t = t0 + fr;
    if (t < T) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int e = 64 * wave + 32 * j + 8 * g4 + 4 * fh + q;
                    if (j < nb && e < E) logits[(size_t)t * E + e] = acc[j][g4 * 4 + q];
                }
    }
}

// fp32 router (small shapes): one thread per (token, expert), fp32 FMA in h order.
__global__ __launch_bounds__(kThreads) void router_f32_kernel(int T, int E, int H,
                                                              const float* __restrict__ x,
                                                              const float* __restrict__ wr,
                                                              float* __restrict__ logits)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)T * E) return;
    const int t = (int)(i / E), e = (int)(i % E);
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) acc = fmaf(x[(size_t)t * H + h], wr[(size_t)e * H + h], acc);
    logits[i] = acc;
}

// Sign-rule bias update (an assumption, see above): delta = +-gamma or 0 from
// the sign of N - E * counts[e], in integers; one fp32 add.
__global__ __launch_bounds__(kThreads) void bias_update_kernel(int E, int64_t N,
                                                               const int32_t* __restrict__ counts,
                                                               float gamma, float* __restrict__ bias)
{
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= E) return;
    const int64_t s = N - (int64_t)E * counts[e];
    const float delta = s > 0 ? gamma : (s < 0 ? -gamma : 0.0f);
    bias[e] = bias[e] + delta;
}

}  // namespace

hipError_t moe_launch_router_logits(const moe_shape_t& s, const void* x, const void* w_router,
                                    float* logits, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    if (s.dtype == MOE_BF16) {
        const int grid = (s.T + kRM - 1) / kRM;
        const uint16_t* xv = static_cast<const uint16_t*>(x);
        const uint16_t* wv = static_cast<const uint16_t*>(w_router);
        if (s.E <= 32)
            router_gemm_kernel<32><<<grid, kThreads, 0, st>>>(s.T, s.E, s.H, xv, wv, logits);
        else if (s.E <= 64)
            router_gemm_kernel<64><<<grid, kThreads, 0, st>>>(s.T, s.E, s.H, xv, wv, logits);
        else if (s.E <= 128)
            router_gemm_kernel<128><<<grid, kThreads, 0, st>>>(s.T, s.E, s.H, xv, wv, logits);
        else
            router_gemm_kernel<256><<<grid, kThreads, 0, st>>>(s.T, s.E, s.H, xv, wv, logits);
    } else {
        const int64_t n = (int64_t)s.T * s.E;
        router_f32_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(
            s.T, s.E, s.H, static_cast<const float*>(x), static_cast<const float*>(w_router),
            logits);
    }
    return hipGetLastError();
}

hipError_t moe_launch_bias_update(const moe_shape_t& s, const int32_t* counts, float gamma,
                                  float* bias, hipStream_t st)
{
    bias_update_kernel<<<(s.E + kThreads - 1) / kThreads, kThreads, 0, st>>>(
        s.E, (int64_t)s.T * s.k, counts, gamma, bias);
    return hipGetLastError();
}
