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
// bf16 router GEMM. A workgroup (4 waves) owns a tile of TM = 32 or 64 tokens
// against all E (<= 256) experts, padded to EB = 32/64/128/256 rows, over one
// K-range (moe::router_split). K runs in 64-deep stages of whole 128-byte row
// lines through an LDS ring of up to 120 KB (global -> LDS copies, the same
// swizzle and waits as the expert GEMM); a small stage (8 KB at TM = EB = 32)
// leaves up to 15 stages in flight. The 32x32 output tiles are shared out so
// that every wave issues MFMAs: with four or more tiles each wave owns whole
// tiles; with fewer, the waves of a tile split its four 16-deep K slices and
// add their accumulators in wave order at the end. A stage's fragments are
// all read before its MFMAs, so LDS latency is paid once per stage.
// v_mfma_f32_32x32x16_bf16 takes the W_r fragment as its first operand, so a
// lane holds four consecutive experts of one token. With more than one
// K-range each range writes an fp32 partial plane that the top-k step sums.
#include "common.h"
#include "lds_pipe.h"

namespace {

using namespace moe::lds;

constexpr int kThreads = 256;
constexpr int kRK = 64;              // K per stage
constexpr int kRRing = 120 * 1024;   // LDS for the ring

template <int TM, int EB>
struct RouterTile {
    static constexpr int kTB = TM / 32;                          // token blocks
    static constexpr int kNB = EB / 32;                          // expert blocks
    static constexpr int kTiles = kTB * kNB;                     // 32x32 output tiles
    static constexpr int kKW = kTiles >= 4 ? 1 : 4 / kTiles;     // waves sharing a tile
    static constexpr int kTW = kTiles >= 4 ? kTiles / 4 : 1;     // tiles per wave
    static constexpr int kKK = 4 / kKW;                          // K slices per wave per stage
    static constexpr int kNBStep = kTiles >= 4 ? 4 / kTB : 0;    // expert-block step of a wave's tiles
    static constexpr int kA = TM * kRK * 2;                      // x bytes per stage
    static constexpr int kSlot = kA + EB * kRK * 2;
    static constexpr int kCopies = (TM + EB) / 32;               // copies per wave per stage
    static constexpr int kSlots = kRRing / kSlot < 16 ? kRRing / kSlot : 16;
    static_assert(kSlots >= 3 && (kSlots - 2) * kCopies < 64, "ring depth");
};

// wait until at most n (uniform, 0 <= n <= N) stages of C copies each remain in flight
template <int C, int N>
__device__ __forceinline__ void wait_stages(int n)
{
    if constexpr (N > 0) {
        if (n >= N) {
            wait_vm_lgkm<N * C>();
            return;
        }
        wait_stages<C, N - 1>(n);
    } else {
        wait_vm_lgkm<0>();
    }
}

template <int TM, int EB>
__global__ __launch_bounds__(kThreads, 1) void router_gemm_kernel(int T, int E, int H, int KTp,
                                                                  const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr,
                                                                  float* __restrict__ out)
{
    using P = RouterTile<TM, EB>;
    __shared__ __attribute__((aligned(1024))) char ring[P::kSlots * P::kSlot];

    const int KT = H / kRK;
    const int t0 = blockIdx.x * TM;
    const int s0 = blockIdx.y * KTp;
    const int ns = min(KT, s0 + KTp) - s0;  // >= 1: the launcher makes no empty range
    float* outp = out + (size_t)blockIdx.y * T * E;
    const int tid = threadIdx.x;
    const int wave = uni(tid >> 6), lane = tid & 63;
    const int fr = lane & 31, fh = lane >> 5;
    const uint32_t ring_u = (uint32_t)(uintptr_t)ring;
    const char* xb = uni_ptr(reinterpret_cast<const char*>(x) + (size_t)s0 * kRK * 2);
    const char* wb = uni_ptr(reinterpret_cast<const char*>(wr) + (size_t)s0 * kRK * 2);

    // copy sources: tile row 32 i + 8 wave + lane / 8 (token clamped to T-1,
    // expert to E-1), K-chunk lane % 8 stored at its swizzled slot
    uint32_t aoff[P::kTB], boff[P::kNB];
#pragma unroll
    for (int i = 0; i < P::kTB; ++i) {
        const int r = 32 * i + 8 * wave + (lane >> 3);
        const uint32_t ch = (uint32_t)(((lane & 7) ^ swz(r)) * 16);
        aoff[i] = (uint32_t)min(t0 + r, T - 1) * (uint32_t)H * 2u + ch;
    }
#pragma unroll
    for (int i = 0; i < P::kNB; ++i) {
        const int r = 32 * i + 8 * wave + (lane >> 3);
        const uint32_t ch = (uint32_t)(((lane & 7) ^ swz(r)) * 16);
        boff[i] = (uint32_t)min(r, E - 1) * (uint32_t)H * 2u + ch;
    }
    auto copy_stage = [&](int j) {
        const uint32_t slot = ring_u + (uint32_t)(j % P::kSlots) * P::kSlot;
#pragma unroll
        for (int i = 0; i < P::kTB; ++i) copy16(xb + j * (kRK * 2), aoff[i], slot + i * 4096 + wave * 1024);
#pragma unroll
        for (int i = 0; i < P::kNB; ++i)
            copy16(wb + j * (kRK * 2), boff[i], slot + P::kA + i * 4096 + wave * 1024);
    };

    // this wave's work: token block tb, expert blocks nb0 + i * kNBStep
    // (i < kTW), K slices kk0 .. kk0 + kKK - 1 of every stage
    int tb, nb0, kk0;
    if constexpr (P::kTiles >= 4) {
        tb = wave % P::kTB;
        nb0 = wave / P::kTB;
        kk0 = 0;
    } else {
        const int tile = wave / P::kKW;
        tb = tile % P::kTB;
        nb0 = tile / P::kTB;
        kk0 = (wave % P::kKW) * P::kKK;
    }
    uint32_t fa[P::kKK], fb[P::kKK];
#pragma unroll
    for (int kk = 0; kk < P::kKK; ++kk) {
        const uint32_t ch = (uint32_t)(((2 * (kk0 + kk) + fh) ^ swz(fr)) * 16);
        fa[kk] = (uint32_t)(32 * tb + fr) * 128u + ch;
        fb[kk] = (uint32_t)P::kA + (uint32_t)(32 * nb0 + fr) * 128u + ch;
    }

    f32x16 acc[P::kTW];
#pragma unroll
    for (int i = 0; i < P::kTW; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][q] = 0.0f;
    constexpr int kAhead = P::kSlots - 1;
    for (int j = 0; j < kAhead && j < ns; ++j) copy_stage(j);
    for (int j = 0; j < ns; ++j) {
        // stage j landed; stages j+1 .. (at most kAhead-1 of them) may stay in flight
        wait_stages<P::kCopies, kAhead - 1>(min(kAhead - 1, ns - 1 - j));
        slot_barrier();  // ... in every wave; and stage j-1's slot is free
        if (j + kAhead < ns) copy_stage(j + kAhead);
        const char* slot = ring + (j % P::kSlots) * P::kSlot;
        bf16x8 af[P::kKK], bfr[P::kKK][P::kTW];
#pragma unroll
        for (int kk = 0; kk < P::kKK; ++kk) {
            af[kk] = lds_frag(slot + fa[kk]);
#pragma unroll
            for (int i = 0; i < P::kTW; ++i)
                bfr[kk][i] = lds_frag(slot + fb[kk] + i * P::kNBStep * 32 * 128);
        }
#pragma unroll
        for (int kk = 0; kk < P::kKK; ++kk)
#pragma unroll
            for (int i = 0; i < P::kTW; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk][i], af[kk], acc[i], 0, 0, 0);
    }

    bool lead = true;
    if constexpr (P::kKW > 1) {
        // the waves of a tile add their K-slice accumulators in wave order
        slot_barrier();  // every wave is done with the ring
        float4* red = reinterpret_cast<float4*>(ring);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            red[(wave * 64 + lane) * 4 + q] =
                make_float4(acc[0][4 * q], acc[0][4 * q + 1], acc[0][4 * q + 2], acc[0][4 * q + 3]);
        __syncthreads();
        lead = wave % P::kKW == 0;
        if (lead) {
#pragma unroll
            for (int w2 = 1; w2 < P::kKW; ++w2)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = red[((wave + w2) * 64 + lane) * 4 + q];
                    acc[0][4 * q] += v.x;
                    acc[0][4 * q + 1] += v.y;
                    acc[0][4 * q + 2] += v.z;
                    acc[0][4 * q + 3] += v.w;
                }
        }
    }
    // acc[i][4 g4 + q]: token t0 + 32 tb + fr, expert 32 (nb0 + i kNBStep) + 8 g4 + 4 fh + q
    const int t = t0 + 32 * tb + fr;
    if (!lead || t >= T) return;
    const bool vec = (E & 3) == 0;
#pragma unroll
    for (int i = 0; i < P::kTW; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int e0 = 32 * (nb0 + i * P::kNBStep) + 8 * g4 + 4 * fh;
            float* o = outp + (size_t)t * E + e0;
            if (vec && e0 + 3 < E) {
                *reinterpret_cast<float4*>(o) = make_float4(acc[i][4 * g4], acc[i][4 * g4 + 1],
                                                            acc[i][4 * g4 + 2], acc[i][4 * g4 + 3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (e0 + q < E) o[q] = acc[i][4 * g4 + q];
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

namespace {

template <int TM, int EB>
void launch_router(const moe_shape_t& s, const moe::RouterSplit& sp, const uint16_t* x,
                   const uint16_t* w, float* out, hipStream_t st)
{
    const dim3 grid((s.T + TM - 1) / TM, sp.parts);
    router_gemm_kernel<TM, EB><<<grid, kThreads, 0, st>>>(s.T, s.E, s.H, sp.kt_part, x, w, out);
}

template <int TM>
void launch_router_eb(const moe_shape_t& s, const moe::RouterSplit& sp, const uint16_t* x,
                      const uint16_t* w, float* out, hipStream_t st)
{
    if (s.E <= 32) launch_router<TM, 32>(s, sp, x, w, out, st);
    else if (s.E <= 64) launch_router<TM, 64>(s, sp, x, w, out, st);
    else if (s.E <= 128) launch_router<TM, 128>(s, sp, x, w, out, st);
    else launch_router<TM, 256>(s, sp, x, w, out, st);
}

}  // namespace

hipError_t moe_launch_router_logits(const moe_shape_t& s, const void* x, const void* w_router,
                                    float* logits, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    if (s.dtype == MOE_BF16) {
        const moe::RouterSplit sp = moe::router_split(s);
        const uint16_t* xv = static_cast<const uint16_t*>(x);
        const uint16_t* wv = static_cast<const uint16_t*>(w_router);
        if (sp.tm == 64) launch_router_eb<64>(s, sp, xv, wv, logits, st);
        else launch_router_eb<32>(s, sp, xv, wv, logits, st);
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
