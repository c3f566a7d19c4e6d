// gemm.hip -- the grouped SwiGLU expert GEMM over the plan.
//
// "DeepEP-on-EFA Guidance, section 1", phase (c): every expert runs its FFN
// over the rows it received, as a batched grouped GEMM.
// "Moonshot AI drops MoonEP ..." paragraph 3: one contiguous weight tensor
// per projection ([E][F][H] gate and up, [E][H][F] down); replicas of an
// expert read the same slice (one GPU holds every expert).
//
// Rows of expert e are its pieces in rank order, i.e. the virtual rows
// v = 0 .. c_e-1 map to buf rows piece_row[p] + (v - cum_p). M-tiles are cut
// per expert over these virtual rows (not per piece), so a replica split
// costs no extra tile. A device-side schedule (prefix of per-expert tile
// counts) lets a static grid find its tile with no host round trip.
//
// Two launches:
//   gate/up: h[row_start[e] + v][f] = silu(a_v . Wg[e][f]) * (a_v . Wu[e][f])
//            (h stored expert-contiguous, rounded to bf16 in bf16 mode);
//   down:    y[buf row of v][o] = h[row_start[e] + v] . Wd[e][o].
// bf16 path: a persistent MFMA kernel (below); fp32 path: plain LDS-tiled
// VALU kernels for small shapes.
#include <type_traits>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// plain vector (not HIP's struct uint4) so staging arrays promote to registers
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// schedule layout inside the workspace region (int32):
//   [0 .. E]        tile_start (prefix of ceil(c_e / BM))
//   [E+1 .. 2E+1]   row_start  (prefix of c_e)
__global__ __launch_bounds__(kThreads) void schedule_kernel(int E, int R, int bm,
                                                            const int32_t* __restrict__ plan,
                                                            int32_t* __restrict__ sched)
{
    __shared__ int32_t st[256], sr[256];
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int e = threadIdx.x;
    int c = 0;
    if (e < E) {
        const int np = plan[L.piece_num + e];
        for (int p = 0; p < np && p < R; ++p) c += plan[L.piece_cnt + (size_t)e * R + p];
    }
    st[e] = (c + bm - 1) / bm;
    sr[e] = c;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int a = e >= off ? st[e - off] : 0;
        const int b = e >= off ? sr[e - off] : 0;
        __syncthreads();
        st[e] += a;
        sr[e] += b;
        __syncthreads();
    }
    if (e < E) {
        sched[e + 1] = st[e];
        sched[E + 1 + e + 1] = sr[e];
    }
    if (e == 0) {
        sched[0] = 0;
        sched[E + 1] = 0;
    }
}

// vrow[g] = buf row of the g-th row in expert-sorted order (expert e owns
// g in [row_start[e], row_start[e+1]); its v-th row lives in the piece that
// covers v, pieces taken in rank order).
__global__ __launch_bounds__(kThreads) void vrow_kernel(int N, int E, int R,
                                                        const int32_t* __restrict__ plan,
                                                        const int32_t* __restrict__ sched,
                                                        int32_t* __restrict__ vrow)
{
    const int g = blockIdx.x * kThreads + threadIdx.x;
    if (g >= N) return;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int32_t* row_start = sched + E + 1;
    int lo = 0, hi = E - 1;  // last expert with row_start <= g
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (row_start[mid] <= g) lo = mid;
        else hi = mid - 1;
    }
    const int v = g - row_start[lo];
    const int np = plan[L.piece_num + lo];
    int cum = 0, row = 0;
    for (int p = 0; p < np && p < R; ++p) {
        const int c = plan[L.piece_cnt + (size_t)lo * R + p];
        if (v < cum + c) {
            row = plan[L.piece_row + (size_t)lo * R + p] + (v - cum);
            break;
        }
        cum += c;
    }
    vrow[g] = row;
}

struct Tile {
    int e, v0, rows, hrow0;  // expert, first virtual row, rows in tile, h row of v0
};

// Finds the tile of M-tile index mt; rows == 0 if past the end.
__device__ __forceinline__ Tile find_tile(int mt, int E, int bm, const int32_t* sched)
{
    Tile t{0, 0, 0, 0};
    if (mt >= sched[E]) return t;
    int lo = 0, hi = E - 1;  // largest e with tile_start[e] <= mt
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sched[mid] <= mt) lo = mid;
        else hi = mid - 1;
    }
    const int c = sched[E + 1 + lo + 1] - sched[E + 1 + lo];
    t.e = lo;
    t.v0 = (mt - sched[lo]) * bm;
    t.rows = min(bm, c - t.v0);
    t.hrow0 = sched[E + 1 + lo] + t.v0;
    return t;
}

// Virtual row v of expert e -> buf row (walks at most R pieces).
__device__ __forceinline__ int buf_row_of(int e, int v, int R, const int32_t* plan,
                                          const moe::PlanLayout& L)
{
    const int np = plan[L.piece_num + e];
    int cum = 0;
    for (int p = 0; p < np && p < R; ++p) {
        const int c = plan[L.piece_cnt + (size_t)e * R + p];
        if (v < cum + c) return plan[L.piece_row + (size_t)e * R + p] + (v - cum);
        cum += c;
    }
    return 0;
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- bf16 ----
// Persistent kernel, one 256-thread workgroup per CU. Workgroup tile: 256
// rows x 256 B-rows (gate/up: 128 F-columns of gate and the same 128 of up;
// down: 256 output columns); K in 64-deep stages, two LDS buffers per operand.
//  * Global -> LDS with global_load_lds_dwordx4 (lane l of an instruction
//    lands at its LDS base + 16 l): tiles never pass through VGPRs. A stage
//    buffer is 256 rows of 9 16-byte slots (8 K-chunks + 1 pad = 144-byte
//    rows), which keeps the MFMA fragment reads (32 consecutive rows, one
//    chunk) free of bank conflicts; pad slots receive a harmless copy.
//    Every DMA source is a wave-uniform base plus a fixed 32-bit lane offset.
//  * 4 waves in 2 x 2, each 128 rows x 128 B-rows with
//    v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane, in AGPRs).
//    Operands are swapped so a lane holds 4 consecutive output columns: the
//    epilogue stores 8 bytes per lane straight to global memory.
//  * Software pipeline per stage s: fragments of k-step kk+1 are read while
//    the MFMAs of kk run; the barrier sits before the last k-step's MFMAs;
//    after it the buffer stage s used is refilled with stage s+2 and the next
//    stage's first fragments are read under those MFMAs.
//  * Tile order: expert, N-tile, M-tile (M fastest), so the M-tiles sharing
//    a weight tile run together; each XCD takes a contiguous run of tiles so
//    they share its L2.
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kSlotsPerRow = kTK / 8 + 1;            // 8 K-chunks + 1 pad slot (16 bytes each)
constexpr int kRowElems = kSlotsPerRow * 8;          // 72 bf16 = 144 bytes per LDS row
constexpr int kStageElems = kTM * kRowElems;         // 36 KB per A or B stage buffer
constexpr int kDmaPerStage = kTM * kSlotsPerRow / 64; // 36 DMA instructions per operand
constexpr int kDmaPerWave = kDmaPerStage / 4;        // 9
constexpr int kGateDma = 128 * kSlotsPerRow / 64;    // instructions 0..17 hold gate rows
enum { kGateUp = 0, kDown = 1 };

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// global -> LDS, 16 bytes per lane; lane l of the wave lands at l_base + 16 l
__device__ __forceinline__ void dma16(const void* g, uint16_t* l_base)
{
    __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)l_base, 16, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(
    int E, int ntiles_n, int H, int F, int ksplit, int N, const uint16_t* __restrict__ a_src,
    const int32_t* __restrict__ sched, const int32_t* __restrict__ vrow,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, uint16_t* __restrict__ out,
    float* __restrict__ part)
{
    __shared__ __attribute__((aligned(16))) uint16_t sA0[kStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t sA1[kStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t sB0[kStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t sB1[kStageElems];
    __shared__ int32_t rowmap[kTM];
    __shared__ int32_t ssched[2 * 257];  // tile_start[E+1], row_start[E+1]

    for (int i = threadIdx.x; i < 2 * (E + 1); i += kThreads) ssched[i] = sched[i];
    __syncthreads();
    const int K = MODE == kGateUp ? H : F;
    const int KT_all = K / kTK;
    const int KT_half = (KT_all + ksplit - 1) / ksplit;
    const int total = ssched[E] * ntiles_n * ksplit;
    const int P = gridDim.x;
    const int per_xcd = P / 8;
    const int my_slot = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int fl = lane & 31, fh = lane >> 5;
    const int frag_off = fl * kRowElems + fh * 8;      // fragment row, K-chunk

    for (int base = 0;; base += P) {
        const int Lu = base + my_slot;
        if (Lu >= total) break;
        // ---- decode the work unit: K-part (split-K), then the tile: expert,
        // N-tile, M-tile
        const int Lt = Lu / ksplit, kpart = Lu % ksplit;
        const int KT = min(KT_all, (kpart + 1) * KT_half) - kpart * KT_half;
        const int kofs = kpart * KT_half * kTK;
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ssched[mid] * ntiles_n <= Lt) lo = mid;
            else hi = mid - 1;
        }
        const int e = lo;
        const int mt_e = ssched[e + 1] - ssched[e];
        const int local = Lt - ssched[e] * ntiles_n;
        const int nt = local / mt_e, mt = local % mt_e;
        const int c_e = ssched[E + 1 + e + 1] - ssched[E + 1 + e];
        const int v0 = mt * kTM;
        const int rows = min(kTM, c_e - v0);
        const int hrow0 = ssched[E + 1 + e] + v0;
        rowmap[tid] = vrow[hrow0 + (tid < rows ? tid : 0)];
        __syncthreads();

        // ---- DMA sources. Stage buffer = 256 rows x 9 slots; DMA instruction
        // q (0..35) fills slots 64q .. 64q+63, lane l slot 64q + l, i.e. row
        // (64q+l)/9, slot (64q+l)%9 (slot 8 is the pad: it gets the row's
        // chunk 0, never read). Wave w issues instructions q = 4i + w. Each
        // source is a wave-uniform base plus a fixed 32-bit lane offset.
        const int n0 = nt * (MODE == kGateUp ? kTN / 2 : kTN);
        const char* abase = reinterpret_cast<const char*>(
            (MODE == kGateUp ? a_src : a_src + (size_t)hrow0 * F) + kofs);
        const char* bbase0 = reinterpret_cast<const char*>(
            (MODE == kGateUp ? w0 + (size_t)e * F * H : w0 + (size_t)e * H * F) + kofs);
        const char* bbase1 = MODE == kGateUp ? reinterpret_cast<const char*>(w1 + (size_t)e * F * H + kofs)
                                             : bbase0;
        uint32_t aoff[kDmaPerWave], boff[kDmaPerWave];
#pragma unroll
        for (int i = 0; i < kDmaPerWave; ++i) {
            const int slot = 64 * (4 * i + wave) + lane;
            const int r = slot / kSlotsPerRow, c = slot % kSlotsPerRow;
            const uint32_t chunk = (c < 8 ? c : 0) * 16;
            if (MODE == kGateUp) {
                aoff[i] = (uint32_t)rowmap[r] * (uint32_t)H * 2u + chunk;
                const int f = min(n0 + (r & 127), F - 1);   // rows 0..127 gate, 128..255 up
                boff[i] = (uint32_t)f * (uint32_t)H * 2u + chunk;
            } else {
                aoff[i] = (uint32_t)min(r, rows - 1) * (uint32_t)F * 2u + chunk;
                const int o = min(n0 + r, H - 1);
                boff[i] = (uint32_t)o * (uint32_t)F * 2u + chunk;
            }
        }
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

        auto issue = [&](uint16_t* sA, uint16_t* sB, int k0) {
            const char* ab = abase + (size_t)k0 * 2;
            const char* b0 = bbase0 + (size_t)k0 * 2;
            const char* b1 = bbase1 + (size_t)k0 * 2;
#pragma unroll
            for (int i = 0; i < kDmaPerWave; ++i) {
                const int q = 4 * i + wave_u;
                dma16(ab + aoff[i], sA + q * 512);
                dma16((q < kGateDma ? b0 : b1) + boff[i], sB + q * 512);
            }
        };
        auto frags = [&](const uint16_t* sA, const uint16_t* sB, int kk, bf16x8* af, bf16x8* bf) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = lds_frag(sA + frag_off + (wm * 128 + i * 32) * kRowElems + kk * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r0 = MODE == kGateUp ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32)
                                               : (wn * 128 + j * 32);
                bf[j] = lds_frag(sB + frag_off + r0 * kRowElems + kk * 16);
            }
        };
        auto mfmas = [&](const bf16x8* af, const bf16x8* bf) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
        };

        bf16x8 af[2][4], bf[2][4];
        // One stage on buffer c while n holds the next one. REFILL: refill c
        // with stage s_+2 right after the barrier that retires c's reads, its
        // DMA instructions threaded between the last k-step's MFMAs (the caller
        // guarantees s_+2 < KT). Otherwise no refill.
        auto stage = [&](auto refill, uint16_t* cA, uint16_t* cB, uint16_t* nA, uint16_t* nB,
                         int s_) {
            constexpr bool REFILL = decltype(refill)::value;
#pragma unroll
            for (int kk = 0; kk < 3; ++kk) {
                frags(cA, cB, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mfmas(af[kk & 1], bf[kk & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA into n has landed
            __syncthreads();                // all of n landed; everyone is done reading c
            if (s_ + 1 < KT) frags(nA, nB, 0, af[0], bf[0]);
            __builtin_amdgcn_sched_barrier(0);
            if (REFILL) issue(cA, cB, (s_ + 2) * kTK);
            mfmas(af[1], bf[1]);
            if (REFILL) {
#pragma unroll
                for (int g = 0; g < 16; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 DMA
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        using Refill = std::true_type;
        using NoRefill = std::false_type;

        issue(sA0, sB0, 0);
        if (KT > 1) issue(sA1, sB1, kTK);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        frags(sA0, sB0, 0, af[0], bf[0]);
        // Stages go in pairs (buffer 0, buffer 1). The refill of buffer 1 that
        // the second stage of a pair owes is issued at the top of the next pair
        // instead (the same barrier covers it), so no DMA is in flight across
        // the loop back edge: the compiler then keeps tracking DMAs per buffer
        // and never makes a read of one buffer wait for a refill of the other.
        // The loop runs while the first stage of a pair has a stage to refill
        // (kt + 2 < KT); at most two stages remain after it, neither refills.
        int kt = 0;
        for (; kt + 2 < KT; kt += 2) {
            if (kt >= 2) issue(sA1, sB1, (kt + 1) * kTK);
            stage(Refill{}, sA0, sB0, sA1, sB1, kt);
            stage(NoRefill{}, sA1, sB1, sA0, sB0, kt + 1);
        }
        if (kt >= 2 && kt + 1 < KT) issue(sA1, sB1, (kt + 1) * kTK);
        stage(NoRefill{}, sA0, sB0, sA1, sB1, kt);
        if (kt + 1 < KT) stage(NoRefill{}, sA1, sB1, sA0, sB0, kt + 1);

        // ---- epilogue: acc[i][j][4*g4 + q] is row wm*128 + 32 i + (lane & 31),
        // column (block j) 8 g4 + 4 (lane >> 5) + q, q = 0..3: 8-byte stores.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wm * 128 + i * 32 + fl;
            if (row >= rows) continue;
            if (MODE == kGateUp) {
                uint16_t* dst = out + (size_t)(hrow0 + row) * F;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int col = n0 + wn * 64 + j * 32 + g4 * 8 + fh * 4;
                        if (col >= F) continue;
                        float hv[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            hv[q] = moe::silu(acc[i][j][g4 * 4 + q]) * acc[i][j + 2][g4 * 4 + q];
                        uint2 pk;
                        pk.x = moe::pack_bf16x2(hv[0], hv[1]);
                        pk.y = moe::pack_bf16x2(hv[2], hv[3]);
                        *reinterpret_cast<uint2*>(dst + col) = pk;
                    }
            } else if (ksplit > 1) {
                // fp32 partial sums, expert-sorted rows; summed by ksum_kernel
                float* dst = part + ((size_t)kpart * N + hrow0 + row) * H;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int col = n0 + wn * 128 + j * 32 + g4 * 8 + fh * 4;
                        if (col >= H) continue;
                        *reinterpret_cast<float4*>(dst + col) =
                            make_float4(acc[i][j][g4 * 4 + 0], acc[i][j][g4 * 4 + 1],
                                        acc[i][j][g4 * 4 + 2], acc[i][j][g4 * 4 + 3]);
                    }
            } else {
                uint16_t* dst = out + (size_t)rowmap[row] * H;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int col = n0 + wn * 128 + j * 32 + g4 * 8 + fh * 4;
                        if (col >= H) continue;
                        uint2 pk;
                        pk.x = moe::pack_bf16x2(acc[i][j][g4 * 4 + 0], acc[i][j][g4 * 4 + 1]);
                        pk.y = moe::pack_bf16x2(acc[i][j][g4 * 4 + 2], acc[i][j][g4 * 4 + 3]);
                        *reinterpret_cast<uint2*>(dst + col) = pk;
                    }
            }
        }
        __syncthreads();
    }
}

// Split-K epilogue of the down GEMM: y[vrow[g]] = bf16(part0[g] + part1[g]),
// 8 columns per thread. Two partials, so the sum is independent of order.
__global__ __launch_bounds__(kThreads) void ksum_kernel(int N, int H, const float* __restrict__ part,
                                                        const int32_t* __restrict__ vrow,
                                                        uint16_t* __restrict__ y)
{
    const int per_row = H / 8;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)N * per_row) return;
    const int g = (int)(i / per_row), c = (int)(i % per_row) * 8;
    const float* p0 = part + (size_t)g * H + c;
    const float* p1 = p0 + (size_t)N * H;
    const float4 a0 = *reinterpret_cast<const float4*>(p0), a1 = *reinterpret_cast<const float4*>(p0 + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(p1), b1 = *reinterpret_cast<const float4*>(p1 + 4);
    uint4 o;
    o.x = moe::pack_bf16x2(a0.x + b0.x, a0.y + b0.y);
    o.y = moe::pack_bf16x2(a0.z + b0.z, a0.w + b0.w);
    o.z = moe::pack_bf16x2(a1.x + b1.x, a1.y + b1.y);
    o.w = moe::pack_bf16x2(a1.z + b1.z, a1.w + b1.w);
    *reinterpret_cast<uint4*>(y + (size_t)vrow[g] * H + c) = o;
}

// ---------------------------------------------------------------- fp32 ----
// Plain LDS-tiled VALU kernels for the fp32 dtype (small shapes): 32-row x
// 32-column tiles, K in chunks of 32, each thread 2 x 2 outputs.
constexpr int kFM = 32;

__global__ __launch_bounds__(kThreads) void gateup_f32_kernel(
    int E, int R, int H, int F, int mtiles, const float* __restrict__ a,
    const int32_t* __restrict__ plan, const int32_t* __restrict__ sched,
    const float* __restrict__ wg, const float* __restrict__ wu, float* __restrict__ h)
{
    __shared__ float As[kFM][33], Gs[kFM][33], Us[kFM][33];
    __shared__ int32_t rowmap[kFM];
    const int mt = blockIdx.x % mtiles;
    const int nt = blockIdx.x / mtiles;
    const Tile tile = find_tile(mt, E, kFM, sched);
    if (tile.rows <= 0) return;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int tid = threadIdx.x;
    if (tid < kFM) rowmap[tid] = buf_row_of(tile.e, tile.v0 + (tid < tile.rows ? tid : 0), R, plan, L);
    __syncthreads();
    const int n0 = nt * kFM;
    const int ty = tid / 16, tx = tid % 16;
    float g[2][2] = {}, u[2][2] = {};
    for (int k0 = 0; k0 < H; k0 += 32) {
        for (int i = tid; i < kFM * 32; i += kThreads) {
            const int r = i / 32, c = i % 32;
            const int kc = k0 + c;
            const bool kin = kc < H;
            As[r][c] = kin ? a[(size_t)rowmap[r] * H + kc] : 0.f;
            const int f = min(n0 + r, F - 1);
            Gs[r][c] = kin ? wg[((size_t)tile.e * F + f) * H + kc] : 0.f;
            Us[r][c] = kin ? wu[((size_t)tile.e * F + f) * H + kc] : 0.f;
        }
        __syncthreads();
        for (int c = 0; c < 32; ++c)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    g[i][j] = fmaf(As[ty * 2 + i][c], Gs[tx * 2 + j][c], g[i][j]);
                    u[i][j] = fmaf(As[ty * 2 + i][c], Us[tx * 2 + j][c], u[i][j]);
                }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = ty * 2 + i, col = n0 + tx * 2 + j;
            if (row < tile.rows && col < F)
                h[(size_t)(tile.hrow0 + row) * F + col] = moe::silu(g[i][j]) * u[i][j];
        }
}

__global__ __launch_bounds__(kThreads) void down_f32_kernel(
    int E, int R, int H, int F, int mtiles, const float* __restrict__ h,
    const int32_t* __restrict__ plan, const int32_t* __restrict__ sched,
    const float* __restrict__ wd, float* __restrict__ y)
{
    __shared__ float As[kFM][33], Bs[kFM][33];
    __shared__ int32_t rowmap[kFM];
    const int mt = blockIdx.x % mtiles;
    const int nt = blockIdx.x / mtiles;
    const Tile tile = find_tile(mt, E, kFM, sched);
    if (tile.rows <= 0) return;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int tid = threadIdx.x;
    if (tid < kFM) rowmap[tid] = tid < tile.rows ? buf_row_of(tile.e, tile.v0 + tid, R, plan, L) : -1;
    __syncthreads();
    const int n0 = nt * kFM;
    const int ty = tid / 16, tx = tid % 16;
    float acc[2][2] = {};
    for (int k0 = 0; k0 < F; k0 += 32) {
        for (int i = tid; i < kFM * 32; i += kThreads) {
            const int r = i / 32, c = i % 32;
            const int kc = k0 + c;
            const bool kin = kc < F;
            const int ar = r < tile.rows ? r : 0;
            As[r][c] = kin ? h[(size_t)(tile.hrow0 + ar) * F + kc] : 0.f;
            const int o = min(n0 + r, H - 1);
            Bs[r][c] = kin ? wd[((size_t)tile.e * H + o) * F + kc] : 0.f;
        }
        __syncthreads();
        for (int c = 0; c < 32; ++c)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = fmaf(As[ty * 2 + i][c], Bs[tx * 2 + j][c], acc[i][j]);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = ty * 2 + i, col = n0 + tx * 2 + j;
            if (row < tile.rows && col < H) y[(size_t)rowmap[row] * H + col] = acc[i][j];
        }
}

// Workgroups of the persistent bf16 kernels: one per CU, a multiple of 8 so
// that every XCD gets the same number.
int persistent_grid()
{
    static int grid = 0;
    if (grid == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 256;
        grid = cus >= 8 ? (cus / 8) * 8 : 8;
    }
    return grid;
}

int max_mtiles(const moe_shape_t& s, int bm)
{
    const int64_t N = (int64_t)s.T * s.k;
    return (int)((N + bm - 1) / bm + s.E);
}

}  // namespace

hipError_t moe_launch_gemm_schedule(const moe_shape_t& s, const int32_t* plan, char* ws,
                                    hipStream_t st)
{
    const moe::WsLayout W = moe::ws_layout(s);
    int32_t* sched = reinterpret_cast<int32_t*>(ws + W.sched);
    const bool bf = s.dtype == MOE_BF16;
    schedule_kernel<<<1, kThreads, 0, st>>>(s.E, s.R, bf ? kTM : kFM, plan, sched);
    hipError_t e = hipGetLastError();
    const int N = s.T * s.k;
    if (e != hipSuccess || !bf || N == 0) return e;
    int32_t* vrow = reinterpret_cast<int32_t*>(ws + W.vrow);
    vrow_kernel<<<(N + kThreads - 1) / kThreads, kThreads, 0, st>>>(N, s.E, s.R, plan, sched, vrow);
    return hipGetLastError();
}

hipError_t moe_launch_gemm_gateup(const moe_shape_t& s, const void* a, const int32_t* plan,
                                  const void* w_gate, const void* w_up, char* ws,
                                  hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    const moe::WsLayout W = moe::ws_layout(s);
    const int32_t* sched = reinterpret_cast<const int32_t*>(ws + W.sched);
    if (s.dtype == MOE_BF16) {
        const int ntn = (s.F + kTN / 2 - 1) / (kTN / 2);
        gemm_bf16_kernel<kGateUp><<<persistent_grid(), kThreads, 0, st>>>(
            s.E, ntn, s.H, s.F, 1, s.T * s.k, static_cast<const uint16_t*>(a), sched,
            reinterpret_cast<const int32_t*>(ws + W.vrow), static_cast<const uint16_t*>(w_gate),
            static_cast<const uint16_t*>(w_up), reinterpret_cast<uint16_t*>(ws + W.h), nullptr);
    } else {
        const int mtiles = max_mtiles(s, kFM);
        const int nt = (s.F + kFM - 1) / kFM;
        gateup_f32_kernel<<<mtiles * nt, kThreads, 0, st>>>(
            s.E, s.R, s.H, s.F, mtiles, static_cast<const float*>(a), plan, sched,
            static_cast<const float*>(w_gate), static_cast<const float*>(w_up),
            reinterpret_cast<float*>(ws + W.h));
    }
    return hipGetLastError();
}

hipError_t moe_launch_gemm_down(const moe_shape_t& s, const int32_t* plan, const void* w_down,
                                void* y, char* ws, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    const moe::WsLayout W = moe::ws_layout(s);
    const int32_t* sched = reinterpret_cast<const int32_t*>(ws + W.sched);
    const bool bf = s.dtype == MOE_BF16;
    if (bf) {
        const int ntn = (s.H + kTN - 1) / kTN;
        const int ks = moe::down_ksplit(s);
        const int32_t* vrow = reinterpret_cast<const int32_t*>(ws + W.vrow);
        float* part = reinterpret_cast<float*>(ws + W.part);
        gemm_bf16_kernel<kDown><<<persistent_grid(), kThreads, 0, st>>>(
            s.E, ntn, s.H, s.F, ks, s.T * s.k, reinterpret_cast<const uint16_t*>(ws + W.h), sched, vrow,
            static_cast<const uint16_t*>(w_down), nullptr, static_cast<uint16_t*>(y), part);
        if (ks > 1) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t n = (int64_t)s.T * s.k * (s.H / 8);
            ksum_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(
                s.T * s.k, s.H, part, vrow, static_cast<uint16_t*>(y));
        }
    } else {
        const int mtiles = max_mtiles(s, kFM);
        const int nt = (s.H + kFM - 1) / kFM;
        down_f32_kernel<<<mtiles * nt, kThreads, 0, st>>>(
            s.E, s.R, s.H, s.F, mtiles, reinterpret_cast<const float*>(ws + W.h), plan, sched,
            static_cast<const float*>(w_down), static_cast<float*>(y));
    }
    return hipGetLastError();
}
