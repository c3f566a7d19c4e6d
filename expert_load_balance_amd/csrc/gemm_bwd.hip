// gemm_bwd.hip -- the grouped GEMMs of the expert FFN backward (bf16 in,
// fp32 accumulate, v_mfma_f32_32x32x16_bf16).
//
// The chain rule of the SwiGLU expert FFN ("DeepEP-on-EFA Guidance, section
// 1", phase (c), run in reverse): with g = x W_gate^T, u = x W_up^T,
// h = silu(g) u, y = h W_down^T and the incoming dy,
//   dh = dy W_down            dg = dh u s (1 + g (1 - s)),  du = dh silu(g)
//   dx = dg W_gate + du W_up  (s = 1 / (1 + e^-g))
//   dW_down = dy^T h,  dW_gate = dg^T x,  dW_up = du^T x  (sums over the
// expert's rows: every piece of an expert, home or replica, adds into the
// one gradient of the home expert -- "Moonshot AI drops MoonEP ..."
// paragraph 3 reduces replica gradients home).
//
// Rows are first gathered into expert order (x and dy), so every operand is
// a run of contiguous rows. Five GEMMs, three instances of the row kernel
// and two of the weight-gradient kernel:
//   GU   g | u = x [W_gate; W_up]^T   (recomputed; M = rows, N = 2F, K = H)
//   DH   dh = dy W_down, with the SwiGLU backward in the epilogue
//        (M = rows, N = F, K = H) -> dg | du, h
//   DX   dx = [dg | du] [W_gate; W_up]   (M = rows, N = H, K = 2F),
//        rows scattered back to buffer order
//   WD   dW_down = dy^T h                 (M = F, N = H, K = rows)
//   WGU  [dW_gate; dW_up] = x^T [dg | du] (M = H, N = 2F, K = rows)
// An operand is either K-contiguous (rows of the tile along K) or k-major
// (rows of 256 elements per k, as the weights are laid out for DH and DX and
// the activations for the weight gradients): its k-rows sit in LDS as
// 512-byte rows with 16-byte chunk c at c ^ 4 (k & 3), and each fragment is
// two ds_read_b64_tr_b16 (gfx950's transposing LDS read) -- no transposed
// copy of any tensor is made. Both kernels are warp-specialised: two loader
// waves stream 32-deep stages of a 256 x 256 tile's operands through a ring
// of five LDS slots (global -> LDS copies), eight compute waves only read
// LDS, issue MFMAs and store. The weight gradients are fp32, written once
// per (expert, tile); K past an expert's rows reads a zero page.
#include "common.h"
#include "lds_pipe.h"

namespace {

using namespace moe::lds;

constexpr int kThreads = 256;   // the elementwise and fp32 kernels
constexpr int kK = 64;          // K granule of the DX K-split's part-length rule

enum Kind { kGU = 0, kDH = 1, kDX = 2, kWD = 3, kWGU = 4 };

struct BwdArgs {
    int G, H, F, N;
    const int32_t* sched;  // by-expert schedule, 256-row M-tiles, no skinny tiles
    const int32_t* vrow;   // expert-order row -> buffer row
    const uint16_t* xs;    // x in expert order [N][H]
    const uint16_t* dys;   // dy in expert order [N][H]
    const uint16_t *wg, *wu, *wd;
    uint16_t* gu;          // [N][2F]: g | u
    uint16_t* dgu;         // [N][2F]: dg | du
    uint16_t* hb;          // [N][F]: h
    uint16_t* dxbuf;       // [N][H], buffer order
    float *dwg, *dwu, *dwd;
    const char* zero;      // >= 512 zero bytes
    int dx_split_max;      // DX K-split bound (partials allocated for it)
    float* dxpart;         // DX partials [split][N][H], expert order
    // replica mode of the weight gradients: groups [2E] of {e, k0, k1, out}
    // (out -1: the home gradient; >= 0: replica slot r*n + j; -2: unused)
    const int32_t* rgroups;
    float* rgrad;          // [R*n][3][F*H]
};

// DX K-split: the part count in [1, smax] that fills the workgroups best
// (ties: fewer parts), each part at least 8 stages. Few, long tiles (a few
// experts with a wide F) otherwise leave a round of workgroups mostly idle.
__host__ __device__ inline int dx_split(int tiles, int P, int smax, int stages)
{
    int best = 1;
    double best_u = 0.0;
    for (int sp = 1; sp <= smax; ++sp) {
        if (sp > 1 && stages / sp < 8) break;
        const long units = (long)tiles * sp;
        const long rounds = (units + P - 1) / P;
        const double u = rounds > 0 ? (double)units / (double)(rounds * P) : 1.0;
        if (u > best_u + 1e-9) {
            best_u = u;
            best = sp;
        }
    }
    return best;
}

// chunk swizzle of a k-major row: 4 consecutive k-rows cover all 64 banks
__device__ __forceinline__ int kswz(int kr) { return (kr & 3) << 2; }

__device__ __forceinline__ float sigm(float z)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// The weight gradients, warp-specialised. Their fp32 outputs (F x H floats
// per matrix and expert) outweigh the bf16 operands, so the stores must run
// under the MFMAs: eight compute waves never load from global memory (their
// vmcnt only ever counts their own stores, so no wait of theirs waits for
// one), and two loader waves stream the operand stages into a ring of LDS
// slots, across tile boundaries, one barrier per stage.
//   tile 256 x 256, K in 32-deep stages of k-major rows (512 bytes per k-row
//   and operand, chunk c at c ^ 4 (k & 3), transposing reads), compute waves
//   2 x 4, each 128 x 64. M is the gradient's contiguous dimension (h for
//   dW_gate|up, f for dW_down).
//   Stage g sits in slot g % kWSlots. At barrier g the loaders have waited
//   for stage g's copies and the compute waves have consumed stage g - 1's
//   fragments; the loaders then refill slot (g - 1) % kWSlots with stage
//   g + kWSlots - 1. A tile's last stage is followed by one more barrier,
//   after which that stage's slot (not refilled before the next barrier)
//   is the compute waves' scratch: each 32 x 32 fp32 block turns there so
//   that every dwordx4 store writes whole 128-byte lines.
constexpr int kWT = 256, kWK = 32;
constexpr int kWOp = kWK * kWT * 2;                       // 16 KB: one operand of a stage
constexpr int kWSlot = 2 * kWOp;                          // A, then B
constexpr int kWSlots = 5;                                // 160 KB of LDS
constexpr int kWCompute = 8, kWLoaders = 2;               // waves
constexpr int kWThreads = (kWCompute + kWLoaders) * 64;
constexpr int kWCopies = kWSlot / 1024 / kWLoaders;       // copies per loader wave per stage
constexpr int kWPer = kWCopies / 2;                       // of them per operand
static_assert(kWCopies * (kWSlots - 2) < 64, "vmcnt range");
constexpr int kWScratch = 32 * 32 * 4;                    // a compute wave's 32 x 32 fp32 block
static_assert(kWCompute * kWScratch <= kWSlot, "scratch fits a slot");

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct WTile {
    int e, out, hrow0, rows, ns, m0, n0;
};

// tile u of the weight-gradient stream: group (home expert, or a row range of
// one in replica mode), then its M x N tiles
__device__ __forceinline__ WTile wtile(const BwdArgs& a, int u, int mtw, int ntw)
{
    const int32_t* rs = a.sched + a.G + 1;
    const int g = u / (mtw * ntw), local = u % (mtw * ntw);
    WTile t;
    // bands of 4 M-tiles, N-tiles across a band, M fastest: an XCD's run of
    // consecutive tiles covers 4 A panels and few B panels
    const int band = local / (4 * ntw), rb = local % (4 * ntw);
    const int bm = min(4, mtw - band * 4);
    t.m0 = uni((band * 4 + rb % bm) * kWT);
    t.n0 = uni((rb / bm) * kWT);
    int k0 = 0, k1 = 0;
    if (a.rgroups) {
        t.out = ldc(a.rgroups, 4 * g + 3);
        t.e = t.out == -2 ? 0 : ldc(a.rgroups, 4 * g);
        if (t.out != -2) {
            k0 = ldc(a.rgroups, 4 * g + 1);
            k1 = ldc(a.rgroups, 4 * g + 2);
        }
    } else {
        t.e = g;
        t.out = -1;
        k1 = ldc(rs, g + 1) - ldc(rs, g);
    }
    t.hrow0 = uni(ldc(rs, t.e) + k0);
    t.rows = uni(k1 - k0);
    t.ns = t.out == -2 ? 0 : (t.rows + kWK - 1) / kWK;
    return t;
}

template <int KIND>
__global__ __launch_bounds__(kWThreads, 1) void wgrad_kernel(BwdArgs a)
{
    __shared__ __attribute__((aligned(1024))) char slots[kWSlots * kWSlot];
    const int H = a.H, F = a.F;
    // A columns (M, the gradient's contiguous dimension), B columns (N)
    const int M = KIND == kWD ? F : H, Nc = KIND == kWD ? H : 2 * F;
    const int mtw = (M + kWT - 1) / kWT, ntw = (Nc + kWT - 1) / kWT;
    const int groups = a.rgroups ? 2 * a.G : a.G;
    const int total = groups * mtw * ntw;
    const int tid = threadIdx.x;
    const int wave = uni(tid >> 6), lane = tid & 63;
    const int P = gridDim.x;
    // each XCD (workgroups are dealt to the 8 XCDs round-robin) takes a
    // contiguous run of tiles, so tiles sharing an operand share that L2
    const int my_slot = (blockIdx.x % 8) * (P / 8) + blockIdx.x / 8;

    if (wave >= kWCompute) {
        // loader lw: copies q = lw + kWLoaders i (i < kWPer) of each operand, copy q
        // covering k-rows 2q and 2q + 1 (512 bytes each)
        const int lw = wave - kWCompute;
        const uint32_t slots_u = (uint32_t)(uintptr_t)slots;
        const char* zero = a.zero;
        const uint16_t* asrc = KIND == kWD ? a.hb : a.xs;
        const uint16_t* bsrc = KIND == kWD ? a.dys : a.dgu;
        const int astride = KIND == kWD ? F : H, bstride = KIND == kWD ? H : 2 * F;
        // issue cursor (lu, ls) and its tile lt; per-tile lane offsets of the
        // full-stage copies (the chunk column clamped into the matrix: a
        // column past M or N only feeds outputs that are not stored)
        int lu = my_slot, ls = 0;
        WTile lt = {};
        uint32_t aoff[kWPer], boff[kWPer];
        auto seek = [&]() {
            for (; lu < total; lu += P) {
                lt = wtile(a, lu, mtw, ntw);
                if (lt.ns > 0) break;
            }
            if (lu >= total) return;
#pragma unroll
            for (int i = 0; i < kWPer; ++i) {
                const int kr = 2 * (lw + kWLoaders * i) + (lane >> 5), c = (lane & 31) ^ kswz(kr);
                aoff[i] = (uint32_t)(kr * astride + min(lt.m0 + 8 * c, M - 8)) * 2u;
                boff[i] = (uint32_t)(kr * bstride + min(lt.n0 + 8 * c, Nc - 8)) * 2u;
            }
        };
        seek();
        int issued = 0;
        auto issue = [&]() {
            const uint32_t slot = slots_u + (uint32_t)(issued % kWSlots) * kWSlot;
            const int kb = ls * kWK;
            if (kb + kWK <= lt.rows) {
                // a full stage: uniform row base + the tile's lane offsets
                const size_t r0 = (size_t)(lt.hrow0 + kb);
                const uint16_t* ab = uni_ptr(asrc + r0 * astride);
                const uint16_t* bb = uni_ptr(bsrc + r0 * bstride);
#pragma unroll
                for (int i = 0; i < kWPer; ++i) copy16(ab, aoff[i], slot + (lw + kWLoaders * i) * 1024);
#pragma unroll
                for (int i = 0; i < kWPer; ++i) copy16(bb, boff[i], slot + kWOp + (lw + kWLoaders * i) * 1024);
            } else {
                // the ragged last stage: k-rows past the rows read the zero page
#pragma unroll
                for (int i = 0; i < kWPer; ++i) {
                    const int q = lw + kWLoaders * i;
                    const int kr = 2 * q + (lane >> 5), c = (lane & 31) ^ kswz(kr);
                    const int k = kb + kr, ca = lt.m0 + 8 * c, cb = lt.n0 + 8 * c;
                    const bool kin = k < lt.rows;
                    const size_t row = (size_t)(lt.hrow0 + k);
                    const char* pa = kin && ca < M ? (const char*)(asrc + row * astride + ca) : zero + c * 16;
                    const char* pb = kin && cb < Nc ? (const char*)(bsrc + row * bstride + cb) : zero + c * 16;
                    copy16_at(pa, slot + q * 1024);
                    copy16_at(pb, slot + kWOp + q * 1024);
                }
            }
            ++issued;
            if (++ls >= lt.ns) {
                ls = 0;
                lu += P;
                seek();
            }
        };
        // consume cursor: stages left in the tile being computed, for the
        // barrier that ends each tile
        int cu = my_slot, crem = 0;
        auto cseek = [&]() {
            for (; cu < total; cu += P) {
                crem = wtile(a, cu, mtw, ntw).ns;
                if (crem > 0) break;
            }
        };
        cseek();
        while (issued < kWSlots - 1 && lu < total) issue();
        for (int g = 0; g < issued; ++g) {
            // stage g landed; the stages issued after it may be in flight
            const int after = issued - 1 - g;
            if (after >= 3) wait_vm_lgkm<3 * kWCopies>();
            else if (after == 2) wait_vm_lgkm<2 * kWCopies>();
            else if (after == 1) wait_vm_lgkm<kWCopies>();
            else wait_vm_lgkm<0>();
            slot_barrier();
            if (lu < total) issue();
            if (--crem == 0) {
                slot_barrier();  // the tile's end: its last slot becomes scratch
                cu += P;
                cseek();
            }
        }
        return;
    }

    // compute waves, 2 x 4, each 128 x 64 of the tile
    const int wm = wave >> 2, wn = wave & 3;
    const size_t FH = (size_t)F * H;
    int g = 0;  // stages consumed
    for (int u = my_slot; u < total; u += P) {
        const WTile t = wtile(a, u, mtw, ntw);
        if (t.out == -2) continue;  // an unused replica slot
        // k-major fragments (k-steps 0..1, reads h = 0, 1): lane reads 4
        // columns m_in (+ 32 b) at k-row kr; block b's 64 bytes sit at
        // (b ^ (kr & 3)) * 64 (bits 6..8 of the offset, which the rest of it
        // leaves clear), so block b0 + i of A (B) is at fa (fb) ^ (i << 6).
        // Recomputed per tile from an opaque copy of the lane index, so that
        // they are not held (or spilled) across the epilogue.
        uint32_t fa0[2], fa1[2], fb0[2], fb1[2];
        {
            int ln;
            asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
            const int m_in = 16 * ((ln >> 4) & 1) + 4 * (ln & 3);
            const int lx = (ln >> 2) & 3;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kr = 16 * kk + 8 * (ln >> 5) + 4 * h + ((ln & 15) >> 2);
                    const uint32_t in = (uint32_t)kr * 512u + (uint32_t)((m_in >> 3) << 4) +
                                        (uint32_t)((m_in & 7) * 2);
                    (h ? fa1 : fa0)[kk] = in | (uint32_t)(((wm * 4) ^ lx) << 6);
                    (h ? fb1 : fb0)[kk] = in | (uint32_t)(((wn * 2) ^ lx) << 6);
                }
            }
        }
        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

        for (int s = 0; s < t.ns; ++s, ++g) {
            slot_barrier();
            const char* sa = slots + (g % kWSlots) * kWSlot;
            const char* sb = sa + kWOp;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 af[4], bfr[2];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = lds_frag_tr(sa + (fa0[kk] ^ (i << 6)), sa + (fa1[kk] ^ (i << 6)));
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bfr[j] = lds_frag_tr(sb + (fb0[kk] ^ (j << 6)), sb + (fb1[kk] ^ (j << 6)));
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
        }

        // acc[i][j][4 g4 + q] is (m, n) = (128 wm + 32 i + 8 g4 + 4 fh + q,
        // 64 wn + 32 j + fr): four consecutive floats of gradient row n. Each
        // 32 x 32 block turns in the wave's scratch (row n, 16-byte unit u at
        // u ^ (n & 7): conflict-free both ways), so that every dwordx4 store
        // writes whole 128-byte lines of 8 rows. An empty tile (no rows of
        // its expert) stores zeros straight away.
        // indices from the lane, again through an opaque copy (not hoisted out
        // of the tile loop and held through it)
        int el;
        asm volatile("v_mov_b32 %0, %1" : "=v"(el) : "v"(lane));
        const int er = el & 31, eh = el >> 5;
        char* scr = nullptr;
        if (t.ns > 0) {
            slot_barrier();  // every wave has read the last stage's slot
            scr = slots + ((g - 1) % kWSlots) * kWSlot + wave * kWScratch;
        }
        float* gdst = t.out < 0 ? a.dwg + t.e * FH : a.rgrad + ((size_t)t.out * 3 + 0) * FH;
        float* udst = t.out < 0 ? a.dwu + t.e * FH : a.rgrad + ((size_t)t.out * 3 + 1) * FH;
        float* ddst = t.out < 0 ? a.dwd + t.e * FH : a.rgrad + ((size_t)t.out * 3 + 2) * FH;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (scr) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const f32x4 v = {acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                         acc[i][j][4 * g4 + 3]};
                        const int u4 = 2 * g4 + eh;
                        *reinterpret_cast<f32x4*>(scr + er * 128 + ((u4 ^ (er & 7)) << 4)) = v;
                    }
                }
                const int m = t.m0 + wm * 128 + i * 32 + 4 * (el & 7);
#pragma unroll
                for (int rb = 0; rb < 32; rb += 8) {
                    const int r = rb + (el >> 3);
                    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
                    if (scr) v = *reinterpret_cast<const f32x4*>(scr + r * 128 + (((el & 7) ^ (r & 7)) << 4));
                    const int n = t.n0 + wn * 64 + j * 32 + r;
                    if (m >= M || n >= Nc) continue;
                    float* dst;
                    if (KIND == kWD) dst = ddst + (size_t)n * F + m;
                    else dst = (n < F ? gdst + (size_t)n * H : udst + (size_t)(n - F) * H) + m;
                    // streaming: the gradients are not read again here
                    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
                }
            }
    }
}

// The row GEMMs GU, DH and DX on the same ring (32-deep stages, two loader
// waves, eight compute waves 2 x 4 of 128 x 64, one barrier per stage). A
// (x, dy or dg | du rows) is K-contiguous: a stage holds 64-byte segments of
// 256 rows, 16-byte unit c of row r at c ^ ((r >> 2) & 3), so the 16 rows
// one ds_read_b128 pass reads hit 16 distinct bank groups. B is the weights:
// for DH and DX their k-major rows as above, for GU the rows n of
// [W_gate; W_up], K-contiguous like A. Rows past an M-tile's valid rows
// repeat its last row and weight columns (rows) past the end repeat the last
// one (those outputs are dropped). Units: K-split part, then expert, N-tile,
// M-tile (M fastest). The bf16 outputs are small beside the weight
// gradients' and leave straight from the accumulators.
struct DTile {
    int e, m0, n0, rows, hrow0, s0, ns, part;
};

__device__ __forceinline__ DTile dtile(const BwdArgs& a, int u, int tiles, int ntn, int nsplit, int k32)
{
    const int32_t* ts = a.sched;
    const int32_t* rs = a.sched + a.G + 1;
    const int part = u / tiles, t = u % tiles;
    int lo = 0, hi = a.G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ldc(ts, mid) * ntn <= t) lo = mid;
        else hi = mid - 1;
    }
    const int t0 = ldc(ts, lo), mt_e = ldc(ts, lo + 1) - t0;
    const int local = t - t0 * ntn;
    DTile d;
    d.e = uni(lo);
    d.n0 = uni((local / mt_e) * kWT);
    d.m0 = uni((local % mt_e) * kWT);
    const int r0 = ldc(rs, lo);
    d.rows = uni(min(kWT, ldc(rs, lo + 1) - r0 - d.m0));
    d.hrow0 = uni(r0 + d.m0);
    d.part = uni(part);
    d.s0 = uni(part * k32 / nsplit);
    d.ns = uni((part + 1) * k32 / nsplit - d.s0);
    return d;
}

template <int KIND>
__global__ __launch_bounds__(kWThreads, 1) void dgrad_kernel(BwdArgs a)
{
    __shared__ __attribute__((aligned(1024))) char slots[kWSlots * kWSlot];
    const int H = a.H, F = a.F;
    const int K = KIND == kDX ? 2 * F : H, k32 = K / kWK;
    const int Nc = KIND == kDX ? H : KIND == kGU ? 2 * F : F;  // output columns
    const int ntn = (Nc + kWT - 1) / kWT;
    const int tiles = a.sched[a.G] * ntn;
    const int P = gridDim.x;
    const int nsplit = KIND == kDX ? dx_split(tiles, P, a.dx_split_max, 2 * F / kK) : 1;
    const int total = tiles * nsplit;
    const int tid = threadIdx.x;
    const int wave = uni(tid >> 6), lane = tid & 63;
    const int my_slot = (blockIdx.x % 8) * (P / 8) + blockIdx.x / 8;
    const size_t FH = (size_t)F * H;

    if (wave >= kWCompute) {
        // loader lw: A copy q (q = lw + kWLoaders i, i < kWPer) covers rows 16q .. 16q + 15
        // (four lanes a row), B copy q k-rows 2q and 2q + 1
        const int lw = wave - kWCompute;
        const uint32_t slots_u = (uint32_t)(uintptr_t)slots;
        const uint16_t* asrc = KIND == kDX ? a.dgu : KIND == kGU ? a.xs : a.dys;
        const int lda = KIND == kDX ? 2 * F : H;
        const int ldb = KIND == kDX ? H : KIND == kGU ? H : F;  // weight row length
        int lu = my_slot, ls = 0;
        DTile lt = {};
        uint32_t aoff[kWPer], boff[kWPer];
        const uint16_t* gbase[kWPer];  // GU: the weight matrix of copy i's 16 rows
        auto seek = [&]() {
            for (; lu < total; lu += P) {
                lt = dtile(a, lu, tiles, ntn, nsplit, k32);
                if (lt.ns > 0) break;
            }
            if (lu >= total) return;
#pragma unroll
            for (int i = 0; i < kWPer; ++i) {
                const int q = lw + kWLoaders * i;
                const int row = 16 * q + (lane >> 2), c = (lane & 3) ^ ((row >> 2) & 3);
                aoff[i] = (uint32_t)min(row, lt.rows - 1) * (uint32_t)lda * 2u + (uint32_t)c * 16u;
                if (KIND == kGU) {
                    // rows n0 + 16q .. + 15 of [W_gate; W_up] (F % 16 == 0: one side)
                    const bool up = lt.n0 + 16 * q >= F;
                    const int n = min(lt.n0 + row, 2 * F - 1) - (up ? F : 0);
                    gbase[i] = uni_ptr((up ? a.wu : a.wg) + lt.e * FH);
                    boff[i] = (uint32_t)n * (uint32_t)H * 2u + (uint32_t)c * 16u;
                } else {
                    const int kr = 2 * q + (lane >> 5), cb = (lane & 31) ^ kswz(kr);
                    boff[i] = (uint32_t)kr * (uint32_t)ldb * 2u + (uint32_t)min(lt.n0 + 8 * cb, ldb - 8) * 2u;
                }
            }
        };
        seek();
        int issued = 0;
        auto issue = [&]() {
            const uint32_t slot = slots_u + (uint32_t)(issued % kWSlots) * kWSlot;
            if (KIND == kDH && ls >= lt.ns) {
                // g | u rows 32 c .. 32 c + 31 of the tile: copy q is row q,
                // lanes 0..31 its 256 g columns, 32..63 its 256 u columns;
                // logical 16-byte unit v at v ^ (q & 31) (rows past the
                // tile's repeat its last; columns past F repeat the last chunk)
                const int c = ls - lt.ns;
                const uint16_t* gb = uni_ptr(a.gu + (size_t)lt.hrow0 * 2 * F);
#pragma unroll
                for (int i = 0; i < 2 * kWPer; ++i) {
                    const int q = lw + kWLoaders * i;
                    const int row = min(32 * c + q, lt.rows - 1);
                    const int v = lane ^ (q & 31);
                    const int col = min(lt.n0 + 8 * (v & 31), F - 8) + (v >= 32 ? F : 0);
                    copy16(gb, (uint32_t)(row * 2 * F + col) * 2u, slot + q * 1024);
                }
                ++issued;
                if (++ls >= lt.ns + (lt.rows + 31) / 32) {
                    ls = 0;
                    lu += P;
                    seek();
                }
                return;
            }
            const int s = lt.s0 + ls;
            const uint16_t* ab = uni_ptr(asrc + (size_t)lt.hrow0 * lda + s * kWK);
            const uint16_t* wb = nullptr;
            if (KIND == kDH) {
                wb = a.wd + lt.e * FH + (size_t)s * kWK * F;
            } else if (KIND == kDX) {
                const int k0 = s * kWK;  // F % 32 == 0: a stage is all gate or all up
                wb = k0 < F ? a.wg + lt.e * FH + (size_t)k0 * H : a.wu + lt.e * FH + (size_t)(k0 - F) * H;
            }
            wb = uni_ptr(wb);
#pragma unroll
            for (int i = 0; i < kWPer; ++i) copy16(ab, aoff[i], slot + (lw + kWLoaders * i) * 1024);
#pragma unroll
            for (int i = 0; i < kWPer; ++i)
                copy16(KIND == kGU ? gbase[i] + s * kWK : wb, boff[i], slot + kWOp + (lw + kWLoaders * i) * 1024);
            ++issued;
            if (++ls >= lt.ns + (KIND == kDH ? (lt.rows + 31) / 32 : 0)) {
                ls = 0;
                lu += P;
                seek();
            }
        };
        while (issued < kWSlots - 1 && lu < total) issue();
        for (int g = 0; g < issued; ++g) {
            const int after = issued - 1 - g;
            if (after >= 3) wait_vm_lgkm<3 * kWCopies>();
            else if (after == 2) wait_vm_lgkm<2 * kWCopies>();
            else if (after == 1) wait_vm_lgkm<kWCopies>();
            else wait_vm_lgkm<0>();
            slot_barrier();
            if (lu < total) issue();
        }
        return;
    }

    const int wm = wave >> 2, wn = wave & 3;
    int g = 0;  // stages consumed
    for (int u = my_slot; u < total; u += P) {
        const DTile t = dtile(a, u, tiles, ntn, nsplit, k32);
        if (t.ns <= 0) continue;
        // fragment offsets from an opaque copy of the lane index (recomputed
        // per tile, not held through the epilogue): A row 32 blk + fr, unit
        // 2 kk + fh; B as in the weight gradients
        uint32_t fa[2], fb0[2], fb1[2];  // GU: fb0 is B's K-contiguous offset
        {
            int ln;
            asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
            const int fr = ln & 31, fh = ln >> 5;
            const int m_in = 16 * ((ln >> 4) & 1) + 4 * (ln & 3);
            const int lx = (ln >> 2) & 3;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                fa[kk] = (uint32_t)(fr * 64 + 16 * ((2 * kk + fh) ^ ((fr >> 2) & 3)) + wm * 4 * 2048);
                fb0[kk] = fb1[kk] = (uint32_t)(fr * 64 + 16 * ((2 * kk + fh) ^ ((fr >> 2) & 3)) + wn * 2 * 2048);
                if (KIND == kGU) continue;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kr = 16 * kk + 8 * fh + 4 * h + ((ln & 15) >> 2);
                    const uint32_t in = (uint32_t)kr * 512u + (uint32_t)((m_in >> 3) << 4) +
                                        (uint32_t)((m_in & 7) * 2);
                    (h ? fb1 : fb0)[kk] = in | (uint32_t)(((wn * 2) ^ lx) << 6);
                }
            }
        }
        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

        for (int s = 0; s < t.ns; ++s, ++g) {
            slot_barrier();
            const char* sa = slots + (g % kWSlots) * kWSlot;
            const char* sb = sa + kWOp;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 af[4], bfr[2];
#pragma unroll
                for (int i = 0; i < 4; ++i) af[i] = lds_frag(sa + fa[kk] + i * 2048);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bfr[j] = KIND == kGU ? lds_frag(sb + fb0[kk] + j * 2048)
                                         : lds_frag_tr(sb + (fb0[kk] ^ (j << 6)), sb + (fb1[kk] ^ (j << 6)));
                // B first: a lane holds 4 consecutive output columns
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
            }
        }

        // acc[i][j][4 g4 + q] is (m, n) = (128 wm + 32 i + fr,
        // 64 wn + 32 j + 8 g4 + 4 fh + q) of the tile
        int el;
        asm volatile("v_mov_b32 %0, %1" : "=v"(el) : "v"(lane));
        const int er = el & 31, eh = el >> 5;
        if (KIND == kGU) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = wm * 128 + i * 32 + er;
                if (m >= t.rows) continue;
                uint16_t* grow = a.gu + (size_t)(t.hrow0 + m) * 2 * F;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int col = t.n0 + wn * 64 + j * 32 + g4 * 8 + eh * 4;
                        if (col >= 2 * F) continue;
                        uint2 pk;
                        pk.x = moe::pack_bf16x2(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1]);
                        pk.y = moe::pack_bf16x2(acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]);
                        *reinterpret_cast<uint2*>(grow + col) = pk;
                    }
            }
        } else if (KIND == kDX && nsplit > 1) {
            // fp32 partials (expert order), summed by dx_fixup_kernel
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = wm * 128 + i * 32 + er;
                if (m >= t.rows) continue;
                float* prow = a.dxpart + ((size_t)t.part * a.N + t.hrow0 + m) * H;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int col = t.n0 + wn * 64 + j * 32 + g4 * 8 + eh * 4;
                        if (col >= H) continue;
                        *reinterpret_cast<f32x4*>(prow + col) =
                            f32x4{acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                  acc[i][j][4 * g4 + 3]};
                    }
            }
        } else if (KIND == kDX) {
            // bf16 rows scattered back to buffer order (every row index
            // loaded before the first store)
            int orow[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                orow[i] = a.vrow[t.hrow0 + min(wm * 128 + i * 32 + er, t.rows - 1)];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = wm * 128 + i * 32 + er;
                if (m >= t.rows) continue;
                uint16_t* orp = a.dxbuf + (size_t)orow[i] * H;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int col = t.n0 + wn * 64 + j * 32 + g4 * 8 + eh * 4;
                        if (col >= H) continue;
                        uint2 pk;
                        pk.x = moe::pack_bf16x2(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1]);
                        pk.y = moe::pack_bf16x2(acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]);
                        *reinterpret_cast<uint2*>(orp + col) = pk;
                    }
            }
        } else {
            // DH: the SwiGLU backward. The tile's g | u follows its K stages
            // through the ring, 32 rows a slot: slot c = 4 hb + i holds rows
            // 32 c .. 32 c + 31, row block i of the waves with wm = hb (the
            // other four only pass the barrier)
            const int nch = (t.rows + 31) / 32;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (hb * 4 + i >= nch) break;
                    slot_barrier();
                    const char* sg = slots + (g % kWSlots) * kWSlot + er * 1024;
                    ++g;
                    const int m = wm * 128 + i * 32 + er;
                    if (wm != hb || m >= t.rows) continue;
                    const size_t r2 = (size_t)(t.hrow0 + m) * 2 * F;
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const int col = t.n0 + wn * 64 + j * 32 + g4 * 8 + eh * 4;
                            if (col >= F) continue;
                            const int v = wn * 8 + j * 4 + g4;  // logical unit of the 8 columns
                            const uint2 gq = *reinterpret_cast<const uint2*>(sg + ((v ^ er) << 4) + eh * 8);
                            const uint2 uq = *reinterpret_cast<const uint2*>(sg + (((v + 32) ^ er) << 4) + eh * 8);
                            const float gv[4] = {__uint_as_float(gq.x << 16), __uint_as_float(gq.x & 0xffff0000u),
                                                 __uint_as_float(gq.y << 16), __uint_as_float(gq.y & 0xffff0000u)};
                            const float uv[4] = {__uint_as_float(uq.x << 16), __uint_as_float(uq.x & 0xffff0000u),
                                                 __uint_as_float(uq.y << 16), __uint_as_float(uq.y & 0xffff0000u)};
                            float dg[4], du[4], hv[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const float dh = acc[i][j][4 * g4 + q];
                                const float sgm = sigm(gv[q]);
                                const float sl = gv[q] * sgm;
                                hv[q] = sl * uv[q];
                                du[q] = dh * sl;
                                dg[q] = dh * uv[q] * sgm * (1.0f + gv[q] * (1.0f - sgm));
                            }
                            uint2 pk;
                            pk.x = moe::pack_bf16x2(dg[0], dg[1]);
                            pk.y = moe::pack_bf16x2(dg[2], dg[3]);
                            *reinterpret_cast<uint2*>(a.dgu + r2 + col) = pk;
                            pk.x = moe::pack_bf16x2(du[0], du[1]);
                            pk.y = moe::pack_bf16x2(du[2], du[3]);
                            *reinterpret_cast<uint2*>(a.dgu + r2 + F + col) = pk;
                            pk.x = moe::pack_bf16x2(hv[0], hv[1]);
                            pk.y = moe::pack_bf16x2(hv[2], hv[3]);
                            *reinterpret_cast<uint2*>(a.hb + (size_t)(t.hrow0 + m) * F + col) = pk;
                        }
                }
        }
    }
}

// rows of src (buffer order) into expert order: dst[x] = src[vrow[x]]
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(int N, int row_vecs,
                                                               const int32_t* __restrict__ vrow,
                                                               const uint4* __restrict__ src,
                                                               uint4* __restrict__ dst)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)N * row_vecs) return;
    const int x = (int)(i / row_vecs), c = (int)(i % row_vecs);
    dst[i] = src[(size_t)vrow[x] * row_vecs + c];
}

// DX partials summed in part order, rounded once, rows scattered back to
// buffer order. The part count is the DX kernel's own choice.
__global__ __launch_bounds__(kThreads) void dx_fixup_kernel(BwdArgs a, int P)
{
    const int H = a.H;
    const int tiles = a.sched[a.G] * ((H + kWT - 1) / kWT);
    const int nsplit = dx_split(tiles, P, a.dx_split_max, 2 * a.F / kK);
    if (nsplit <= 1) return;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // 4 columns each
    if (i >= (int64_t)a.N * (H / 4)) return;
    const int x = (int)(i / (H / 4)), c = (int)(i % (H / 4)) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = 0; p < nsplit; ++p) {
        const float4 v = *reinterpret_cast<const float4*>(a.dxpart + ((size_t)p * a.N + x) * H + c);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    uint2 pk;
    pk.x = moe::pack_bf16x2(acc.x, acc.y);
    pk.y = moe::pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2*>(a.dxbuf + (size_t)a.vrow[x] * H + c) = pk;
}

// Replica mode: one group per expert (its home piece's rows, possibly none)
// and one per replica slot (r, j) of the plan (the replica piece's rows on
// rank r); rows are offsets into the expert's rows in expert order, where
// its pieces follow in rank order. slot_of[e][r] = j, or -1.
__global__ __launch_bounds__(kThreads) void replica_groups_kernel(int E, int R,
                                                                  const int32_t* __restrict__ plan,
                                                                  int32_t* __restrict__ groups,
                                                                  int32_t* __restrict__ slot_of)
{
    const int t = blockIdx.x * kThreads + threadIdx.x;
    const int n = E / R;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    if (t >= E) {  // replica slot t - E without an expert: unused
        const int sl = t - E;
        if (sl < R * n && plan[L.slot_expert + sl] < 0) {
            int32_t* g = groups + 4 * (E + sl);
            g[0] = 0; g[1] = 0; g[2] = 0; g[3] = -2;
        }
        return;
    }
    const int e = t, home = e / n;
    for (int r = 0; r < R; ++r) slot_of[(size_t)e * R + r] = -1;
    int32_t* hg = groups + 4 * e;
    hg[0] = e; hg[1] = 0; hg[2] = 0; hg[3] = -1;
    const int np = plan[L.piece_num + e];
    int cum = 0;
    for (int p = 0; p < np && p < R; ++p) {
        const int r = plan[L.piece_rank + (size_t)e * R + p];
        const int c = plan[L.piece_cnt + (size_t)e * R + p];
        if (r == home) {
            hg[1] = cum;
            hg[2] = cum + c;
        } else if (r >= 0 && r < R) {
            for (int j = 0; j < n; ++j) {
                if (plan[L.slot_expert + (size_t)r * n + j] == e) {
                    int32_t* g = groups + 4 * (E + r * n + j);
                    g[0] = e; g[1] = cum; g[2] = cum + c; g[3] = r * n + j;
                    slot_of[(size_t)e * R + r] = j;
                    break;
                }
            }
        }
        cum += c;
    }
}

// The replica-gradient reduction: dW[e] += the gradients in e's replica
// slots, added in rank order after the home part; experts without replicas
// are left alone. blockIdx.y = expert; 4 floats per thread, grid-stride.
__global__ __launch_bounds__(kThreads) void reduce_replicas_kernel(int E, int R, int64_t FH,
                                                                   const int32_t* __restrict__ slot_of,
                                                                   const float* __restrict__ rgrad,
                                                                   float* __restrict__ dwg,
                                                                   float* __restrict__ dwu,
                                                                   float* __restrict__ dwd)
{
    const int e = blockIdx.y;
    const int n = E / R;
    const int32_t* so = slot_of + (size_t)e * R;
    bool any = false;
    for (int r = 0; r < R; ++r) any |= so[r] >= 0;
    if (!any) return;
    const int64_t n4 = 3 * FH / 4;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t w = i * 4;
        const int q = (int)(w / FH);
        const int64_t o = w % FH;
        float* d = (q == 0 ? dwg : q == 1 ? dwu : dwd) + (size_t)e * FH + o;
        float4 acc = *reinterpret_cast<const float4*>(d);
        for (int r = 0; r < R; ++r) {
            const int j = so[r];
            if (j < 0) continue;
            const float4 v = *reinterpret_cast<const float4*>(
                rgrad + ((size_t)(r * n + j) * 3 + q) * FH + o);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        *reinterpret_cast<float4*>(d) = acc;
    }
}

__global__ void zero_kernel(uint4* p, int n)
{
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = make_uint4(0, 0, 0, 0);
}

// ---- fp32 (small shapes): one thread per output element, FMA in index
// order, rows in expert order; e(x) by a search over row_start.
__device__ __forceinline__ int expert_of_row(int x, int E, const int32_t* row_start)
{
    int lo = 0, hi = E - 1;  // last expert with row_start <= x (non-empty)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (row_start[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// per (row x, f): g, u, h; dh = dy . W_down[:, f]; dg, du
__global__ __launch_bounds__(kThreads) void bwd_f32_rows_kernel(int N, int E, int H, int F,
                                                                const int32_t* __restrict__ sched,
                                                                const float* __restrict__ xs,
                                                                const float* __restrict__ dys,
                                                                const float* __restrict__ wg,
                                                                const float* __restrict__ wu,
                                                                const float* __restrict__ wd,
                                                                float* __restrict__ dgu,
                                                                float* __restrict__ hb)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)N * F) return;
    const int x = (int)(i / F), f = (int)(i % F);
    const int e = expert_of_row(x, E, sched + E + 1);
    const size_t FH = (size_t)F * H;
    const float* xr = xs + (size_t)x * H;
    const float* dyr = dys + (size_t)x * H;
    float g = 0.f, u = 0.f, dh = 0.f;
    for (int c = 0; c < H; ++c) {
        g = fmaf(wg[e * FH + (size_t)f * H + c], xr[c], g);
        u = fmaf(wu[e * FH + (size_t)f * H + c], xr[c], u);
        dh = fmaf(wd[e * FH + (size_t)c * F + f], dyr[c], dh);
    }
    const float s = 1.0f / (1.0f + expf(-g));
    const float sl = g * s;
    hb[(size_t)x * F + f] = sl * u;
    dgu[(size_t)x * 2 * F + f] = dh * u * s * (1.0f + g * (1.0f - s));
    dgu[(size_t)x * 2 * F + F + f] = dh * sl;
}

// per (row x, c): dx = dg . W_gate[:, c] + du . W_up[:, c], to buffer order
__global__ __launch_bounds__(kThreads) void bwd_f32_dx_kernel(int N, int E, int H, int F,
                                                              const int32_t* __restrict__ sched,
                                                              const int32_t* __restrict__ vrow,
                                                              const float* __restrict__ dgu,
                                                              const float* __restrict__ wg,
                                                              const float* __restrict__ wu,
                                                              float* __restrict__ dbuf)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)N * H) return;
    const int x = (int)(i / H), c = (int)(i % H);
    const int e = expert_of_row(x, E, sched + E + 1);
    const size_t FH = (size_t)F * H;
    const float* d = dgu + (size_t)x * 2 * F;
    float acc = 0.f;
    for (int f = 0; f < F; ++f) {
        acc = fmaf(wg[e * FH + (size_t)f * H + c], d[f], acc);
        acc = fmaf(wu[e * FH + (size_t)f * H + c], d[F + f], acc);
    }
    dbuf[(size_t)vrow[x] * H + c] = acc;
}

// per (expert e, row m, column n) of the weight gradients, summed over e's
// rows in order: dW_down[e][o][f] = sum dy[r][o] h[r][f];
// dW_gate[e][f][c] = sum dg[r][f] x[r][c]; dW_up the same with du
__global__ __launch_bounds__(kThreads) void bwd_f32_wgrad_kernel(int E, int H, int F,
                                                                 const int32_t* __restrict__ sched,
                                                                 const float* __restrict__ xs,
                                                                 const float* __restrict__ dys,
                                                                 const float* __restrict__ dgu,
                                                                 const float* __restrict__ hb,
                                                                 float* __restrict__ dwg,
                                                                 float* __restrict__ dwu,
                                                                 float* __restrict__ dwd)
{
    const size_t FH = (size_t)F * H;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)E * 3 * FH) return;
    const int e = (int)(i / (3 * FH));
    const size_t j = (size_t)(i % (3 * FH));
    const int q = (int)(j / FH);
    const size_t w = j % FH;
    const int32_t* rs = sched + E + 1;
    const int r0 = rs[e], r1 = rs[e + 1];
    float acc = 0.f;
    if (q == 2) {  // dW_down [H][F]
        const int o = (int)(w / F), f = (int)(w % F);
        for (int r = r0; r < r1; ++r) acc = fmaf(dys[(size_t)r * H + o], hb[(size_t)r * F + f], acc);
        dwd[e * FH + w] = acc;
    } else {  // dW_gate / dW_up [F][H]
        const int f = (int)(w / H), c = (int)(w % H);
        for (int r = r0; r < r1; ++r)
            acc = fmaf(dgu[(size_t)r * 2 * F + q * F + f], xs[(size_t)r * H + c], acc);
        (q == 0 ? dwg : dwu)[e * FH + w] = acc;
    }
}

}  // namespace

hipError_t moe_launch_ffn_backward(const moe_shape_t& s, const void* buf, const int32_t* plan,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const void* gu, const void* dy, void* dbuf, float* dw_gate,
                                   float* dw_up, float* dw_down, char* ws, hipStream_t st,
                                   float* rgrad)
{
    const int64_t N = (int64_t)s.T * s.k;
    const moe::BwdWsLayout B = moe::bwd_ws_layout(s);
    int32_t* sched = reinterpret_cast<int32_t*>(ws + B.sched);
    int32_t* vrow = reinterpret_cast<int32_t*>(ws + B.vrow);
    // the zero page, then the by-expert schedule with 256-row M-tiles only
    zero_kernel<<<1, kThreads, 0, st>>>(reinterpret_cast<uint4*>(ws + B.zero), 32);
    hipError_t e = moe_launch_gemm_schedule_bm(s, plan, sched, vrow, st);
    if (e != hipSuccess) return e;
    BwdArgs a;
    a.G = s.E;
    a.H = s.H;
    a.F = s.F;
    a.N = (int)N;
    a.dx_split_max = moe::bwd_dx_split_max(s);
    a.dxpart = reinterpret_cast<float*>(ws + B.dxpart);
    a.rgroups = nullptr;
    a.rgrad = rgrad;
    int32_t* slot_of = reinterpret_cast<int32_t*>(ws + B.slot_of);
    if (rgrad && s.dtype == MOE_BF16) {
        int32_t* groups = reinterpret_cast<int32_t*>(ws + B.rgroups);
        const int nt = s.E + s.R * (s.E / s.R);
        replica_groups_kernel<<<(nt + kThreads - 1) / kThreads, kThreads, 0, st>>>(s.E, s.R, plan,
                                                                                 groups, slot_of);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        a.rgroups = groups;
    }
    a.sched = sched;
    a.vrow = vrow;
    a.xs = reinterpret_cast<const uint16_t*>(ws + B.xs);
    a.dys = reinterpret_cast<const uint16_t*>(ws + B.dys);
    a.wg = static_cast<const uint16_t*>(w_gate);
    a.wu = static_cast<const uint16_t*>(w_up);
    a.wd = static_cast<const uint16_t*>(w_down);
    // g | u saved by the training forward, else recomputed into the workspace
    a.gu = gu ? static_cast<uint16_t*>(const_cast<void*>(gu)) : reinterpret_cast<uint16_t*>(ws + B.gu);
    a.dgu = reinterpret_cast<uint16_t*>(ws + B.dgu);
    a.hb = reinterpret_cast<uint16_t*>(ws + B.hb);
    a.dxbuf = static_cast<uint16_t*>(dbuf);
    a.dwg = dw_gate;
    a.dwu = dw_up;
    a.dwd = dw_down;
    a.zero = ws + B.zero;
    const int grid = moe::kGemmMaxGrid;
    if (s.dtype == MOE_F32) {
        const float* xs = reinterpret_cast<const float*>(ws + B.xs);
        const float* dys = reinterpret_cast<const float*>(ws + B.dys);
        float* dgu = reinterpret_cast<float*>(ws + B.dgu);
        float* hb = reinterpret_cast<float*>(ws + B.hb);
        const float* wgf = static_cast<const float*>(w_gate);
        const float* wuf = static_cast<const float*>(w_up);
        const float* wdf = static_cast<const float*>(w_down);
        if (N > 0) {
            const int row_vecs = s.H * 4 / 16;
            const int64_t n = N * row_vecs;
            const unsigned gb = (unsigned)((n + kThreads - 1) / kThreads);
            gather_rows_kernel<<<gb, kThreads, 0, st>>>((int)N, row_vecs, vrow,
                                                        static_cast<const uint4*>(buf),
                                                        reinterpret_cast<uint4*>(ws + B.xs));
            gather_rows_kernel<<<gb, kThreads, 0, st>>>((int)N, row_vecs, vrow,
                                                        static_cast<const uint4*>(dy),
                                                        reinterpret_cast<uint4*>(ws + B.dys));
            const int64_t nf = N * s.F, nh = N * s.H;
            bwd_f32_rows_kernel<<<(unsigned)((nf + kThreads - 1) / kThreads), kThreads, 0, st>>>(
                (int)N, s.E, s.H, s.F, sched, xs, dys, wgf, wuf, wdf, dgu, hb);
            bwd_f32_dx_kernel<<<(unsigned)((nh + kThreads - 1) / kThreads), kThreads, 0, st>>>(
                (int)N, s.E, s.H, s.F, sched, vrow, dgu, wgf, wuf, static_cast<float*>(dbuf));
        }
        const int64_t nw = (int64_t)s.E * 3 * s.F * s.H;
        bwd_f32_wgrad_kernel<<<(unsigned)((nw + kThreads - 1) / kThreads), kThreads, 0, st>>>(
            s.E, s.H, s.F, sched, xs, dys, dgu, hb, dw_gate, dw_up, dw_down);
        return hipGetLastError();
    }
    if (N > 0) {
        const int row_vecs = s.H * 2 / 16;
        const int64_t n = N * row_vecs;
        const unsigned gb = (unsigned)((n + kThreads - 1) / kThreads);
        gather_rows_kernel<<<gb, kThreads, 0, st>>>((int)N, row_vecs, vrow,
                                                    static_cast<const uint4*>(buf),
                                                    reinterpret_cast<uint4*>(ws + B.xs));
        gather_rows_kernel<<<gb, kThreads, 0, st>>>((int)N, row_vecs, vrow,
                                                    static_cast<const uint4*>(dy),
                                                    reinterpret_cast<uint4*>(ws + B.dys));
        if (!gu) {
            dgrad_kernel<kGU><<<grid, kWThreads, 0, st>>>(a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        dgrad_kernel<kDH><<<grid, kWThreads, 0, st>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        dgrad_kernel<kDX><<<grid, kWThreads, 0, st>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (a.dx_split_max > 1) {
            const int64_t n4 = N * (s.H / 4);
            dx_fixup_kernel<<<(unsigned)((n4 + kThreads - 1) / kThreads), kThreads, 0, st>>>(a, grid);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    // weight gradients: one warp-specialised workgroup per CU
    wgrad_kernel<kWD><<<grid, kWThreads, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    wgrad_kernel<kWGU><<<grid, kWThreads, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.rgroups) {
        const int64_t FH = (int64_t)s.F * s.H;
        reduce_replicas_kernel<<<dim3(1024, s.E), kThreads, 0, st>>>(s.E, s.R, FH, slot_of, rgrad,
                                                                     dw_gate, dw_up, dw_down);
        e = hipGetLastError();
    }
    return e;
}
