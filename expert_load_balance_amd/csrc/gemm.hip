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
// bf16 path: v_mfma_f32_16x16x32_bf16 (fp32 accumulate), 128x128 workgroup
// tiles, 64-deep K steps double-buffered through LDS. Workgroup ids run
// M-tile fastest so the M-tiles that share a weight tile are in flight
// together and the weight bytes come from HBM once.
#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBM = 128;   // rows per tile (both kernels)
constexpr int kBK = 64;    // K per LDS stage
constexpr int kLds = kBK + 8;  // padded LDS row (bf16 elements): 144 bytes

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
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// ---------------------------------------------------------------- bf16 ----
// gate/up: tile = 128 rows x 64 F-columns of both gate and up (128 B rows).
// 4 waves in 2 (M) x 2 (N); each wave: 64 rows x 32 columns of gate and of up.
__global__ __launch_bounds__(kThreads) void gateup_bf16_kernel(
    int E, int R, int H, int F, int mtiles, const uint16_t* __restrict__ a,
    const int32_t* __restrict__ plan, const int32_t* __restrict__ sched,
    const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu, uint16_t* __restrict__ h)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLds];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * kLds];
    __shared__ int32_t rowmap[kBM];

    const int mt = blockIdx.x % mtiles;
    const int nt = blockIdx.x / mtiles;
    const Tile tile = find_tile(mt, E, kBM, sched);
    if (tile.rows <= 0) return;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int tid = threadIdx.x;
    if (tid < kBM) {
        const int v = tile.v0 + (tid < tile.rows ? tid : 0);
        rowmap[tid] = buf_row_of(tile.e, v, R, plan, L);
    }
    __syncthreads();

    const int n0 = nt * 64;
    const int lrow = tid >> 3;        // 0..31
    const int lcol = (tid & 7) * 8;   // bf16 offset of this thread's 16 bytes
    const uint16_t* arow[4];
    const uint16_t* brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = lrow + 32 * i;
        arow[i] = a + (size_t)rowmap[r] * H + lcol;
        const int br = r < 64 ? r : r - 64;
        const uint16_t* wbase = r < 64 ? wg : wu;
        brow[i] = wbase + ((size_t)tile.e * F + n0 + br) * H + lcol;
    }

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 15, fk = (lane >> 4) * 8;

    f32x4 accg[4][2], accu[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    uint4 ra[4], rb[4];
    const int KT = H / kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const uint4*>(arow[i]);
        rb[i] = *reinterpret_cast<const uint4*>(brow[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&As[0][(lrow + 32 * i) * kLds + lcol]) = ra[i];
        *reinterpret_cast<uint4*>(&Bs[0][(lrow + 32 * i) * kLds + lcol]) = rb[i];
    }
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) {
            const int ko = (kt + 1) * kBK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = *reinterpret_cast<const uint4*>(arow[i] + ko);
                rb[i] = *reinterpret_cast<const uint4*>(brow[i] + ko);
            }
        }
        const uint16_t* as = As[cur];
        const uint16_t* bs = Bs[cur];
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8 af[4], bgf[2], buf_[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_frag(as + (wm * 64 + i * 16 + fr) * kLds + kk + fk);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bgf[j] = lds_frag(bs + (wn * 32 + j * 16 + fr) * kLds + kk + fk);
                buf_[j] = lds_frag(bs + (64 + wn * 32 + j * 16 + fr) * kLds + kk + fk);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    accg[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bgf[j], accg[i][j], 0, 0, 0);
                    accu[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], buf_[j], accu[i][j], 0, 0, 0);
                }
        }
        if (kt + 1 < KT) {
            const int nb = cur ^ 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<uint4*>(&As[nb][(lrow + 32 * i) * kLds + lcol]) = ra[i];
                *reinterpret_cast<uint4*>(&Bs[nb][(lrow + 32 * i) * kLds + lcol]) = rb[i];
            }
        }
        __syncthreads();
    }

    // epilogue: h = silu(g) * u, rounded to bf16; output lane layout of the
    // 16x16 MFMA: column = lane % 16, rows 4 * (lane / 16) + r.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
                const int col = n0 + wn * 32 + j * 16 + (lane & 15);
                if (row < tile.rows) {
                    const float g = accg[i][j][r], u = accu[i][j][r];
                    h[(size_t)(tile.hrow0 + row) * F + col] = moe::f32_to_bf16_bits(moe::silu(g) * u);
                }
            }
}

// down: tile = 128 rows x 128 output columns; 4 waves 2 x 2, each 64 x 64.
__global__ __launch_bounds__(kThreads) void down_bf16_kernel(
    int E, int R, int H, int F, int mtiles, const uint16_t* __restrict__ h,
    const int32_t* __restrict__ plan, const int32_t* __restrict__ sched,
    const uint16_t* __restrict__ wd, uint16_t* __restrict__ y)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLds];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * kLds];
    __shared__ int32_t rowmap[kBM];

    const int mt = blockIdx.x % mtiles;
    const int nt = blockIdx.x / mtiles;
    const Tile tile = find_tile(mt, E, kBM, sched);
    if (tile.rows <= 0) return;
    const moe::PlanLayout L = moe::plan_layout(E, R);
    const int tid = threadIdx.x;
    if (tid < kBM) rowmap[tid] = tid < tile.rows ? buf_row_of(tile.e, tile.v0 + tid, R, plan, L) : -1;
    __syncthreads();

    const int n0 = nt * 128;
    const int lrow = tid >> 3;
    const int lcol = (tid & 7) * 8;
    const uint16_t* arow[4];
    const uint16_t* brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = lrow + 32 * i;
        const int ar = r < tile.rows ? r : 0;
        arow[i] = h + (size_t)(tile.hrow0 + ar) * F + lcol;
        const int bc = min(n0 + r, H - 1);
        brow[i] = wd + ((size_t)tile.e * H + bc) * F + lcol;
    }

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 15, fk = (lane >> 4) * 8;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[4], rb[4];
    const int KT = F / kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const uint4*>(arow[i]);
        rb[i] = *reinterpret_cast<const uint4*>(brow[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&As[0][(lrow + 32 * i) * kLds + lcol]) = ra[i];
        *reinterpret_cast<uint4*>(&Bs[0][(lrow + 32 * i) * kLds + lcol]) = rb[i];
    }
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) {
            const int ko = (kt + 1) * kBK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = *reinterpret_cast<const uint4*>(arow[i] + ko);
                rb[i] = *reinterpret_cast<const uint4*>(brow[i] + ko);
            }
        }
        const uint16_t* as = As[cur];
        const uint16_t* bs = Bs[cur];
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_frag(as + (wm * 64 + i * 16 + fr) * kLds + kk + fk);
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = lds_frag(bs + (wn * 64 + j * 16 + fr) * kLds + kk + fk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) {
            const int nb = cur ^ 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<uint4*>(&As[nb][(lrow + 32 * i) * kLds + lcol]) = ra[i];
                *reinterpret_cast<uint4*>(&Bs[nb][(lrow + 32 * i) * kLds + lcol]) = rb[i];
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
            if (row >= tile.rows) continue;
            const int brow_out = rowmap[row];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn * 64 + j * 16 + (lane & 15);
                if (col < H) y[(size_t)brow_out * H + col] = moe::f32_to_bf16_bits(acc[i][j][r]);
            }
        }
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

int max_mtiles(const moe_shape_t& s, int bm)
{
    const int64_t N = (int64_t)s.T * s.k;
    return (int)((N + bm - 1) / bm + s.E);
}

}  // namespace

hipError_t moe_launch_gemm_gateup(const moe_shape_t& s, const void* a, const int32_t* plan,
                                  const void* w_gate, const void* w_up, char* ws,
                                  hipStream_t st)
{
    const moe::WsLayout W = moe::ws_layout(s);
    int32_t* sched = reinterpret_cast<int32_t*>(ws + W.sched);
    const bool bf = s.dtype == MOE_BF16;
    const int bm = bf ? kBM : kFM;
    schedule_kernel<<<1, kThreads, 0, st>>>(s.E, s.R, bm, plan, sched);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s.T == 0) return e;
    const int mtiles = max_mtiles(s, bm);
    if (bf) {
        const int nt = s.F / 64;
        gateup_bf16_kernel<<<mtiles * nt, kThreads, 0, st>>>(
            s.E, s.R, s.H, s.F, mtiles, static_cast<const uint16_t*>(a), plan, sched,
            static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
            reinterpret_cast<uint16_t*>(ws + W.h));
    } else {
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
    const int bm = bf ? kBM : kFM;
    const int mtiles = max_mtiles(s, bm);
    if (bf) {
        const int nt = (s.H + 127) / 128;
        down_bf16_kernel<<<mtiles * nt, kThreads, 0, st>>>(
            s.E, s.R, s.H, s.F, mtiles, reinterpret_cast<const uint16_t*>(ws + W.h), plan, sched,
            static_cast<const uint16_t*>(w_down), static_cast<uint16_t*>(y));
    } else {
        const int nt = (s.H + kFM - 1) / kFM;
        down_f32_kernel<<<mtiles * nt, kThreads, 0, st>>>(
            s.E, s.R, s.H, s.F, mtiles, reinterpret_cast<const float*>(ws + W.h), plan, sched,
            static_cast<const float*>(w_down), static_cast<float*>(y));
    }
    return hipGetLastError();
}
