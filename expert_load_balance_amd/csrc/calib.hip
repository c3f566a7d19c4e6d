// calib.hip -- calibration probes for the measurements, the measured
// counterparts of the spec peaks the rooflines divide by: the bf16 MFMA rate
// this GPU sustains with no memory traffic at all, a plain streaming copy
// for HBM, and a read-only stream (the ceiling of a kernel that mostly
// reads, such as one streaming expert weights).
//
// Every wave runs four independent accumulator chains of
// v_mfma_f32_32x32x16_bf16, each on its own pair of operands, so
// consecutive MFMAs switch inputs the way a GEMM's do: the matrix cores
// draw the power of real data (operands that never change draw less and
// run at a higher clock under the power limit).
#include "common.h"

namespace {

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr int kChains = 4;

// eight bf16 values of magnitude in [2^-7, 2^-6) with hashed sign and
// mantissa bits (no zeros, no specials)
__device__ __forceinline__ probe_bf16x8 operand(unsigned seed)
{
    probe_bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        unsigned h = (seed * 8u + (unsigned)i + 1u) * 2654435761u;
        h ^= h >> 13;
        h *= 0x85ebca6bu;
        h ^= h >> 16;
        const unsigned short bits =
            (unsigned short)(((h >> 8) & 0x8000u) | (120u << 7) | (h & 0x7fu));
        v[i] = __builtin_bit_cast(__bf16, bits);
    }
    return v;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters,
                                                                  float* __restrict__ sink)
{
    const unsigned id = blockIdx.x * kProbeThreads + threadIdx.x;
    probe_bf16x8 a[kChains], b[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        a[c] = operand(id * 2u * kChains + 2u * c);
        b[c] = operand(id * 2u * kChains + 2u * c + 1u);
    }
    probe_f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[c][q] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int q = 0; q < 16; ++q) s += acc[c][q];
    sink[id] = s;  // keeps every chain live
}

// a streaming copy: each thread moves kCopyVecs 16-byte vectors per round
// (all loads issued before the stores), rounds striding over the grid
constexpr int kCopyVecs = 4;

__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const uint4* __restrict__ src,
                                                                  uint4* __restrict__ dst,
                                                                  int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads * kCopyVecs;
    for (int64_t base = ((int64_t)blockIdx.x * kProbeThreads) * kCopyVecs + threadIdx.x; base < n;
         base += stride) {
        uint4 v[kCopyVecs];
#pragma unroll
        for (int j = 0; j < kCopyVecs; ++j) {
            const int64_t i = base + (int64_t)j * kProbeThreads;
            if (i < n) v[j] = src[i];
        }
#pragma unroll
        for (int j = 0; j < kCopyVecs; ++j) {
            const int64_t i = base + (int64_t)j * kProbeThreads;
            if (i < n) dst[i] = v[j];
        }
    }
}

// a read-only stream: workgroup b reads bytes [b * chunk, (b + 1) * chunk)
// through a buffer descriptor that ends at its chunk (loads past the end
// return zeros and read no memory; the whole offset goes in the lane offset,
// which the range check covers), kReadDepth 16-byte loads in flight per
// lane; each thread folds every vector it reads into an XOR (so the loads
// stay live and the result can be checked).
constexpr int kReadDepth = 8;
constexpr int kReadStep = kProbeThreads * 16;  // bytes per load instruction per workgroup

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const char* __restrict__ src,
                                                                  int64_t bytes, int64_t chunk,
                                                                  unsigned* __restrict__ sink)
{
    const int64_t off = (int64_t)blockIdx.x * chunk;
    const int64_t len = off < bytes ? min(chunk, bytes - off) : 0;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + (off < bytes ? off : 0)), 0, (int)len, 0x00020000);
    const int voff = (int)threadIdx.x * 16;
    const int rounds = (int)((len + (int64_t)kReadStep * kReadDepth - 1) / ((int64_t)kReadStep * kReadDepth));
    probe_u32x4 v[kReadDepth];
    unsigned acc = 0;
#pragma unroll
    for (int j = 0; j < kReadDepth; ++j)
        v[j] = __builtin_bit_cast(probe_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + j * kReadStep, 0, 0));
    // round r folds the loads of round r - 1 as it issues its own, one at a
    // time, so kReadDepth - 1 loads stay in flight
    for (int r = 1; r < rounds; ++r) {
#pragma unroll
        for (int j = 0; j < kReadDepth; ++j) {
            acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
            v[j] = __builtin_bit_cast(probe_u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rs, voff + (r * kReadDepth + j) * kReadStep, 0, 0));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < kReadDepth; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" moe_status_t moe_probe_read(const void* d_src, size_t bytes, int32_t workgroups,
                                       uint32_t* d_sink, size_t sink_words, moe_stream_t stream)
{
    if (d_src == nullptr || d_sink == nullptr || bytes == 0 || bytes % 16 != 0 || workgroups < 1 ||
        reinterpret_cast<uintptr_t>(d_src) % 16 != 0 || sink_words < (size_t)workgroups * kProbeThreads)
        return MOE_EINVAL;
    // each workgroup's chunk: a multiple of 16 bytes, below 2^31 (the
    // descriptor's range and the 32-bit load offsets)
    const size_t chunk = (bytes / 16 + (size_t)workgroups - 1) / (size_t)workgroups * 16;
    if (chunk > ((size_t)1 << 31) - (size_t)kReadStep * kReadDepth) return MOE_EINVAL;
    read_probe_kernel<<<workgroups, kProbeThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const char*>(d_src), (int64_t)bytes, (int64_t)chunk, d_sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

extern "C" moe_status_t moe_probe_copy(const void* d_src, void* d_dst, size_t bytes,
                                       int32_t workgroups, moe_stream_t stream)
{
    if (d_src == nullptr || d_dst == nullptr || bytes == 0 || bytes % 16 != 0 || workgroups < 1 ||
        reinterpret_cast<uintptr_t>(d_src) % 16 != 0 || reinterpret_cast<uintptr_t>(d_dst) % 16 != 0)
        return MOE_EINVAL;
    copy_probe_kernel<<<workgroups, kProbeThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4*>(d_src), static_cast<uint4*>(d_dst), (int64_t)(bytes / 16));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

extern "C" moe_status_t moe_probe_mfma(int32_t workgroups, int32_t iters, float* d_sink,
                                       size_t sink_floats, moe_stream_t stream)
{
    if (workgroups < 1 || iters < 1 || d_sink == nullptr ||
        sink_floats < (size_t)workgroups * kProbeThreads)
        return MOE_EINVAL;
    mfma_probe_kernel<<<workgroups, kProbeThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        iters, d_sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}
