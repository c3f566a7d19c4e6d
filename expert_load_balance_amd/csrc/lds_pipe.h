// lds_pipe.h -- internal helpers of the MFMA kernels that stage operands
// through LDS with global -> LDS copies (gfx950, wave64): the 128-byte row
// swizzle, the copy wrapper, explicit waits and a fence-free barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace lds {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// plain vector (not HIP's struct uint4) so staging arrays promote to registers
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Slot of K-chunk c (0..7) in LDS row r is c ^ swz(r): 8 consecutive rows
// reading one chunk hit 8 distinct 16-byte groups of a 128-byte bank line,
// 16 consecutive rows 16 distinct groups of a 256-byte line.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// Global -> LDS copy, 16 bytes per lane; lane l's bytes land at lds + 16 l.
// Written as asm so the compiler's wait-count pass does not see the slots as
// targets of outstanding loads (it would wait for every copy in flight before
// each LDS read); the kernel orders them itself with explicit vmcnt waits and
// barriers. m0 is reserved but unused by the compiler in these kernels; each
// copy sets it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16(const void* base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// The same copy through a buffer descriptor (base, byte range kCopyRange,
// 32-bit data format: the gfx9 family's raw-buffer setting). A lane whose
// offset is kZeroRow or more is out of the descriptor's range: the hardware
// reads no memory for it and writes zeros to its 16 LDS bytes. Padding rows
// of a ragged tile take kZeroRow, so their MFMAs multiply zeros (measured:
// zero operands draw less power, and these MFMAs run at a higher clock).
// Every other lane's offset must stay below kZeroRow.
constexpr uint32_t kZeroRow = 0xFFFFFFF0u;
constexpr uint32_t kCopyRange = kZeroRow;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_or_zero(const void* base, uint32_t voff, uint32_t lds)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    i32x4 rsrc;
    rsrc[0] = (int32_t)(uint32_t)b;
    rsrc[1] = (int32_t)(uint32_t)(b >> 32);  // stride 0, no swizzle
    rsrc[2] = (int32_t)kCopyRange;
    rsrc[3] = 0x00020000;  // data format 32
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// The same copy from a per-lane 64-bit address (no uniform base): for
// operands whose rows come from several places (a zero page for padding).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_at(const void* addr, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(addr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(VM) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in bits 15:14)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm()
{
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads (whose release
// half would wait for every copy in flight). LDS reads are complete
// (lgkmcnt(0)) before it; copies are covered by the explicit vmcnt waits.
__device__ __forceinline__ void slot_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
}

// A uniform read of a table no kernel writes while this one runs, as a scalar
// load: a vector load would make the compiler wait for every vector memory
// operation in flight (copies, stores) before its first use.
__device__ __forceinline__ int ldc(const int32_t* p, int i)
{
    typedef const __attribute__((address_space(4))) int32_t cint;
    return ((cint*)p)[i];
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uni_ptr(T* p)
{
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ bf16x8 lds_frag(const char* p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// MFMA fragment from a k-major LDS tile (rows = k, contiguous along m) with
// gfx950's transposing LDS read: within each 16-lane group, lane j of the
// result gets element j of the 16 x 4 block the group's lanes read (lane i
// reads 4 consecutive m at k-row i / 4), i.e. one column m, four k-rows. Two
// reads (k-rows 0-3 and 4-7 of the lane's eight) make the 8-element operand.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 lds_frag_tr(const char* p0, const char* p1)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) char*)p0));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) char*)p1));
    const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}

}  // namespace lds
}  // namespace moe
