// tile_common.h -- device helpers shared by the gfx950 attention kernels (prefill forward and
// backward): bf16 vector types, the LDS chunk swizzles, the direct HBM -> LDS load, the
// transposing LDS read, cross-half lane reductions and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Chunk swizzles (physical chunk = logical chunk ^ swizzle(row)).  K rows are read
// 16 (or 8) at a time at one logical chunk by the S^T operand loads; V rows are read
// 8 at a time, 64 bytes each, by the transposing loads.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
    if constexpr (D == 128) return row & 15;
    else return (row ^ (row >> 3)) & 7;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
    if constexpr (D == 128) return 4 * (row & 3);
    else return 4 * ((row >> 1) & 1);
}

// 16-byte direct HBM -> LDS load from sbase + voff (sbase wave-uniform, in SGPRs; voff a
// per-lane byte offset): lane l's 16 bytes land at LDS byte lds_base + 16*l (lds_base is
// wave-uniform and goes through M0).  Written as inline asm on purpose: the instruction
// has no destination register, and hiding it from the compiler's wait-count pass stops
// that pass from assuming the in-flight write may alias every later LDS read of the
// other slots (it would then wait for the whole prefetch before the operand reads).
// The kernel itself waits for vmcnt(0) before the barrier that publishes a tile.
__device__ __forceinline__ void load_lds_16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory", "m0");
}

// The same pointer value taken from the first active lane, so that it lives in SGPRs.
__device__ __forceinline__ const u16* uniform_ptr(const u16* p) {
    const uint64_t x = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return (const u16*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

__device__ __forceinline__ i16x4 read_tr16(const char* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
}

// x + (value of x in lane ^ 32) and max of the two, through v_permlane32_swap (no LDS).
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Bijection blockIdx -> logical work id that keeps consecutive logical ids on one
// XCD (workgroups are dealt to the 8 XCDs round-robin by blockIdx).
__device__ __forceinline__ int xcd_remap(int x, int total) {
    constexpr int kXcd = 8;
    const int per = total / kXcd;
    if (x >= per * kXcd) return x;
    return (x % kXcd) * per + x / kXcd;
}

}  // namespace tile
}  // namespace flux
