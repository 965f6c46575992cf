// Internal helpers shared by the gfx950 kernels of libpagedattn.
//
// Element formats, 16-byte vector types, wavefront DPP reductions, the
// asynchronous global->LDS copy and explicit memory-counter waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"

#ifndef PA_CHECK_CONTENTS
#define PA_CHECK_CONTENTS 0
#endif
#if PA_CHECK_CONTENTS
#include "pa_checks.hpp"
#endif

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Stored element formats, as template tags.
enum class Fmt { F32, F16, BF16, FP8 };

template <Fmt F> struct FmtBytes;
template <> struct FmtBytes<Fmt::F32> { static constexpr int value = 4; };
template <> struct FmtBytes<Fmt::F16> { static constexpr int value = 2; };
template <> struct FmtBytes<Fmt::BF16> { static constexpr int value = 2; };
template <> struct FmtBytes<Fmt::FP8> { static constexpr int value = 1; };

inline int dtype_bytes(int dtype) {
    switch (dtype) {
        case PA_DTYPE_F32: return 4;
        case PA_DTYPE_F16: return 2;
        case PA_DTYPE_BF16: return 2;
        case PA_DTYPE_FP8_E4M3: return 1;
        default: return 0;
    }
}

// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// a * b rounded to float and never fused into a later add.  The online
// softmax takes its running maximum of the scaled scores and then the
// exponent of (score - maximum): both must see the same rounded score, or the
// largest score's weight is 2^(unrounded - rounded) instead of exactly 1
// (hipcc contracts a * b - c into an fma by default).
__device__ __forceinline__ float mul_rounded(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

// Sum over groups of N consecutive lanes (N = 8 or 16, inside one DPP row);
// every lane of the group receives the group's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16, "group must be 8 or 16 lanes");
    x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
    x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
    x = dpp_add<0x141>(x);  // row_half_mirror: lane i <-> 7-i within 8
    if constexpr (N == 16) x = dpp_add<0x140>(x);  // row_mirror: lane i <-> 15-i within 16
    return x;
}

// --------------------------------------------------------- memory movement

// Asynchronous copy of 16 bytes per lane from global memory straight into
// LDS: lane l's bytes land at lds_addr + 16*l.  lds_addr must be
// wavefront-uniform.  Completion is counted by vmcnt; wait with wait_vmcnt
// before reading the destination.
__device__ __forceinline__ void dma16_to_lds(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_addr) : "memory");
}

// The same copy with the non-temporal hint, for data read exactly once (the
// K/V tiles): streamed lines are not kept in the caches at the expense of
// reused ones.  Measured on gfx950, the hint raises the rate of a paged tile
// stream by about an eighth.
__device__ __forceinline__ void dma16_to_lds_stream(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "{m0}"(lds_addr) : "memory");
}

// The same copies from a wavefront-uniform base (held in scalar registers)
// plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16_to_lds_s(const void* sbase, uint32_t off, uint32_t lds_addr) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma16_to_lds_stream_s(const void* sbase, uint32_t off, uint32_t lds_addr) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(sbase), "{m0}"(lds_addr) : "memory");
}

// Stores of a partition state, which the reduce kernel reads once right after
// the partition kernel.  Which hint pays depends on the kernel (same-box
// interleaved A/Bs, three rounds each): the GQA-4 kernel, whose states are
// few (3.3 MB on the gqa workload), runs 3% faster with ordinary stores that
// may leave them in the caches for the reduce (89.2 against 91.9 us); the
// generic kernel on the mha workload, which writes 21 MB of states, runs 3.2%
// faster with the non-temporal hint (881 against 910 us), and the FP8
// matrix-core kernel 0.7% faster (195.0 against 196.6 us).
__device__ __forceinline__ void store_state(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_state_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// A wave-uniform read of memory that no workgroup of the launch writes
// (lengths, the work order, scales), through the constant address space: the
// compiler then reads it with a scalar load even in a kernel that stores to
// other global memory, where it cannot prove the two apart and would issue a
// vector load and a wait for it instead.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace pa
