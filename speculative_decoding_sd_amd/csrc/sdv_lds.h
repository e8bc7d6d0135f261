// Device helpers for the attention kernels on gfx950: direct
// global->LDS DMA issued outside the compiler's view, explicit vmcnt waits,
// the transposing LDS reads, half-wave reductions and hardware bf16 packing.
#pragma once

#include "sdv_device.h"

namespace sdv {

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte-per-lane LDS DMA (global_load_lds_dwordx4): lane l's 16 bytes
// from gptr land at LDS byte address m0 + 16 l.  Issued from inline asm so that
// the compiler does not see the LDS write (it would otherwise wait for every
// DMA in flight before each LDS read); callers order it with explicit vmcnt
// waits (and barriers when other waves read the data).  The kernels that use
// it have no other M0 use.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(m0), "v"(gptr)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the release fence of __syncthreads (which would
// make the compiler wait for all memory operations in flight).
__device__ __forceinline__ void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane t receives element t%4
// of the 8-byte reads of lanes 4e + t/4 (e = 0..3).  With lane s reading four
// consecutive dims d0 + 4(s%4) .. +3 of key row key0 + s/4 of a row-major
// [key][dim] tile, lane t receives V[key0 .. key0+3][d0 + t]: the transposed
// operand of O^T += V^T P^T.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// ds_read_b64_tr_b8: in each group of 16 lanes, lane t receives byte t%8 of
// the 8-byte reads of lanes t/8 + 2e (e = 0..7), as byte e of its result.
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 lds_read_tr8(const char* p) {
    const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap exchanges the
// upper half of one copy with the lower half of the other: the pair then
// holds both halves' values in every lane).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two floats -> packed bf16 (lo in the low half), round to nearest even
// (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

}  // namespace sdv
