// Device-side helpers shared by the gfx950 kernels of libsdv (not part of the
// public ABI).  CDNA4: 64-lane wavefronts, MFMA bf16 32x32x16 tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sdv.h"

namespace sdv {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// MI355X has 8 XCDs (each with its own L2); workgroups are dispatched to
// them round-robin, dispatch order i going to XCD i % 8.  xcd_tile maps the
// dispatch order to a tile index so that XCD x receives the contiguous run
// [first(x), first(x) + count(x)) of tiles; neighbouring tiles that share
// operands then share an L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int bid, int total) {
    const int q = total / kXcds, r = total % kXcds;
    const int x = bid % kXcds, idx = bid / kXcds;
    return (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float32 -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// MFMA D = A(32x16) * B(16x32) + C with bf16 inputs and fp32 accumulation.
// Operand lane layout (lane l, h = l / 32): A row l%32, k = 8h..8h+7;
// B column l%32, k = 8h..8h+7.  Result: lane l holds column l%32 and rows
// 8*(r/4) + 4h + r%4 for register r = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int mfma_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
    return v;
}

// Orderable 16-bit key of a bfloat16 value: larger key <=> larger value.
// -0 is folded onto +0 so equal values share one key.
__device__ __forceinline__ uint32_t bf16_key(uint32_t bits) {
    if (bits == 0x8000u) bits = 0;
    return (bits & 0x8000u) ? (~bits & 0xffffu) : (bits | 0x8000u);
}

__device__ __forceinline__ uint32_t key_to_bf16(uint32_t key) {
    return (key & 0x8000u) ? (key & 0x7fffu) : (~key & 0xffffu);
}

// Orderable 32-bit key of a float32 value (-0 folded onto +0).
__device__ __forceinline__ uint32_t f32_key(uint32_t bits) {
    if (bits == 0x80000000u) bits = 0;
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

__device__ __forceinline__ uint32_t key_to_f32(uint32_t key) {
    return (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
}

__device__ __forceinline__ void set_error(int32_t* err, int bits) {
    if (err) atomicOr(err, bits);
}

}  // namespace sdv
