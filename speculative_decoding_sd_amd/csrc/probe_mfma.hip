// Measurement probe (not part of the verify step): the sustained rate of
// bf16 MFMA 32x32x16 on this device when nothing but the matrix pipes works.
//
// Every wave holds twelve operand fragments in registers and issues, per
// iteration, the sixteen MFMAs of two k-steps on a 128 x 64 block of
// accumulators (4 x 2 tiles of 32 x 32), in the order the LM head's 256 x 256
// kernel issues them; eight waves per workgroup (two per SIMD), one
// workgroup per CU.  No memory traffic inside the loop, so the rate measures
// the matrix pipes at the clock the chip holds under that load.  With random
// operands the chip lowers its clock to stay within its power limit; with
// equal operands (little switching activity) it does not, which separates
// the power ceiling from the issue ceiling.  bench.py --mfma-ceiling times it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;
constexpr int kFrags = 12;  // per thread: 4 + 4 A fragments, 2 + 2 B fragments

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads, 1) void probe_mfma_bf16(const u32x4* __restrict__ ops,
                                                               float* __restrict__ sink,
                                                               int iters) {
    const int t = threadIdx.x;
    u32x4 a0[4], a1[4], b0[2], b1[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a0[i] = ops[i * kThreads + t];
        a1[i] = ops[(4 + i) * kThreads + t];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        b0[j] = ops[(8 + j) * kThreads + t];
        b1[j] = ops[(10 + j) * kThreads + t];
    }
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int idx = 0; idx < 8; ++idx) {
            acc[idx / 2][idx % 2] = mfma(a0[idx / 2], b0[idx % 2], acc[idx / 2][idx % 2]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int idx = 0; idx < 8; ++idx) {
            acc[idx / 2][idx % 2] = mfma(a1[idx / 2], b1[idx % 2], acc[idx / 2][idx % 2]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][j][r];
    sink[(size_t)blockIdx.x * kThreads + t] = s;
}

}  // namespace

// Launches the probe on `stream`: `blocks` workgroups of 512 threads, `iters`
// iterations of 16 MFMAs per wave (flops = blocks * 8 waves * iters * 16 *
// 32768).  `ops` (device) holds 12 * 512 16-byte operand fragments
// (ops_bytes >= 98304); `sink` (device) receives blocks * 512 floats.
// Returns 0, or -1 on a bad argument or launch error.
extern "C" int sdv_probe_mfma_bf16(const void* ops, size_t ops_bytes, float* sink,
                                   size_t sink_floats, int blocks, int iters, void* stream) {
    if (!ops || !sink || blocks <= 0 || iters <= 0) return -1;
    if (ops_bytes < (size_t)kFrags * kThreads * 16) return -1;
    if (sink_floats < (size_t)blocks * kThreads) return -1;
    probe_mfma_bf16<<<blocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)ops, sink, iters);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
