// Measurement probe (not part of the verify step): the read bandwidth this
// device sustains from HBM with a plain streaming kernel, the practical
// ceiling for the HBM-bound calls (attention, streaming LM head, accept).
//
// Each workgroup reads contiguous tiles of 256 x 8 16-byte words (its 256
// threads read consecutive words, eight loads in flight per thread), tiles
// at a grid stride, and folds them with XOR into one word per thread (so no
// load can be dropped); one store per thread at the end.  The buffer is
// far larger than the L2 caches and the 256 MB MALL, so every byte comes
// from HBM once per launch.  bench.py --hbm-ceiling times it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void probe_hbm_read(const u32x4* __restrict__ src,
                                                           size_t n_words,
                                                           uint32_t* __restrict__ sink) {
    constexpr size_t kTile = (size_t)kThreads * kUnroll;
    const size_t stride = (size_t)gridDim.x * kTile;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t t = (size_t)blockIdx.x * kTile; t < n_words; t += stride) {
        const size_t i = t + threadIdx.x;
        if (t + kTile <= n_words) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * kThreads];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
        } else {
            for (size_t j = i; j < n_words; j += kThreads) acc ^= src[j];
        }
    }
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

// Launches the probe on `stream`: `blocks` workgroups of 256 threads read
// n_bytes (a multiple of 16) from `src` (device); `sink` (device) receives
// blocks * 256 words.  Returns 0, or -1 on a bad argument or launch error.
extern "C" int sdv_probe_hbm_read(const void* src, size_t n_bytes, uint32_t* sink,
                                  size_t sink_words, int blocks, void* stream) {
    if (!src || !sink || blocks <= 0 || n_bytes == 0 || n_bytes % 16 != 0) return -1;
    if (sink_words < (size_t)blocks * kThreads) return -1;
    probe_hbm_read<<<blocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, n_bytes / 16,
                                                                 sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
