// LM head on gfx950: logits[m][v] = sum_k H[m][k] * W[v][k].
//
// [CSDN-MTP] "整体计算流程" step 4: the verified positions' hidden vectors are
// stacked into one matrix and multiplied by the output-layer weights in one
// product (hidden size -> vocabulary size).
//
// bf16 path: one workgroup per 128 x 128 output tile, k in steps of 64,
// double-buffered LDS tiles fed by 16-byte coalesced loads, 4 waves each
// owning a 64 x 64 sub-tile of 2 x 2 MFMA 32x32x16 accumulators (fp32),
// bf16 round-to-nearest-even epilogue.  Both operands are k-contiguous, so
// A and B fragments use the same LDS read pattern.  Tiles are ordered with the
// M tile fastest and handed out so that each XCD (own L2) gets a contiguous
// run of tiles: the M tiles sharing one W tile run on the same XCD, which
// reads that slice of W from HBM once.
#include "sdv_device.h"
#include "sdv_internal.h"

namespace sdv {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsStride = kBK + 8;  // bf16 per LDS row (144 bytes)
constexpr int kXcds = 8;

// Bijection from dispatch order to tile index when dispatch order i runs on
// XCD i % 8: XCD x receives tiles [first(x), first(x) + count(x)).
__device__ __forceinline__ int xcd_tile(int bid, int total) {
    const int q = total / kXcds, r = total % kXcds;
    const int x = bid % kXcds, idx = bid / kXcds;
    return (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
}

__global__ __launch_bounds__(256, 1) void lm_head_bf16(const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ B,
                                                       uint16_t* __restrict__ C, int M, int N,
                                                       int K) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLdsStride];
    const int tiles_m = (M + kBM - 1) / kBM;
    const int tiles_n = (N + kBN - 1) / kBN;
    const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 31, lh = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;

    // Global -> register staging: 4 x 16 bytes per operand per thread.
    u32x4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 3, kc = (c & 7) * 8;
            const int k = k0 + kc;
            const bool kin = k < K;
            const int gm = m0 + row, gn = n0 + row;
            ra[i] = (kin && gm < M) ? *(const u32x4*)(A + (size_t)gm * K + k) : u32x4{0, 0, 0, 0};
            rb[i] = (kin && gn < N) ? *(const u32x4*)(B + (size_t)gn * K + k) : u32x4{0, 0, 0, 0};
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 3, kc = (c & 7) * 8;
            *(u32x4*)(&sA[buf][row * kLdsStride + kc]) = ra[i];
            *(u32x4*)(&sB[buf][row * kLdsStride + kc]) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (K + kBK - 1) / kBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            u32x4 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i] = *(const u32x4*)(&sA[buf][(wm * 64 + i * 32 + ln) * kLdsStride + 16 * s + 8 * lh]);
                fb[i] = *(const u32x4*)(&sB[buf][(wn * 64 + i * 32 + ln) * kLdsStride + 16 * s + 8 * lh]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(fa[i], fb[j], acc[i][j]);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds column ln of each 32x32 block, rows mfma_row(r).
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int gn = n0 + wn * 64 + j * 32 + ln;
            if (gn >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm * 64 + i * 32 + mfma_row(r, lane);
                if (gm < M) C[(size_t)gm * N + gn] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
            }
        }
    }
}

// fp32 path: one wave per output element, lanes split k (coalesced rows),
// fixed-order butterfly reduction.
__global__ __launch_bounds__(256) void lm_head_f32(const float* __restrict__ A,
                                                   const float* __restrict__ B,
                                                   float* __restrict__ C, int M, int N, int K) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long e = (long)blockIdx.x * 4 + wave;
    if (e >= (long)M * N) return;
    const int m = (int)(e / N), n = (int)(e % N);
    const float* a = A + (size_t)m * K;
    const float* b = B + (size_t)n * K;
    float acc = 0.f;
    for (int k = lane; k < K; k += 64) acc += a[k] * b[k];
    acc = wave_sum_f(acc);
    if (lane == 0) C[(size_t)m * N + n] = acc;
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int sd_lm_head(int M, int hidden, int vocab, int dtype, const void* H, const void* W,
                          void* logits, void* stream) {
    clear_error();
    if (M <= 0 || hidden <= 0 || vocab <= 0)
        return fail(SD_EINVAL, "sd_lm_head: non-positive size");
    if (!H || !W || !logits) return fail(SD_EINVAL, "sd_lm_head: NULL pointer");
    if (dtype != SD_BF16 && dtype != SD_F32)
        return fail(SD_EINVAL, "sd_lm_head: unknown dtype %d", dtype);
    if (hidden % 8 != 0) return fail(SD_EUNSUPPORTED, "sd_lm_head: hidden must be a multiple of 8");
    if (!aligned16(H) || !aligned16(W) || !aligned16(logits))
        return fail(SD_EINVAL, "sd_lm_head: pointers must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    if (dtype == SD_F32) {
        const long total = (long)M * vocab;
        lm_head_f32<<<(unsigned)((total + 3) / 4), 256, 0, s>>>(
            (const float*)H, (const float*)W, (float*)logits, M, vocab, hidden);
        return check_launch("lm_head_f32");
    }
    const long tiles = (long)((M + kBM - 1) / kBM) * ((vocab + kBN - 1) / kBN);
    if (tiles > 0x7fffffffL) return fail(SD_EUNSUPPORTED, "sd_lm_head: too many tiles");
    lm_head_bf16<<<(unsigned)tiles, 256, 0, s>>>((const uint16_t*)H, (const uint16_t*)W,
                                                  (uint16_t*)logits, M, vocab, hidden);
    return check_launch("lm_head_bf16");
}
