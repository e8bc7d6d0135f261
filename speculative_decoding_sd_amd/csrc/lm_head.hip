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

// ---------------------------------------------------------------------------
// Main bf16 path.  Computes the transposed tile D[v][m] = sum_k W[v][k] H[m][k]
// (A = W rows, B = H rows) so that each lane's MFMA accumulator holds four
// consecutive vocab entries of one output row: the epilogue stores 8 bytes.
// TN x TM tile (vocab x rows), k in stages of 32, four LDS stages filled by
// direct global->LDS DMA (global_load_lds_dwordx4) up to four stages ahead.  Each
// stage has its own __shared__ array, so the compiler's wait tracking sees
// which in-flight DMA a fragment read depends on; each wave waits for its own
// oldest stage (s_waitcnt vmcnt) before the workgroup barrier.
// LDS layout per stage: row r (W rows then H rows) holds 4 granules of 16
// bytes (8 k values); chunk c sits at slot c ^ ((r >> 2) & 3), so the 16 lanes
// of a quarter-wave reading 16 consecutive rows hit 16 distinct bank groups.
// ---------------------------------------------------------------------------
constexpr int kStages = 4;
constexpr int kBKs = 32;
constexpr int kStageRows = 512;  // largest TN + TM
__shared__ __attribute__((aligned(16))) uint16_t g_st0[kStageRows * kBKs];
__shared__ __attribute__((aligned(16))) uint16_t g_st1[kStageRows * kBKs];
__shared__ __attribute__((aligned(16))) uint16_t g_st2[kStageRows * kBKs];
__shared__ __attribute__((aligned(16))) uint16_t g_st3[kStageRows * kBKs];

template <int S>
__device__ __forceinline__ uint16_t* stage_buf() {
    return S == 0 ? g_st0 : S == 1 ? g_st1 : S == 2 ? g_st2 : g_st3;
}

__device__ __forceinline__ int swz(int row, int c) { return row * 4 + (c ^ ((row >> 2) & 3)); }

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left free), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void block_barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int TN, int TM, int WN, int WM>
struct LmTile {
    static constexpr int kRows = TN + TM;
    static constexpr int kDmaPerWave = kRows * 4 / 64 / 4;  // 64-granule DMA ops per wave per stage
    static constexpr int FN = TN / WN / 32;                  // 32-row MFMA blocks per wave (vocab)
    static constexpr int FM = TM / WM / 32;                  // 32-col MFMA blocks per wave (rows)
    static_assert(kRows * 4 % 256 == 0, "stage must split into whole wave DMAs");
    static_assert(kRows <= kStageRows, "stage buffer too small");
};

template <int TN, int TM, int WN, int WM, int S>
__device__ __forceinline__ void lm_issue(const uint16_t* __restrict__ W,
                                         const uint16_t* __restrict__ H, int n0, int m0, int M,
                                         int N, int K, int kt, int wave, int lane) {
    using T = LmTile<TN, TM, WN, WM>;
    uint16_t* buf = stage_buf<S>();
    const int k0 = kt * kBKs;
#pragma unroll
    for (int i = 0; i < T::kDmaPerWave; ++i) {
        const int g0 = (i * 4 + wave) * 64;
        const int g = g0 + lane;
        const int row = g >> 2;
        const int c = (g & 3) ^ ((row >> 2) & 3);
        const uint16_t* src;
        if (row < TN) {
            const int n = min(n0 + row, N - 1);
            src = W + (size_t)n * K + k0 + 8 * c;
        } else {
            const int m = min(m0 + row - TN, M - 1);
            src = H + (size_t)m * K + k0 + 8 * c;
        }
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + g0 * 8),
                                         16, 0, 0);
    }
}

// LDS byte address of a __shared__ element (for the inline-asm reads).
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// Fragment reads are issued as inline asm so the compiler does not treat
// them as reads of memory the in-flight LDS DMA writes (it would otherwise
// wait for every outstanding DMA, collapsing the pipeline).  The explicit
// lgkmcnt wait takes the fragments as in/out operands, so no MFMA using them
// can be scheduled before it.
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

template <int NA, int NB>
__device__ __forceinline__ void wait_frags(u32x4 (&a)[NA], u32x4 (&b)[NB]) {
    static_assert(NA + NB <= 8, "at most 8 fragments per wait");
    if constexpr (NA == 4 && NB == 4)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                       "+v"(b[2]), "+v"(b[3]));
    else if constexpr (NA == 4 && NB == 2)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]));
    else if constexpr (NA == 2 && NB == 2)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]));
    else
        static_assert(NA < 0, "unsupported fragment counts");
}

template <int TN, int TM, int WN, int WM, int S>
__device__ __forceinline__ void lm_read_frags(u32x4 (&fa)[TN / WN / 32],
                                              u32x4 (&fb)[TM / WM / 32], int s, int wn, int wm,
                                              int lane) {
    const uint16_t* buf = stage_buf<S>();
    const int ln = lane & 31, lh = lane >> 5;
    const int c = 2 * s + lh;
#pragma unroll
    for (int i = 0; i < TN / WN / 32; ++i)
        fa[i] = ds_read16(lds_addr(buf + swz(wn * (TN / WN) + i * 32 + ln, c) * 8));
#pragma unroll
    for (int j = 0; j < TM / WM / 32; ++j)
        fb[j] = ds_read16(lds_addr(buf + swz(TN + wm * (TM / WM) + j * 32 + ln, c) * 8));
}

template <int TN, int TM, int WN, int WM, int S>
__device__ __forceinline__ void lm_mfma(f32x16 (&acc)[TN / WN / 32][TM / WM / 32],
                                        const u32x4 (&fa)[TN / WN / 32],
                                        const u32x4 (&fb)[TM / WM / 32]) {
#pragma unroll
    for (int i = 0; i < TN / WN / 32; ++i)
#pragma unroll
        for (int j = 0; j < TM / WM / 32; ++j) acc[i][j] = mfma_32x32x16(fa[i], fb[j], acc[i][j]);
}

// One pipeline stage kt (buffer S).  On entry fa0/fb0 hold the stage's step-0
// fragments.  The workgroup barrier for stage kt+1 sits after step 0's MFMAs
// are queued, so the matrix pipe keeps working through the barrier and the
// next stage's step-0 fragment reads; the freed buffer S is refilled with
// stage kt+4 right after the barrier.
// No branch may separate an asm fragment read from its lgkmcnt wait: at a
// control-flow merge the compiler may copy the (not yet loaded) registers.
// So the reads are unconditional (the last stage reads a spent buffer whose
// values are never used) and K is a multiple of 4 stages.
template <int TN, int TM, int WN, int WM, int S>
__device__ __forceinline__ void lm_stage(
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ H,
    f32x16 (&acc)[TN / WN / 32][TM / WM / 32], u32x4 (&fa0)[TN / WN / 32],
    u32x4 (&fb0)[TM / WM / 32], int n0, int m0, int M, int N, int K, int kt, int nk, int wave,
    int wn, int wm, int lane) {
    using T = LmTile<TN, TM, WN, WM>;
    u32x4 fa1[T::FN], fb1[T::FM];
    lm_read_frags<TN, TM, WN, WM, S>(fa1, fb1, 1, wn, wm, lane);
    // sched_barrier(0) keeps the scheduler from moving the MFMA blocks across
    // the waits and barriers (they do not depend on the asm operands).
    __builtin_amdgcn_sched_barrier(0);
    lm_mfma<TN, TM, WN, WM, S>(acc, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    wait_frags(fa1, fb1);
    // Stage kt+1 must have landed; kt+2 and kt+3 may still be in flight.
    const int later = max(0, min(2, nk - 2 - kt));
    if (later == 2) wait_vmcnt<2 * T::kDmaPerWave>();
    else if (later == 1) wait_vmcnt<T::kDmaPerWave>();
    else wait_vmcnt<0>();
    block_barrier_lds();
    if (kt + kStages < nk)
        lm_issue<TN, TM, WN, WM, S>(W, H, n0, m0, M, N, K, kt + kStages, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
    lm_read_frags<TN, TM, WN, WM, (S + 1) % kStages>(fa0, fb0, 0, wn, wm, lane);
    __builtin_amdgcn_sched_barrier(0);
    lm_mfma<TN, TM, WN, WM, S>(acc, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    wait_frags(fa0, fb0);
}

template <int TN, int TM, int WN, int WM>
__global__ __launch_bounds__(256, 1) void lm_head_dma(const uint16_t* __restrict__ H,
                                                      const uint16_t* __restrict__ W,
                                                      uint16_t* __restrict__ C, int M, int N,
                                                      int K) {
    using T = LmTile<TN, TM, WN, WM>;
    const int tiles_m = (M + TM - 1) / TM;
    const int tiles_n = (N + TN - 1) / TN;
    const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int n0 = tn * TN, m0 = tm * TM;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave % WN, wm = wave / WN;
    const int ln = lane & 31, lh = lane >> 5;

    f32x16 acc[T::FN][T::FM];
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
        for (int j = 0; j < T::FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = K / kBKs;
    lm_issue<TN, TM, WN, WM, 0>(W, H, n0, m0, M, N, K, 0, wave, lane);
    lm_issue<TN, TM, WN, WM, 1>(W, H, n0, m0, M, N, K, 1, wave, lane);
    lm_issue<TN, TM, WN, WM, 2>(W, H, n0, m0, M, N, K, 2, wave, lane);
    lm_issue<TN, TM, WN, WM, 3>(W, H, n0, m0, M, N, K, 3, wave, lane);
    wait_vmcnt<3 * T::kDmaPerWave>();
    block_barrier_lds();
    u32x4 fa0[T::FN], fb0[T::FM];
    lm_read_frags<TN, TM, WN, WM, 0>(fa0, fb0, 0, wn, wm, lane);
    wait_frags(fa0, fb0);
    for (int kt = 0; kt < nk; kt += kStages) {  // nk is a multiple of kStages
        lm_stage<TN, TM, WN, WM, 0>(W, H, acc, fa0, fb0, n0, m0, M, N, K, kt, nk, wave, wn, wm, lane);
        lm_stage<TN, TM, WN, WM, 1>(W, H, acc, fa0, fb0, n0, m0, M, N, K, kt + 1, nk, wave, wn, wm,
                                    lane);
        lm_stage<TN, TM, WN, WM, 2>(W, H, acc, fa0, fb0, n0, m0, M, N, K, kt + 2, nk, wave, wn, wm,
                                    lane);
        lm_stage<TN, TM, WN, WM, 3>(W, H, acc, fa0, fb0, n0, m0, M, N, K, kt + 3, nk, wave, wn, wm,
                                    lane);
    }

    // Lane (ln, lh) holds D[n][m] for m = column ln of each block and, per
    // group q of four registers, the four consecutive n = 8q + 4lh .. +3.
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int j = 0; j < T::FM; ++j) {
        const int m = m0 + wm * (TM / WM) + j * 32 + ln;
        if (m >= M) continue;
        uint16_t* crow = C + (size_t)m * N;
#pragma unroll
        for (int i = 0; i < T::FN; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * (TN / WN) + i * 32 + 8 * q + 4 * lh;
                const f32x16& a = acc[i][j];
                if (vec && n + 3 < N) {
                    u32x2 w;
                    w.x = pack_bf16x2(a[4 * q + 0], a[4 * q + 1]);
                    w.y = pack_bf16x2(a[4 * q + 2], a[4 * q + 3]);
                    *(u32x2*)(crow + n) = w;
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (n + t < N) crow[n + t] = (uint16_t)f32_to_bf16_rne(a[4 * q + t]);
                }
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
    if (hidden % (kBKs * kStages) == 0) {
        // Tile rows to the batch: all rows in one tile where possible, so each
        // W tile is streamed from HBM once.
        int TM = M > 128 ? 256 : (M > 64 ? 128 : 64);
        const long tiles = (long)((M + TM - 1) / TM) * ((vocab + 255) / 256);
        if (tiles > 0x7fffffffL) return fail(SD_EUNSUPPORTED, "sd_lm_head: too many tiles");
        const uint16_t* h = (const uint16_t*)H;
        const uint16_t* w = (const uint16_t*)W;
        uint16_t* c = (uint16_t*)logits;
        if (TM == 256)
            lm_head_dma<256, 256, 2, 2><<<(unsigned)tiles, 256, 0, s>>>(h, w, c, M, vocab, hidden);
        else if (TM == 128)
            lm_head_dma<256, 128, 2, 2><<<(unsigned)tiles, 256, 0, s>>>(h, w, c, M, vocab, hidden);
        else
            lm_head_dma<256, 64, 4, 1><<<(unsigned)tiles, 256, 0, s>>>(h, w, c, M, vocab, hidden);
        return check_launch("lm_head_dma");
    }
    const long tiles = (long)((M + kBM - 1) / kBM) * ((vocab + kBN - 1) / kBN);
    if (tiles > 0x7fffffffL) return fail(SD_EUNSUPPORTED, "sd_lm_head: too many tiles");
    lm_head_bf16<<<(unsigned)tiles, 256, 0, s>>>((const uint16_t*)H, (const uint16_t*)W,
                                                  (uint16_t*)logits, M, vocab, hidden);
    return check_launch("lm_head_bf16");
}
