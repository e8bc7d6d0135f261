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
#include <algorithm>

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
// Main bf16 path (lm_head_ring for 256 x 256 tiles, lm_head_stream for 256 x
// 128, 256 x 64 and 128 x 192, vocabulary x rows).  Both compute the transposed tile D[v][m] =
// sum_k W[v][k] H[m][k] (A = W rows, B = H rows) so that each lane's MFMA
// accumulator holds four consecutive vocab entries of one output row: the
// epilogue stores 8 bytes.  k advances 64 per stage, staged in LDS by direct
// global->LDS DMA (global_load_lds_dwordx4); every DMA request covers whole
// 128-byte rows of W and H (full L2 lines).
// LDS layout of a k-slice: row r holds 8 granules of 16 bytes; granule c sits
// at slot c ^ ((r/2) % 8).  A ds_read_b128 is served 16 lanes (16 rows, one
// logical granule) per pass over the 64 banks; with the XOR those 16 rows land
// in 16 distinct 16-byte bank groups.
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int swz(int row, int c) {
    static_assert(BK == 64, "64-wide k-slices only");
    return row * 8 + (c ^ ((row >> 1) & 7));
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left free), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void block_barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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
    else if constexpr (NA == 2 && NB == 3)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]));
    else if constexpr (NA == 1 && NB == 3)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]));
    else
        static_assert(NA < 0, "unsupported fragment counts");
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles.  Eight waves of 128 (vocab) x 64 (rows), two per SIMD
// (accumulators in 128 registers): a wave waiting on an LDS read or the barrier
// leaves the matrix unit to the other wave of its SIMD.
// The W and H k-slices (64 wide, 32 KB each) are staged separately in a ring of
// five LDS slots: slice j of W in slot 2j % 5, of H in slot (2j+1) % 5.  While
// stage kt computes from its two slots, stage kt+1 is resident or landing and
// the fifth slot receives W of kt+2.  This lets a stage's DMAs be spread over
// all four of its k-steps (two per wave and step) rather than issued as one
// burst after the stage barrier; the burst kept the vector-memory queue full
// and stalled MFMA issue for about a third of every stage.
// Barrier B_kt sits at the start of stage kt's last k-step.  Past it, stage
// kt+1 has landed and stage kt's slots are free (every wave then holds the last
// step's fragments in registers).  DMA issue per stage kt:
//   step 0:     H of kt+1, ops 2-3 (ops 0-1 went out after B_{kt-1})
//   steps 1, 2: W of kt+2, ops 0-1, then 2-3
//   B_kt, waiting until at most W of kt+2 is in flight; step 3: H of kt+2, ops 0-1
// Within a step the next step's six fragment reads and the two DMAs are
// interleaved with the eight MFMAs, so neither the LDS nor the vector-memory
// queue takes the issue slot in one block.
// ---------------------------------------------------------------------------
constexpr int kRingSlotBytes = 256 * 64 * 2;
constexpr int kRingSlots = 5;
__shared__ __attribute__((aligned(1024))) uint16_t g_ring[kRingSlots * kRingSlotBytes / 2];

// DMA op i (0..3) of one operand slice into the slot at byte offset slot_off:
// lane l of wave w writes granule g = 64 (8 i + w) + l, i.e. row g / 8, stored
// granule g % 8 (the sources were set up by the same mapping).
__device__ __forceinline__ void ring_dma(const uint16_t* const* src, int i, int kt,
                                         uint32_t slot_off, int wave) {
    const int g0 = (i * 8 + wave) * 64;
    __builtin_amdgcn_global_load_lds(src[i] + (size_t)kt * 64,
                                     (__attribute__((address_space(3))) void*)(
                                         g_ring + (slot_off + g0 * 16) / 2),
                                     16, 0, 0);
}

// One k-step: the eight MFMAs on (ca, cb); after MFMA r < 6 the read of the
// next step's fragment r (four of W from slot rW, then two of H from slot rH,
// at k-step `step`); DMA op o0 after MFMA 1, op o0+1 after MFMA 3.  Every group
// is fenced so that this order survives scheduling.
__device__ __forceinline__ void ring_step(f32x16 (&acc)[4][2], const u32x4 (&ca)[4],
                                          const u32x4 (&cb)[2], u32x4 (&na)[4], u32x4 (&nb)[2],
                                          uint32_t rW, uint32_t rH, int step, int wn, int wm,
                                          int lane, const uint16_t* const* src, int o0, int kt,
                                          uint32_t slot_off, int wave) {
    const int ln = lane & 31, c = 2 * step + (lane >> 5);
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) {
        acc[idx / 2][idx % 2] = mfma_32x32x16(ca[idx / 2], cb[idx % 2], acc[idx / 2][idx % 2]);
        if (idx < 4)
            na[idx] = ds_read16(rW + swz<64>(wn * 128 + idx * 32 + ln, c) * 16);
        else if (idx < 6)
            nb[idx - 4] = ds_read16(rH + swz<64>(wm * 64 + (idx - 4) * 32 + ln, c) * 16);
        if (idx == 1) ring_dma(src, o0, kt, slot_off, wave);
        if (idx == 3) ring_dma(src, o0 + 1, kt, slot_off, wave);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__global__ __launch_bounds__(512, 1) void lm_head_ring(const uint16_t* __restrict__ H,
                                                       const uint16_t* __restrict__ W,
                                                       uint16_t* __restrict__ C, int M, int N,
                                                       int K) {
    constexpr uint32_t S = kRingSlotBytes;
    const int tiles_m = (M + 255) / 256;
    const int tiles_n = (N + 255) / 256;
    const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int n0 = tn * 256, m0 = tm * 256;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave % 2, wm = wave / 2;
    const int ln = lane & 31, lh = lane >> 5;
    const uint32_t lds0 = lds_addr(g_ring);

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = K / 64;
    // Per-lane sources of the four DMA ops of a W and an H slice at k = 0.
    // Rows past the matrix ends re-read the last row (never stored).
    const uint16_t* sw[4];
    const uint16_t* sh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = (i * 8 + wave) * 64 + lane;
        const int row = g / 8, c = (g % 8) ^ ((row >> 1) & 7);
        sw[i] = W + (size_t)min(n0 + row, N - 1) * K + 8 * c;
        sh[i] = H + (size_t)min(m0 + row, M - 1) * K + 8 * c;
    }
    // Prologue: W and H of slice 0, W of slice 1, ops 0-1 of H of slice 1
    // (slots 0-3), then wait for slice 0.  Slices past the end re-read the
    // last one into free slots; the kernel waits for them before it ends.
    const int kn = min(1, nk - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) ring_dma(sw, i, 0, 0, wave);
#pragma unroll
    for (int i = 0; i < 4; ++i) ring_dma(sh, i, 0, S, wave);
#pragma unroll
    for (int i = 0; i < 4; ++i) ring_dma(sw, i, kn, 2 * S, wave);
    ring_dma(sh, 0, kn, 3 * S, wave);
    ring_dma(sh, 1, kn, 3 * S, wave);
    wait_vmcnt<6>();
    block_barrier_lds();
    u32x4 fa0[4], fb0[2], fa1[4], fb1[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa0[i] = ds_read16(lds0 + swz<64>(wn * 128 + i * 32 + ln, lh) * 16);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        fb0[j] = ds_read16(lds0 + S + swz<64>(wm * 64 + j * 32 + ln, lh) * 16);
    wait_frags(fa0, fb0);
    // No branch may separate an asm fragment read from its lgkmcnt wait (at a
    // control-flow merge the compiler may copy the not yet loaded registers):
    // the loop body is straight-line, slot indices are computed.
    int q = 0;  // slot of W of slice kt: (2 kt) % 5
    for (int kt = 0; kt < nk; ++kt) {
        const int q1 = q + 1 - (q + 1 >= 5 ? 5 : 0), q2 = q + 2 - (q + 2 >= 5 ? 5 : 0);
        const int q3 = q + 3 - (q + 3 >= 5 ? 5 : 0), q4 = q + 4 - (q + 4 >= 5 ? 5 : 0);
        const uint32_t aW = lds0 + q * S, aH = lds0 + q1 * S;
        const uint32_t nW = lds0 + q2 * S, nH = lds0 + q3 * S;
        const int k1 = min(kt + 1, nk - 1), k2 = min(kt + 2, nk - 1);
        ring_step(acc, fa0, fb0, fa1, fb1, aW, aH, 1, wn, wm, lane, sh, 2, k1, q3 * S, wave);
        wait_frags(fa1, fb1);
        ring_step(acc, fa1, fb1, fa0, fb0, aW, aH, 2, wn, wm, lane, sw, 0, k2, q4 * S, wave);
        wait_frags(fa0, fb0);
        ring_step(acc, fa0, fb0, fa1, fb1, aW, aH, 3, wn, wm, lane, sw, 2, k2, q4 * S, wave);
        wait_frags(fa1, fb1);
        // B_kt: slice kt+1 landed (only W of kt+2 may still be in flight).
        wait_vmcnt<4>();
        block_barrier_lds();
        __builtin_amdgcn_sched_barrier(0);
        ring_step(acc, fa1, fb1, fa0, fb0, nW, nH, 0, wn, wm, lane, sh, 0, k2, q * S, wave);
        wait_frags(fa0, fb0);
        q = q2;
    }
    wait_vmcnt<0>();

    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm * 64 + j * 32 + ln;
        if (m >= M) continue;
        uint16_t* crow = C + (size_t)m * N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * 128 + i * 32 + 8 * g + 4 * lh;
                const f32x16& a = acc[i][j];
                if (vec && n + 3 < N) {
                    u32x2 w;
                    w.x = pack_bf16x2(a[4 * g + 0], a[4 * g + 1]);
                    w.y = pack_bf16x2(a[4 * g + 2], a[4 * g + 3]);
                    *(u32x2*)(crow + n) = w;
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (n + t < N) crow[n + t] = (uint16_t)f32_to_bf16_rne(a[4 * g + t]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 128- and 64-row tiles (small batches, where the LM head streams W from HBM):
// a ring of NST whole stages (W and H k-slices of 64, (TN + TM) rows each)
// in the same 160 KB of LDS, three stages of 48 KB for 256 x 128 and four of
// 40 KB for 256 x 64 and 128 x 192, so NST - 1 stages are in flight while one
// computes.  WN x WM waves (the 128 x 192 tile: eight of 32 x 96, two per
// SIMD, 3-5% faster than four of 64 x 96 on 129-192-row batches).
// The refill of the stage buffer freed at a barrier is spread over the four
// k-steps that follow it, a quarter of the ops per step, each interleaved with
// the MFMAs and the next step's fragment reads.  Barrier B_kt at the start of
// stage kt's last k-step: past it stage kt+1 has landed and stage kt's buffer
// is free; after it go a quarter of the ops of slice kt + NST (into that
// buffer), the other three quarters in steps 0-2 of stage kt+1.
// ---------------------------------------------------------------------------
template <int TN_, int TM_, int WN_, int WM_, int NST>
struct StreamTile {
    static constexpr int NW = WN_ * WM_;
    static constexpr int NT = 64 * NW;
    static constexpr int TN = TN_, TM = TM_, WN = WN_, WM = WM_;
    static constexpr int kRows = TN + TM;
    static constexpr int kStageBytes = kRows * 128;  // 64 bf16 of k per row
    static constexpr int kOps = kRows * 8 / NT;      // DMA ops per wave per stage
    static constexpr int FN = TN / WN / 32, FM = TM / WM / 32;
    static_assert(kRows * 8 % NT == 0, "stage must split into whole wave DMAs");
    static_assert(NST >= 3 && NST * kStageBytes <= kRingSlots * kRingSlotBytes, "LDS");
    static_assert((NST - 2) * kOps + kOps / 4 < 64, "vmcnt field");
};

// DMA op i of a stage into the buffer at byte offset off: lane l of wave w
// writes granule g = 64 (NW i + w) + l, row g / 8 (W rows, then H rows).
template <class T>
__device__ __forceinline__ void stream_dma(const uint16_t* const* src, int i, int kt,
                                           uint32_t off, int wave) {
    const int g0 = (i * T::NW + wave) * 64;
    __builtin_amdgcn_global_load_lds(src[i] + (size_t)kt * 64,
                                     (__attribute__((address_space(3))) void*)(
                                         g_ring + (off + g0 * 16) / 2),
                                     16, 0, 0);
}

// One k-step: the MFMAs on (ca, cb), the next step's fragment reads (stage at
// LDS byte address rb, k-step `step`) and DMA ops [D0, D1) of k-slice kt into
// buffer offset doff, spread evenly over the MFMAs in fenced groups.
template <class T, int D0, int D1>
__device__ __forceinline__ void stream_step(f32x16 (&acc)[T::FN][T::FM], const u32x4 (&ca)[T::FN],
                                            const u32x4 (&cb)[T::FM], u32x4 (&na)[T::FN],
                                            u32x4 (&nb)[T::FM], uint32_t rb, int step, int wn,
                                            int wm, int lane, const uint16_t* const* src, int kt,
                                            uint32_t doff, int wave) {
    constexpr int FN = T::FN, FM = T::FM, NMF = FN * FM, NR = FN + FM, ND = D1 - D0;
    const int ln = lane & 31, c = 2 * step + (lane >> 5);
#pragma unroll
    for (int idx = 0; idx < NMF; ++idx) {
        acc[idx / FM][idx % FM] = mfma_32x32x16(ca[idx / FM], cb[idx % FM], acc[idx / FM][idx % FM]);
#pragma unroll
        for (int r = idx * NR / NMF; r < (idx + 1) * NR / NMF; ++r) {
            if (r < FN)
                na[r] = ds_read16(rb + swz<64>(wn * (FN * 32) + r * 32 + ln, c) * 16);
            else
                nb[r - FN] = ds_read16(
                    rb + swz<64>(T::TN + wm * (FM * 32) + (r - FN) * 32 + ln, c) * 16);
        }
#pragma unroll
        for (int d = idx * ND / NMF; d < (idx + 1) * ND / NMF; ++d)
            stream_dma<T>(src, D0 + d, kt, doff, wave);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int TN, int TM, int WN, int WM, int NST>
__global__ __launch_bounds__(64 * WN * WM, 1) void lm_head_stream(const uint16_t* __restrict__ H,
                                                             const uint16_t* __restrict__ W,
                                                             uint16_t* __restrict__ C, int M,
                                                             int N, int K, int nw) {
    using T = StreamTile<TN, TM, WN, WM, NST>;
    constexpr int FN = T::FN, FM = T::FM, OPS = T::kOps;
    constexpr uint32_t SB = T::kStageBytes;
    constexpr int C1 = OPS / 4, C2 = OPS / 2, C3 = 3 * OPS / 4;
    // Block (tm, tn) covers vocabulary rows [tn nw, min((tn + 1) nw, N)):
    // nw <= TN (a multiple of 8) is chosen by the launcher so that the
    // blocks fill whole rounds of the CUs; rows of the TN-row tile past that
    // range re-read its last row and are never stored.
    const int tiles_m = (M + TM - 1) / TM;
    const int tiles_n = (N + nw - 1) / nw;
    const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int n0 = tn * nw, m0 = tm * TM;
    const int n_end = min(n0 + nw, N);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wn = wave % WN, wm = wave / WN;
    const int ln = lane & 31, lh = lane >> 5;
    const uint32_t lds0 = lds_addr(g_ring);

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = K / 64;
    // Rows past the matrix ends re-read the last row (never stored).
    const uint16_t* src[OPS];
#pragma unroll
    for (int i = 0; i < OPS; ++i) {
        const int g = (i * T::NW + wave) * 64 + lane;
        const int row = g / 8, c = (g % 8) ^ ((row >> 1) & 7);
        src[i] = row < TN ? W + (size_t)min(n0 + row, n_end - 1) * K + 8 * c
                          : H + (size_t)min(m0 + row - TN, M - 1) * K + 8 * c;
    }
    // Prologue: slices 0 .. NST-2 whole, the first quarter of slice NST-1;
    // slices past the end re-read the last one into free buffers (waited for
    // before the kernel ends).
#pragma unroll
    for (int st = 0; st < NST - 1; ++st)
#pragma unroll
        for (int i = 0; i < OPS; ++i) stream_dma<T>(src, i, min(st, nk - 1), st * SB, wave);
#pragma unroll
    for (int i = 0; i < C1; ++i) stream_dma<T>(src, i, min(NST - 1, nk - 1), (NST - 1) * SB, wave);
    wait_vmcnt<(NST - 2) * OPS + C1>();
    block_barrier_lds();
    u32x4 fa0[FN], fb0[FM], fa1[FN], fb1[FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
        fa0[i] = ds_read16(lds0 + swz<64>(wn * (FN * 32) + i * 32 + ln, lh) * 16);
#pragma unroll
    for (int j = 0; j < FM; ++j)
        fb0[j] = ds_read16(lds0 + swz<64>(TN + wm * (FM * 32) + j * 32 + ln, lh) * 16);
    wait_frags(fa0, fb0);
    // Straight-line body (no branch between an asm read and its wait).
    int b = 0;  // buffer of stage kt
    for (int kt = 0; kt < nk; ++kt) {
        const int bp = b == 0 ? NST - 1 : b - 1;  // freed at B_{kt-1}: slice kt + NST - 1
        const int bn = b + 1 == NST ? 0 : b + 1;  // stage kt + 1
        const uint32_t cur = lds0 + b * SB, nxt = lds0 + bn * SB;
        const int kr = min(kt + NST - 1, nk - 1), kr2 = min(kt + NST, nk - 1);
        stream_step<T, C1, C2>(acc, fa0, fb0, fa1, fb1, cur, 1, wn, wm, lane, src, kr, bp * SB, wave);
        wait_frags(fa1, fb1);
        stream_step<T, C2, C3>(acc, fa1, fb1, fa0, fb0, cur, 2, wn, wm, lane, src, kr, bp * SB, wave);
        wait_frags(fa0, fb0);
        stream_step<T, C3, OPS>(acc, fa0, fb0, fa1, fb1, cur, 3, wn, wm, lane, src, kr, bp * SB,
                                wave);
        wait_frags(fa1, fb1);
        // B_kt: slice kt+1 landed (slices kt+2 .. kt+NST-1 may be in flight).
        wait_vmcnt<(NST - 2) * OPS>();
        block_barrier_lds();
        __builtin_amdgcn_sched_barrier(0);
        stream_step<T, 0, C1>(acc, fa1, fb1, fa0, fb0, nxt, 0, wn, wm, lane, src, kr2, b * SB, wave);
        wait_frags(fa0, fb0);
        b = bn;
    }
    wait_vmcnt<0>();

    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int m = m0 + wm * (TM / WM) + j * 32 + ln;
        if (m >= M) continue;
        uint16_t* crow = C + (size_t)m * N;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * (TN / WN) + i * 32 + 8 * g + 4 * lh;
                const f32x16& a = acc[i][j];
                if (vec && n + 3 < n_end) {
                    u32x2 w;
                    w.x = pack_bf16x2(a[4 * g + 0], a[4 * g + 1]);
                    w.y = pack_bf16x2(a[4 * g + 2], a[4 * g + 3]);
                    *(u32x2*)(crow + n) = w;
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (n + t < n_end) crow[n + t] = (uint16_t)f32_to_bf16_rne(a[4 * g + t]);
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
    if (hidden % 128 == 0) {
        // Tile rows to the batch: all rows in one tile where possible, so each
        // W tile is streamed from HBM once.  When 256 x 256 tiles would leave
        // CUs idle (a small vocabulary), batches of up to 192 rows take 128 x
        // 192 tiles (all rows, twice the W tiles), larger ones 128-row tiles
        // (the W tile is then read by two workgroups of one XCD).
        int TM = M > 128 ? 256 : (M > 64 ? 128 : 64);
        int num_cus = 0;
        const int rc = cu_count("sd_lm_head", &num_cus);
        if (rc != SD_OK) return rc;
        if (TM == 256 && (long)((M + 255) / 256) * ((vocab + 255) / 256) < num_cus)
            TM = M <= 192 ? 192 : 128;
        const int TN = TM == 192 ? 128 : 256;
        const long tiles_m = (M + TM - 1) / TM;
        long tiles = tiles_m * ((vocab + TN - 1) / TN);
        // Streaming tiles (one workgroup per CU at a time): narrow the
        // vocabulary range per block so that the blocks fill whole rounds of
        // the CUs (a 64 x 5120 x 152064 head: 594 tiles of 256 rows are 2.3
        // rounds, 761 blocks of 200 rows 3 rounds), keeping a multiple of 8
        // and at least half the tile: every block streams all of its M tile's
        // H rows, so narrower blocks would multiply those reads.
        int nw = TN;
        if (TM != 256) {
            const long rounds = (tiles + num_cus - 1) / num_cus;
            const long per_m = (rounds * num_cus + tiles_m - 1) / tiles_m;
            const long w = ((vocab + per_m - 1) / per_m + 7) / 8 * 8;
            nw = (int)std::min<long>(TN, std::max<long>(TN / 2, w));
            tiles = tiles_m * ((vocab + nw - 1) / nw);
        }
        if (tiles > 0x7fffffffL) return fail(SD_EUNSUPPORTED, "sd_lm_head: too many tiles");
        const uint16_t* h = (const uint16_t*)H;
        const uint16_t* w = (const uint16_t*)W;
        uint16_t* c = (uint16_t*)logits;
        if (TM == 256)
            lm_head_ring<<<(unsigned)tiles, 512, 0, s>>>(h, w, c, M, vocab, hidden);
        else if (TM == 192)
            lm_head_stream<128, 192, 4, 2, 4><<<(unsigned)tiles, 512, 0, s>>>(h, w, c, M, vocab,
                                                                              hidden, nw);
        else if (TM == 128)
            lm_head_stream<256, 128, 2, 2, 3><<<(unsigned)tiles, 256, 0, s>>>(h, w, c, M, vocab,
                                                                              hidden, nw);
        else
            lm_head_stream<256, 64, 4, 1, 4><<<(unsigned)tiles, 256, 0, s>>>(h, w, c, M, vocab,
                                                                             hidden, nw);
        return check_launch(TM == 256 ? "lm_head_ring" : "lm_head_stream");
    }
    const long tiles = (long)((M + kBM - 1) / kBM) * ((vocab + kBN - 1) / kBN);
    if (tiles > 0x7fffffffL) return fail(SD_EUNSUPPORTED, "sd_lm_head: too many tiles");
    lm_head_bf16<<<(unsigned)tiles, 256, 0, s>>>((const uint16_t*)H, (const uint16_t*)W,
                                                  (uint16_t*)logits, M, vocab, hidden);
    return check_launch("lm_head_bf16");
}
