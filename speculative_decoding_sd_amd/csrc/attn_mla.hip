// MLA-shaped verify attention on gfx950 (one latent vector per position shared
// by every query head; keys are the whole 576-wide latent row, values its first
// 512 entries).  [TRT-MTP] "支持 MTP 的注意力機制": K+1 queries per request
// under a causal mask (the article's Hopper kernel for this case is FP8
// FlashMLA); [CSDN-MTP] "整体计算流程" step 2: softmax(QK^T/sqrt(d))V.
//
// With 128 query heads and K+1 = 4 positions a request has 512 query rows
// that all read the same latent rows, so this path is bound by the MFMA pipe,
// not by HBM (about 970 flop per latent byte).  Layout of the work:
//   workgroup = 128 query rows of one request x one chunk of keys, 4 waves;
//   wave      = 32 rows (one position i, 32 heads) and all 512 output dims,
//               O^T in 16 MFMA 32x32 accumulators, Q^T of its rows resident
//               (registers and LDS) for the whole chunk.
// Per 32-key tile:
//   S^T = K Q^T   A = latent rows read from LDS with ds_read_b128, B = Q^T;
//   online softmax lane-local (one query row per lane column).  The running
//                 max is only raised when a tile's max exceeds it by more than
//                 2^8, so the O rescale (256 accumulators) is rare; values of
//                 P up to 2^8 are exact enough in the bf16 hi+lo split below;
//   O^T += V^T P^T  A = V^T fragments read with ds_read_b64_tr_b16 (gfx950
//                 transposing LDS read: in a group of 16 lanes, lane t receives
//                 element t%4 of the 8-byte reads of lanes 4e + t/4, so lane s
//                 reading 4 dims of key row key0 + s/4 gives lane t the 4-key
//                 column of dim d0 + t); P split into bf16 hi + lo halves (two
//                 MFMAs per fragment) to hold the fp32 output accuracy.
// Latent tiles arrive by LDS DMA (global_load_lds_dwordx4) into a three-stage
// ring, so no registers stage them.  Register budget (one wave per SIMD, 512
// registers): O^T blocks 0..14 (240) and S^T (16) in AGPRs, the last O^T block
// kept in LDS between tiles so that S^T can use its registers; all of Q^T
// (144) in VGPRs; the rest is fragment prefetch, P and addressing.  LDS:
// 108 KiB latent + 16 KiB O^T.  The 16-byte chunks of each 1152-byte latent row
// are XOR-swizzled so that both LDS read patterns are free of bank conflicts.
// With one chunk per request the kernel writes the normalised output itself;
// otherwise it writes chunk partials for attn_combine.
#include <math.h>

#include "sdv_device.h"
#include "sdv_internal.h"
#include "sdv_lds.h"

namespace sdv {

namespace {

constexpr int kPage = 64;
constexpr int kDqk = 576, kDv = 512;
constexpr int kTileKeys = 32;
constexpr int kRowChunks = kDqk / 8;                       // 72 chunks of 16 bytes
constexpr int kRowBytes = kDqk * 2;                        // 1152
constexpr int kTileElems = kTileKeys * kDqk;               // 18432 bf16 = 36 KiB
constexpr int kStages = 3;
constexpr int kDmaPerWave = kTileKeys * kRowChunks / 256;  // 9 x 1 KiB per wave
constexpr float kRefSlack = 64.f;  // log2 units a later tile may exceed the reference max by
constexpr int kRowsPerBlock = 128;

// XOR applied to the 16-byte chunk index of latent row `row` of a tile
// (values 0..7, so each aligned group of 8 chunks maps onto itself).  The
// 1152-byte row stride puts odd rows 32 banks (8 chunks) over from even
// ones, so a ds_read_b128 pass (16 rows, one logical chunk) is free of bank
// conflicts when the 8 rows of each parity get 8 distinct values: the XOR is
// a bijection of row bits 1..3.  A ds_read_b64_tr_b16 pass (lanes 0..31:
// rows r, r+1, r+2, r+3 of one parity pair, four chunks of each) needs rows
// r and r+2 to differ in bit 2 of the XOR, which bit 1 of the row gives.
__device__ __forceinline__ int mla_swz(int row) { return 4 * ((row >> 1) & 1) + ((row >> 2) & 3); }
constexpr int kQSteps = kDqk / 16;     // 36 MFMA k-steps over the latent
static_assert(2 * (kDmaPerWave - 1) < 32, "a tile's DMAs are issued within the PV steps");

__global__ __launch_bounds__(256, 1) void attn_mla_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ lat,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ valid, float* __restrict__ out, uint16_t* __restrict__ out_lowp,
    float* __restrict__ part_o, float2* __restrict__ part_ml, int32_t* __restrict__ flags, int NQ,
    int Hq, int R, int max_pages, int chunk, int max_splits, int rblks, int total,
    float scale_log2) {
    __shared__ __attribute__((aligned(1024))) uint16_t s_lat[kStages][kTileElems];
    __shared__ __attribute__((aligned(16))) float s_o15[4][16 * 64];
    const int tile_id = xcd_tile(blockIdx.x, total);
    const int rblk = tile_id % rblks;
    const int split = (tile_id / rblks) % max_splits;
    const int b = tile_id / rblks / max_splits;
    if (!valid[b]) return;
    const int L = seq_lens[b];
    const int Ltot = L + NQ;
    const int start = split * chunk;
    if (start >= Ltot) return;
    const int end = min(start + chunk, Ltot);
    const int ntiles = (end - start + kTileKeys - 1) / kTileKeys;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 31, lh = lane >> 5;
    const int row0 = rblk * kRowsPerBlock + wave * 32;  // the wave's 32 rows share position i
    const bool rows_live = row0 < R;
    const int pos_i = rows_live ? row0 / Hq : 0;
    const int lim = L + pos_i;  // causal: keys 0 .. L_b + i

    // Q^T fragments (B operand): lane (row ln, half lh), step s -> dims
    // 16s+8lh..+8, all 36 steps held in registers for the whole chunk.
    u32x4 qf[kQSteps];
    {
        const int row = row0 + ln;
        const int i = rows_live ? row / Hq : 0, h = rows_live ? row - i * Hq : 0;
        const uint16_t* qp = q + (((size_t)b * NQ + i) * Hq + h) * kDqk + 8 * lh;
#pragma unroll
        for (int s = 0; s < kQSteps; ++s)
            qf[s] = rows_live ? *(const u32x4*)(qp + 16 * s) : u32x4{0, 0, 0, 0};
    }

    // DMA slots of this lane: instruction j of wave w fills LDS chunks
    // n = 64 (4j + w) + lane of the tile; chunk n holds latent row n / 72,
    // logical chunk (n % 72) ^ mla_swz(row).
    auto goff = [&](int j) {
        const int n = 64 * (4 * j + wave) + lane;
        const int key = n / kRowChunks;
        return key * kDqk + 8 * ((n - key * kRowChunks) ^ mla_swz(key));
    };
    const uint32_t lds0 = lds_byte_addr(&s_lat[0][0]);
    auto tile_src = [&](int t) {
        const int ks = start + kTileKeys * t;
        const int pg = page_table[(size_t)b * max_pages + ks / kPage];
        return lat + ((size_t)pg * kPage + (ks % kPage)) * kDqk;
    };
    auto tile_dst = [&](int t) { return lds0 + (uint32_t)((t % kStages) * kTileElems * 2); };
    auto tile_dma = [&](const uint16_t* base, uint32_t dst, int j) {
        dma16(base + goff(j), __builtin_amdgcn_readfirstlane(dst + (uint32_t)(1024 * (4 * j + wave))));
    };

    // Per-lane LDS byte offsets within a tile.
    //  S^T reads: key ln, logical chunk 2s + lh -> slot 8(s/4) + (2(s%4) ^ kx).
    const int kx = lh ^ mla_swz(ln);
    int koff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) koff[r] = ln * kRowBytes + 16 * ((2 * r) ^ kx);
    //  V^T reads (16-lane group g, lane sl): key 16tt + 4(g/2) + sl/4 (+8),
    //  logical chunk 4db + 2(g&1) + (sl&3)/2, byte 8(sl&1) of the chunk.
    //  The two key rows of a fragment (kr and kr + 8) have different XORs.
    const int g = lane >> 4, sl = lane & 15;
    const int kr = 4 * (g >> 1) + (sl >> 2);
    const int vll = 2 * (g & 1) + ((sl & 3) >> 1);
    const int vx0 = vll ^ mla_swz(kr), vx1 = vll ^ mla_swz(kr + 8);
    const int vrow = kr * kRowBytes + 8 * (sl & 1);
    const int voff_e0 = vrow + 16 * vx0, voff_o0 = vrow + 16 * (4 ^ vx0);
    const int voff_e1 = vrow + 8 * kRowBytes + 16 * vx1, voff_o1 = vrow + 8 * kRowBytes + 16 * (4 ^ vx1);

    // O^T blocks 0..14 live in registers; block 15 lives in this wave's LDS
    // slot between tiles (layout [q][lane][4] floats: conflict-free 16-byte
    // accesses), so that S^T can use its registers while it is computed.
    float* o15_lds = s_o15[wave];
    float m_r = -INFINITY, l_r = 0.f;
    bool over = false;
    f32x16 o[kDv / 32 - 1];
#pragma unroll
    for (int db = 0; db < kDv / 32 - 1; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) *(f32x4*)(o15_lds + (qd * 64 + lane) * 4) = f32x4{0.f, 0.f, 0.f, 0.f};

    // Three stages: tiles t+1 and t+2 load while tile t is computed.  At the
    // top of iteration t, tile t (issued two iterations earlier) has landed
    // once at most the nine DMAs of tile t+1 are in flight, and every wave
    // has left iteration t-1, so stage (t+2)%3 is free to refill.  The
    // refill's nine DMAs per wave go out during PV, one every two V^T
    // blocks: a DMA instruction holds up the wave's issue for tens of cycles,
    // which the two MFMAs queued per PV block cover and a single S^T MFMA
    // does not (section timing: S^T 2330 -> 1700 cycles per tile, PV
    // 2280 -> 2960, whole tile -4%).
    {
        const uint16_t* base0 = tile_src(0);
        const uint32_t dst0 = tile_dst(0);
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j) tile_dma(base0, dst0, j);
        if (ntiles > 1) {
            const uint16_t* base1 = tile_src(1);
            const uint32_t dst1 = tile_dst(1);
#pragma unroll
            for (int j = 0; j < kDmaPerWave; ++j) tile_dma(base1, dst1, j);
        }
    }
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) wait_vmcnt<kDmaPerWave>();
        else wait_vmcnt<0>();
        // This wave's reads of tile t-1 must have returned before another
        // wave refills that stage after the barrier.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        barrier_only();
        const bool more = t + 2 < ntiles;
        const uint16_t* nbase = more ? tile_src(t + 2) : lat;
        const uint32_t ndst = tile_dst(t + 2);
        const char* tile = (const char*)&s_lat[t % kStages][0];
        const int ks = start + kTileKeys * t;
        if (t == ntiles - 1 && end - ks < kTileKeys) {
            // Rows past the chunk end may hold anything (NaN included): zero
            // their value dims so that P = 0 contributes exactly nothing.
            const int nv = end - ks;
            for (int idx = tid; idx < (kTileKeys - nv) * 64; idx += 256) {
                const int key = nv + (idx >> 6), c = idx & 63;
                *(u32x4*)(tile + key * kRowBytes + 16 * (c ^ mla_swz(key))) = u32x4{0, 0, 0, 0};
            }
            __syncthreads();
        }

        // S^T = K Q^T over 576 dims, K fragments read ahead.
        f32x16 sa;
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[r] = 0.f;
        constexpr int PF = 8;  // read-ahead distance in k-steps
        u32x4 kf[PF];
#pragma unroll
        for (int s = 0; s < PF; ++s) kf[s] = *(const u32x4*)(tile + koff[s & 3] + 128 * (s >> 2));
#pragma unroll
        for (int s = 0; s < kQSteps; ++s) {
            const u32x4 cur = kf[s % PF];
            if (s + PF < kQSteps)
                kf[s % PF] = *(const u32x4*)(tile + koff[(s + PF) & 3] + 128 * ((s + PF) >> 2));
            sa = mfma_32x32x16(cur, qf[s], sa);
            // Bounds how far the scheduler hoists reads.
            __builtin_amdgcn_sched_barrier(0);
        }
        // Online softmax (lane holds 16 keys of query row ln).  The wave's
        // rows share one position, so whether the tile needs the mask (keys
        // past the chunk end or past the causal limit) is wave-uniform.
        float tmax = -INFINITY;
        if (ks + kTileKeys <= end && ks + kTileKeys - 1 <= lim) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sa[r] *= scale_log2;
                tmax = fmaxf(tmax, sa[r]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = ks + mfma_row(r, lane);
                const float v = sa[r] * scale_log2;
                sa[r] = (key >= end || key > lim) ? -INFINITY : v;
                tmax = fmaxf(tmax, sa[r]);
            }
        }
        tmax = halves_max(tmax);
        // The chunk's first tile sets each row's reference max; later tiles
        // are exponentiated against it (P up to 2^64 is exact enough in the
        // hi/lo split and safe in fp32).  A row whose later scores exceed the
        // reference by more than that is left to the exact path (flag).
        if (t == 0) m_r = tmax;
        else over |= tmax > m_r + kRefSlack;
        const float msafe = (m_r == -INFINITY) ? 0.f : m_r;
        float psum = 0.f;
        uint32_t pk[8], pl[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(sa[r] - msafe);
            const float p1 = __builtin_amdgcn_exp2f(sa[r + 1] - msafe);
            const uint32_t hi = cvt_pk_bf16(p0, p1);
            psum += p0 + p1;
            pk[r >> 1] = hi;
            pl[r >> 1] = cvt_pk_bf16(p0 - __uint_as_float(hi << 16),
                                     p1 - __uint_as_float(hi & 0xffff0000u));
        }
        psum = halves_sum(psum);
        l_r += psum;
        // Block 15 back from LDS (S^T is dead now; the barrier keeps the load
        // from being hoisted into S^T's live range).
        __builtin_amdgcn_sched_barrier(0);
        f32x16 o15;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const f32x4 v = *(const f32x4*)(o15_lds + (qd * 64 + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) o15[4 * qd + e] = v[e];
        }
        const u32x4 pb[2] = {u32x4{pk[0], pk[1], pk[2], pk[3]}, u32x4{pk[4], pk[5], pk[6], pk[7]}};
        const u32x4 pbl[2] = {u32x4{pl[0], pl[1], pl[2], pl[3]},
                              u32x4{pl[4], pl[5], pl[6], pl[7]}};
        // O^T += V^T P^T.  Slot 8h + 4a + r of step tt is key 16tt + 8a + 4h + r.
        // V^T fragments are read ahead.
        auto vfrag = [&](int idx) {  // idx = tt * 16 + db
            const int tt = idx >> 4, db = idx & 15;
            const char* vp = tile + 16 * tt * kRowBytes + 128 * (db >> 1);
            const u32x2 v0 = lds_read_tr16(vp + ((db & 1) ? voff_o0 : voff_e0));
            const u32x2 v1 = lds_read_tr16(vp + ((db & 1) ? voff_o1 : voff_e1));
            return u32x4{v0.x, v0.y, v1.x, v1.y};
        };
        constexpr int PV = 3;  // V^T fragments read this many blocks ahead
        u32x4 vf[PV];
#pragma unroll
        for (int idx = 0; idx < PV; ++idx) vf[idx] = vfrag(idx);
#pragma unroll
        for (int idx = 0; idx < 32; ++idx) {
            const u32x4 cur = vf[idx % PV];
            if (idx + PV < 32) vf[idx % PV] = vfrag(idx + PV);
            const int tt = idx >> 4, db = idx & 15;
            if (db < 15) {
                o[db] = mfma_32x32x16(cur, pb[tt], o[db]);
                o[db] = mfma_32x32x16(cur, pbl[tt], o[db]);
            } else {
                o15 = mfma_32x32x16(cur, pb[tt], o15);
                o15 = mfma_32x32x16(cur, pbl[tt], o15);
            }
            if ((idx & 1) == 0 && idx / 2 < kDmaPerWave && more) tile_dma(nbase, ndst, idx / 2);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
            *(f32x4*)(o15_lds + (qd * 64 + lane) * 4) =
                f32x4{o15[4 * qd], o15[4 * qd + 1], o15[4 * qd + 2], o15[4 * qd + 3]};
    }
    // Flag of this wave's rows for this chunk: 1 sends them to the exact path.
    const bool wave_over = __any(over);
    if (lane == 0) flags[(((size_t)b * max_splits + split) * rblks + rblk) * 4 + wave] = wave_over ? 1 : 0;
    if (!rows_live) return;
    f32x16 o15;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
        const f32x4 v = *(const f32x4*)(o15_lds + (qd * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) o15[4 * qd + e] = v[e];
    }
    auto oblk = [&](int db, int r) -> float { return db < 15 ? o[db < 15 ? db : 0][r] : o15[r]; };

    const int nsplit = (Ltot + chunk - 1) / chunk;
    const int row = row0 + ln;
    if (nsplit == 1) {
        // Lane (ln, lh) holds O^T[d = db*32 + 8j + 4lh + (0..3)][row ln].
        const float inv = 1.f / l_r;
        float* op = out + ((size_t)b * R + row) * kDv + 4 * lh;
        uint16_t* lp = out_lowp ? out_lowp + ((size_t)b * R + row) * kDv + 4 * lh : nullptr;
#pragma unroll
        for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = {oblk(db, 4 * j) * inv, oblk(db, 4 * j + 1) * inv,
                                 oblk(db, 4 * j + 2) * inv, oblk(db, 4 * j + 3) * inv};
                *(f32x4*)(op + db * 32 + 8 * j) = v;
                if (lp)
                    *(u32x2*)(lp + db * 32 + 8 * j) =
                        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
        return;
    }
    const size_t pidx = (size_t)b * max_splits + split;
    float* po = part_o + pidx * kDv * R;
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) po[(size_t)(db * 32 + mfma_row(r, lane)) * R + row] = oblk(db, r);
    if (lh == 0) part_ml[pidx * R + row] = make_float2(m_r, l_r);
}

// Exact path for the rows the fast kernel flagged (a later key scoring more
// than 2^64 above the chunk's first-tile max): plain fp32 arithmetic, scores
// by dot products, a max pass, then o = sum p v / sum p.  One workgroup per
// (request, chunk, row block, wave) unit; units without a flag exit at once.
// Writes the same output (single chunk) or partial (m, l, O) as the fast path.
__global__ __launch_bounds__(256) void attn_mla_exact(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ lat,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ valid, const int32_t* __restrict__ flags, float* __restrict__ out,
    uint16_t* __restrict__ out_lowp, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int NQ, int Hq, int R, int max_pages, int chunk, int max_splits, int rblks, float scale) {
    __shared__ float s_q[kDqk];
    __shared__ float s_red[256];
    __shared__ float s_p[256];
    const int unit = blockIdx.x;
    const int wave = unit % 4, rblk = (unit / 4) % rblks;
    const int split = (unit / 4 / rblks) % max_splits, b = unit / 4 / rblks / max_splits;
    if (!valid[b] || !flags[unit]) return;
    const int L = seq_lens[b], Ltot = L + NQ;
    const int start = split * chunk;
    if (start >= Ltot) return;
    const int end = min(start + chunk, Ltot);
    const int nsplit = (Ltot + chunk - 1) / chunk;
    const int tid = threadIdx.x;
    auto latent = [&](int key) {
        const int pg = page_table[(size_t)b * max_pages + key / kPage];
        return lat + ((size_t)pg * kPage + key % kPage) * kDqk;
    };
    for (int rr = 0; rr < 32; ++rr) {
        const int row = rblk * kRowsPerBlock + wave * 32 + rr;
        if (row >= R) break;
        const int i = row / Hq, h = row - i * Hq;
        const int lim = min(end - 1, L + i);
        const uint16_t* qp = q + (((size_t)b * NQ + i) * Hq + h) * kDqk;
        for (int d = tid; d < kDqk; d += 256) s_q[d] = bf16_to_f32(qp[d]);
        __syncthreads();
        // Pass 1: row max over the chunk's visible keys.
        float m = -INFINITY;
        for (int key = start + tid; key <= lim; key += 256) {
            const uint16_t* kp = latent(key);
            float dot = 0.f;
            for (int d = 0; d < kDqk; ++d) dot += s_q[d] * bf16_to_f32(kp[d]);
            m = fmaxf(m, dot * scale);
        }
        s_red[tid] = m;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
            __syncthreads();
        }
        m = s_red[0];
        __syncthreads();
        // Pass 2: p = exp(s - m); thread d accumulates output dims d, d+256.
        float acc0 = 0.f, acc1 = 0.f, lsum = 0.f;
        for (int k0 = start; k0 <= lim; k0 += 256) {
            const int key = k0 + tid;
            float p = 0.f;
            if (key <= lim) {
                const uint16_t* kp = latent(key);
                float dot = 0.f;
                for (int d = 0; d < kDqk; ++d) dot += s_q[d] * bf16_to_f32(kp[d]);
                p = expf(dot * scale - m);
            }
            s_p[tid] = p;
            __syncthreads();
            const int cnt = min(256, lim - k0 + 1);
            for (int k = 0; k < cnt; ++k) {
                const uint16_t* vp = latent(k0 + k);
                acc0 += s_p[k] * bf16_to_f32(vp[tid]);
                acc1 += s_p[k] * bf16_to_f32(vp[tid + 256]);
                lsum += s_p[k];
            }
            __syncthreads();
        }
        if (nsplit == 1) {
            const float inv = 1.f / lsum;
            float* op = out + ((size_t)b * R + row) * kDv;
            op[tid] = acc0 * inv;
            op[tid + 256] = acc1 * inv;
            if (out_lowp) {
                uint16_t* lp = out_lowp + ((size_t)b * R + row) * kDv;
                lp[tid] = (uint16_t)f32_to_bf16_rne(acc0 * inv);
                lp[tid + 256] = (uint16_t)f32_to_bf16_rne(acc1 * inv);
            }
        } else {
            // Partial in the fast path's units: m in log2 units, O and l
            // relative to 2^m.
            const size_t pidx = (size_t)b * max_splits + split;
            float* po = part_o + pidx * kDv * R;
            po[(size_t)tid * R + row] = acc0;
            po[(size_t)(tid + 256) * R + row] = acc1;
            if (tid == 0) part_ml[pidx * R + row] = make_float2(m * 1.4426950408889634f, lsum);
        }
        __syncthreads();
    }
}

}  // namespace

// Launch planning and dispatch for the MLA path (called by sd_verify_attn).
// One workgroup per (request, 128-row block, key chunk) and one workgroup per
// CU (the kernel holds 512 registers per lane and 108 KiB of LDS): split the
// keys into chunks (multiples of the 32-key tile, at least 1024 keys) only
// while the grid has fewer than 256 workgroups.
int mla_plan(int batch, int num_q, int n_q_heads, int max_seq_len, int* chunk, int* max_splits) {
    if (n_q_heads % 32 != 0)
        return fail(SD_EUNSUPPORTED, "sd_verify_attn: MLA needs n_q_heads %% 32 == 0");
    const long maxkeys = (long)max_seq_len + num_q;
    const int R = num_q * n_q_heads;
    const long groups = (long)batch * ((R + kRowsPerBlock - 1) / kRowsPerBlock);
    long c = (maxkeys + kTileKeys - 1) / kTileKeys * kTileKeys;
    while (c > 1024 && groups * ((maxkeys + c - 1) / c) < 256)
        c = (c / 2 + kTileKeys - 1) / kTileKeys * kTileKeys;
    *chunk = (int)c;
    *max_splits = (int)((maxkeys + c - 1) / c);
    return SD_OK;
}

int mla_launch(const sd_attn_desc* d, const int32_t* valid, int32_t* flags, float* po,
               float2* pml, int chunk, int max_splits, float scale, hipStream_t s) {
    const int R = d->num_q * d->n_q_heads;
    const int rblks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
    const long total = (long)d->batch * max_splits * rblks;
    if (total * 4 > 0x7fffffffL) return fail(SD_EUNSUPPORTED, "sd_verify_attn: MLA grid too large");
    attn_mla_bf16<<<dim3((unsigned)total), 256, 0, s>>>(
        (const uint16_t*)d->q, (const uint16_t*)d->k_cache, d->page_table, d->seq_lens, valid,
        d->out, (uint16_t*)d->out_lowp, po, pml, flags, d->num_q, d->n_q_heads, R, d->max_pages,
        chunk, max_splits, rblks, (int)total, scale * 1.4426950408889634f);
    int rc = check_launch("attn_mla_bf16");
    if (rc != SD_OK) return rc;
    attn_mla_exact<<<dim3((unsigned)(total * 4)), 256, 0, s>>>(
        (const uint16_t*)d->q, (const uint16_t*)d->k_cache, d->page_table, d->seq_lens, valid,
        flags, d->out, (uint16_t*)d->out_lowp, po, pml, d->num_q, d->n_q_heads, R, d->max_pages,
        chunk, max_splits, rblks, scale);
    return check_launch("attn_mla_exact");
}

// Workspace ints for the per-unit flags.
size_t mla_flag_count(int batch, int num_q, int n_q_heads, int max_splits) {
    const int R = num_q * n_q_heads;
    return (size_t)batch * max_splits * ((R + kRowsPerBlock - 1) / kRowsPerBlock) * 4;
}

}  // namespace sdv
