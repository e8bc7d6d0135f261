// GQA verify attention on gfx950, bf16 cache, fp32 accumulation.
// [TRT-MTP] "支持 MTP 的注意力機制": the K+1 query positions of a request are
// verified together against its cache under a causal mask; [CSDN-MTP]
// "整体计算流程" step 2: softmax(QK^T/sqrt(d))V over the cached and new keys.
//
// The query rows of one (request, kv head) are the G heads of the group at
// each of the K+1 positions (row = i*G + g, at most 64), so every key/value
// row fetched from HBM serves all of them: the kernel is bound by streaming
// the cache.  Work items are (kv head, request, key chunk) triples; each wave
// runs its own items start to finish (no workgroup barriers) and streams their
// 32-key tiles through private LDS rings filled by LDS DMA (three K stages,
// two V stages: 40 KiB per wave at head dim 128), so that about two tiles per
// wave are in flight while one is computed, also across item boundaries.  The grid holds one workgroup of 4 waves per CU; each wave
// takes an equal contiguous range of the non-empty items.
// Per tile and 32-row block:
//   S^T = K Q^T    A = K rows from LDS (ds_read_b128), B = Q^T in registers;
//   online softmax lane-local (one query row per lane column); the running
//                  max is raised only when a tile exceeds it by more than 2^8;
//   O^T += V^T P^T A = V^T fragments by ds_read_b64_tr_b16 from the row-major
//                  V tile, P in bf16 hi + lo halves (two MFMAs).
// Each item writes its unnormalised O^T and (m, l) per row; attn_combine
// merges the chunks of a request.
#include <math.h>

#include "sdv_device.h"
#include "sdv_internal.h"
#include "sdv_lds.h"

namespace sdv {
namespace {

constexpr int kPage = 64;
constexpr int kTile = 32;
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int D>
struct GqaTile {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kRowChunks = D / 8;
    static constexpr int kHalfBytes = kTile * kRowBytes;  // the K (or V) rows of a tile
    static constexpr int kDmaHalf = kHalfBytes / 1024;    // 1 KiB DMA ops per half tile
    static constexpr int kKStages = 3, kVStages = 2;      // K runs one tile further ahead
    static constexpr int kRingBytes = (kKStages + kVStages) * kHalfBytes;
};

// XOR applied to the 16-byte chunk index of K/V tile row `row`.  The LDS has
// 64 banks of 4 bytes: a ds_read_b128 is served 16 lanes per pass and a
// ds_read_b64_tr_b16 32 lanes per pass, each pass covering 256 bytes.
//  K reads: the 16 lanes of a pass read one logical chunk of 16 consecutive
//    rows, so the 16 rows must land in 16 distinct 16-byte bank groups;
//  V reads: a 32-lane pass reads 4 logical chunks 4c..4c+3 of 4 consecutive
//    rows (4-aligned), two lanes per chunk.
// D = 128 (256-byte rows, every row starts at bank 0): f(row) takes bits 3:2
// from row%4 and bits 1:0 from (row/4)%4, a bijection on each 16-row group
// whose bits 3:2 differ between the 4 rows of a V pass.  D = 64 (128-byte
// rows, row parity picks the bank half): f(row) = 4((row/2)%2) + (row/4)%4, a
// bijection on the 8 rows of one parity in a 16-row group, whose bit 2
// differs between rows r and r+2.
template <int D>
__device__ __forceinline__ int gqa_xor(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Work items are (kv head, request, key chunk) triples of non-empty chunks,
// numbered kv-head-major: item i has kv head i / NRC and request-chunk index
// rc = i % NRC, where request b owns rc in [first[b], first[b+1]) and
// NRC = first[B].  first[] is the exclusive prefix sum of the requests' chunk
// counts (0 for invalid requests), written by attn_items.  Wave w of nw runs
// the contiguous item range [w N / nw, (w+1) N / nw), N = NRC * Hkv, which
// balances the waves to one item; kv-head-major numbering puts concurrent
// waves on different heads, spreading their reads over the cache pages'
// address ranges.  All cursor fields are wave-uniform.
struct ItemCursor {
    int item, hi, t, ntiles, b, kvh, split, rc, L, start, end;
    int pg;  // physical page of the current tile (DMA cursors only)
};

__device__ __forceinline__ void cursor_fill(ItemCursor& c, int NQ, int chunk,
                                            const int32_t* __restrict__ seq_lens) {
    c.L = seq_lens[c.b];
    c.start = c.split * chunk;
    c.end = min(c.start + chunk, c.L + NQ);
    c.ntiles = (c.end - c.start + kTile - 1) / kTile;
    c.t = 0;
}

__device__ __forceinline__ void cursor_begin(ItemCursor& c, int lo, int hi, int B, int NRC,
                                             int NQ, int chunk, const int32_t* __restrict__ first,
                                             const int32_t* __restrict__ seq_lens) {
    c.item = lo;
    c.hi = hi;
    if (lo >= hi) return;
    c.kvh = lo / NRC;
    c.rc = lo - c.kvh * NRC;
    int b0 = 0, b1 = B;  // largest b with first[b] <= rc (first[B] > rc)
    while (b1 - b0 > 1) {
        const int mid = (b0 + b1) >> 1;
        if (first[mid] <= c.rc) b0 = mid; else b1 = mid;
    }
    c.b = b0;
    c.split = c.rc - first[b0];
    cursor_fill(c, NQ, chunk, seq_lens);
}

__device__ __forceinline__ void cursor_next(ItemCursor& c, int NRC, int NQ, int chunk,
                                            const int32_t* __restrict__ first,
                                            const int32_t* __restrict__ seq_lens) {
    if (++c.t < c.ntiles) return;
    if (++c.item >= c.hi) return;
    if (++c.rc == NRC) {
        c.rc = 0;
        ++c.kvh;
        c.b = 0;
        c.split = -1;
    }
    ++c.split;
    while (c.split >= first[c.b + 1] - first[c.b]) {  // next request with chunks
        ++c.b;
        c.split = 0;
    }
    cursor_fill(c, NQ, chunk, seq_lens);
}

template <int D, int RB>
__global__ __launch_bounds__(256, 1) void attn_gqa_stream(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ first,
    float* __restrict__ part_o, float2* __restrict__ part_ml, float* __restrict__ out,
    uint16_t* __restrict__ out_lowp, int B, int NQ, int Hq, int Hkv, int G, int R, int max_pages,
    int chunk, int max_splits, float scale_log2) {
    using T = GqaTile<D>;
    constexpr int NS = D / 16;   // MFMA k-steps over the head dimension
    constexpr int NDB = D / 32;  // 32-dim blocks of O^T
    __shared__ __attribute__((aligned(1024))) char s_ring[4][T::kRingBytes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ln = lane & 31, lh = lane >> 5;
    const int nw = gridDim.x * 4;
    char* ring = s_ring[wave];

    // DMA op j of a half tile fills LDS bytes [1024 j, 1024 j + 1024): chunk
    // slot n = 64 j + lane, holding logical chunk (n % kRowChunks) ^
    // gqa_xor(row) of row n / kRowChunks.
    int goff[T::kDmaHalf];
#pragma unroll
    for (int j = 0; j < T::kDmaHalf; ++j) {
        const int n = 64 * j + lane;
        const int row = n / T::kRowChunks;
        goff[j] = row * D + 8 * ((n % T::kRowChunks) ^ gqa_xor<D>(row));
    }
    const size_t head_elems = (size_t)kPage * D;
    char* const k_ring = ring;
    char* const v_ring = ring + T::kKStages * T::kHalfBytes;
    // The page-table entry of a DMA cursor's tile is read when the cursor
    // reaches the tile, one issue before it is needed, so the scalar load's
    // latency is not on the DMA's critical path.
    auto load_pg = [&](ItemCursor& c) {
        if (c.item < c.hi)
            c.pg = page_table[(size_t)c.b * max_pages + (c.start + kTile * c.t) / kPage];
    };
    auto issue = [&](const uint16_t* __restrict__ cache, const ItemCursor& c, const char* dst_p) {
        const int ks = c.start + kTile * c.t;
        const uint16_t* src =
            cache + ((size_t)c.pg * Hkv + c.kvh) * head_elems + (size_t)(ks % kPage) * D;
        const uint32_t dst = lds_byte_addr(dst_p);
        // The stage's previous tile was read by this wave's ds_reads; make
        // sure they have returned before the DMA may overwrite it.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < T::kDmaHalf; ++j)
            dma16(src + goff[j], __builtin_amdgcn_readfirstlane(dst + 1024u * j));
    };

    // Per-lane LDS byte offsets within a half tile.
    //  K reads of k-step s: row ln, logical chunk 2s + lh.
    int koff[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = ln * T::kRowBytes + 16 * ((2 * s + lh) ^ gqa_xor<D>(ln));
    //  V reads (16-lane group g, lane sl) of dim block db, half h: key
    //  16tt + 4(g/2) + sl/4 + 8h, logical chunk 4db + 2(g&1) + (sl&3)/2, byte
    //  8(sl&1) of the chunk (the swizzle depends on the key only modulo 16).
    const int g4 = lane >> 4, sl = lane & 15;
    const int vch = 2 * (g4 & 1) + ((sl & 3) >> 1);
    int voff[NDB][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int vr = 4 * (g4 >> 1) + (sl >> 2) + 8 * h;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            voff[db][h] = vr * T::kRowBytes + 16 * ((4 * db + vch) ^ gqa_xor<D>(vr)) + 8 * (sl & 1);
    }

    // Three cursors over the wave's tile stream: K DMA (three tiles ahead of
    // the compute), V DMA (two ahead) and compute.  Issue order: K0 K1 V0 K2
    // V1, then after computing tile c: K(c+3) V(c+2).  nk / nv count the
    // halves issued; vmcnt waits count the 1 KiB ops issued after the one
    // needed (DMAs complete in issue order).
    const int NRC = first[B];
    const long n_items = (long)NRC * Hkv;
    const int gw = blockIdx.x * 4 + wave;
    ItemCursor kc;
    cursor_begin(kc, (int)(n_items * gw / nw), (int)(n_items * (gw + 1) / nw), B, NRC, NQ, chunk,
                 first, seq_lens);
    load_pg(kc);
    ItemCursor vc = kc, cc = kc;
    int nk = 0, nv = 0;
    auto issue_k = [&]() {
        if (kc.item < kc.hi) {
            issue(k_cache, kc, k_ring + (nk % T::kKStages) * T::kHalfBytes);
            ++nk;
            cursor_next(kc, NRC, NQ, chunk, first, seq_lens);
            load_pg(kc);
        }
    };
    auto issue_v = [&]() {
        if (vc.item < vc.hi) {
            issue(v_cache, vc, v_ring + (nv % T::kVStages) * T::kHalfBytes);
            ++nv;
            cursor_next(vc, NRC, NQ, chunk, first, seq_lens);
            load_pg(vc);
        }
    };
    auto wait_groups = [&](int g) {  // at most g half tiles still in flight
        switch (g) {
            case 0: wait_vmcnt<0>(); break;
            case 1: wait_vmcnt<1 * T::kDmaHalf>(); break;
            case 2: wait_vmcnt<2 * T::kDmaHalf>(); break;
            case 3: wait_vmcnt<3 * T::kDmaHalf>(); break;
            case 4: wait_vmcnt<4 * T::kDmaHalf>(); break;
            default: wait_vmcnt<5 * T::kDmaHalf>(); break;
        }
    };
    issue_k();
    issue_k();
    issue_v();
    issue_k();
    issue_v();
    int cseq = 0;

    u32x4 qf[RB][NS];
    int lim[RB];
    float m_r[RB], l_r[RB];
    f32x16 o[RB][NDB];
    // Consecutive chunks of one (request, kv head) form a segment: the online
    // softmax state and Q carry over from chunk to chunk, and the segment is
    // written once, at its end.
    int seg_b = -1, seg_kvh = -1, seg_split0 = 0;
    while (cc.item < cc.hi) {
        // K(cseq) has landed once at most the halves issued after it are in
        // flight: K(j > cseq) and V(j >= max(cseq - 1, 0)).
        wait_groups((nk - 1 - cseq) + (nv - max(cseq - 1, 0)));
        if (cc.t == 0 && !(cc.b == seg_b && cc.kvh == seg_kvh)) {
            seg_b = cc.b;
            seg_kvh = cc.kvh;
            seg_split0 = cc.split;
            // New item: Q fragments (B operand; column = query row, k = d).
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = rb * 32 + ln;
                if (row < R) {
                    const int i = row / G, gq = row - i * G;
                    const uint16_t* qp =
                        q + (((size_t)cc.b * NQ + i) * Hq + cc.kvh * G + gq) * D + 8 * lh;
#pragma unroll
                    for (int s = 0; s < NS; ++s) qf[rb][s] = *(const u32x4*)(qp + 16 * s);
                    lim[rb] = cc.L + i;  // causal: keys 0 .. L_b + i
                } else {
#pragma unroll
                    for (int s = 0; s < NS; ++s) qf[rb][s] = u32x4{0, 0, 0, 0};
                    lim[rb] = cc.L + NQ - 1;
                }
                m_r[rb] = -INFINITY;
                l_r[rb] = 0.f;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[rb][db][r] = 0.f;
            }
        }
        const char* ktile = k_ring + (cseq % T::kKStages) * T::kHalfBytes;
        char* vtile = v_ring + (cseq % T::kVStages) * T::kHalfBytes;
        const int ks = cc.start + kTile * cc.t;
        // S^T = K Q^T.
        f32x16 sacc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const u32x4 kf = *(const u32x4*)(ktile + koff[s]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) sacc[rb] = mfma_32x32x16(kf, qf[rb][s], sacc[rb]);
        }

        // Online softmax; lane (ln, lh) holds 16 keys of query row ln.
        u32x4 pb[RB][2], pbl[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = ks + mfma_row(r, lane);
                const float v = sacc[rb][r] * scale_log2;
                sacc[rb][r] = (key >= cc.end || key > lim[rb]) ? -INFINITY : v;
                tmax = fmaxf(tmax, sacc[rb][r]);
            }
            tmax = fmaxf(tmax, shfl_xor(tmax, 32));
            const bool raise = tmax > m_r[rb] + kRescaleSlack;
            if (__any(raise)) {
                const float mnew = raise ? tmax : m_r[rb];
                const float alpha = raise ? __builtin_amdgcn_exp2f(m_r[rb] - mnew) : 1.f;
                l_r[rb] *= alpha;
                m_r[rb] = mnew;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[rb][db] *= alpha;
            }
            const float msafe = (m_r[rb] == -INFINITY) ? 0.f : m_r[rb];
            float psum = 0.f;
            uint32_t pk[8], pl[8];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(sacc[rb][r] - msafe);
                const float p1 = __builtin_amdgcn_exp2f(sacc[rb][r + 1] - msafe);
                const uint32_t hi = pack_bf16_finite(p0, p1);
                psum += p0 + p1;
                pk[r >> 1] = hi;
                pl[r >> 1] =
                    pack_bf16_finite(p0 - bf16_to_f32(hi & 0xffffu), p1 - bf16_to_f32(hi >> 16));
            }
            psum += shfl_xor(psum, 32);
            l_r[rb] += psum;
            pb[rb][0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
            pb[rb][1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
            pbl[rb][0] = u32x4{pl[0], pl[1], pl[2], pl[3]};
            pbl[rb][1] = u32x4{pl[4], pl[5], pl[6], pl[7]};
        }

        // V(cseq) has landed once at most V(j > cseq) and K(j >= cseq + 2) are
        // in flight.
        wait_groups((nv - 1 - cseq) + max(0, nk - (cseq + 2)));
        if (ks + kTile > cc.end) {
            // Rows past the chunk end may hold anything (NaN included): zero
            // their values so that P = 0 contributes exactly nothing.
            const int nv = cc.end - ks;
            for (int idx = lane; idx < (kTile - nv) * T::kRowChunks; idx += 64) {
                const int row = nv + idx / T::kRowChunks, c = idx % T::kRowChunks;
                *(u32x4*)(vtile + row * T::kRowBytes + 16 * (c ^ gqa_xor<D>(row))) =
                    u32x4{0, 0, 0, 0};
            }
        }

        // O^T += V^T P^T.  Slot 8h + 4a + r of step tt is key 16tt + 8a + 4h + r.
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const char* vp = vtile + 16 * tt * T::kRowBytes;
                const u32x2 v0 = lds_read_tr16(vp + voff[db][0]);
                const u32x2 v1 = lds_read_tr16(vp + voff[db][1]);
                const u32x4 vf = u32x4{v0.x, v0.y, v1.x, v1.y};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    o[rb][db] = mfma_32x32x16(vf, pb[rb][tt], o[rb][db]);
                    o[rb][db] = mfma_32x32x16(vf, pbl[rb][tt], o[rb][db]);
                }
            }
        }

        // This tile's stages are read: refill them three (K) and two (V)
        // tiles ahead in the wave's stream.
        issue_k();
        issue_v();
        const int ns_b = (cc.L + NQ + chunk - 1) / chunk;
        const bool last_of_pair = cc.split == ns_b - 1;
        if (cc.t == cc.ntiles - 1 && (last_of_pair || cc.item + 1 >= cc.hi)) {
            const size_t pbase = ((size_t)cc.b * Hkv + cc.kvh) * max_splits;
            if (seg_split0 == 0 && last_of_pair) {
                // The segment covers the whole pair: normalised rows straight
                // to the output.  Lane (ln, lh) holds dims 8(r/4) + 4lh + r%4.
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int row = rb * 32 + ln;
                    if (row >= R) continue;
                    const int i = row / G, gq = row - i * G;
                    const size_t oi = (((size_t)cc.b * NQ + i) * Hq + cc.kvh * G + gq) * D;
                    const float inv = 1.f / l_r[rb];
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int qd = 0; qd < 4; ++qd) {
                            const int d = db * 32 + 8 * qd + 4 * lh;
                            const f32x4 v = {o[rb][db][4 * qd] * inv, o[rb][db][4 * qd + 1] * inv,
                                             o[rb][db][4 * qd + 2] * inv,
                                             o[rb][db][4 * qd + 3] * inv};
                            *(f32x4*)(out + oi + d) = v;
                            if (out_lowp) {
                                u32x2 w;
                                w.x = pack_bf16x2(v[0], v[1]);
                                w.y = pack_bf16x2(v[2], v[3]);
                                *(u32x2*)(out_lowp + oi + d) = w;
                            }
                        }
                }
                if (lane == 0) part_ml[pbase * R] = make_float2(-INFINITY, kPartDirect);
            } else {
                const size_t pidx = pbase + seg_split0;
                float* po = part_o + pidx * D * R;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int row = rb * 32 + ln;
                    if (row >= R) continue;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            po[(size_t)(db * 32 + mfma_row(r, lane)) * R + row] = o[rb][db][r];
                    if (lh == 0) part_ml[pidx * R + row] = make_float2(m_r[rb], l_r[rb]);
                }
                for (int sp = seg_split0 + 1 + lane; sp <= cc.split; sp += 64)
                    part_ml[(pbase + sp) * R] = make_float2(-INFINITY, kPartEmpty);
            }
            seg_b = -1;  // the next item starts a new segment
        }
        cursor_next(cc, NRC, NQ, chunk, first, seq_lens);
        ++cseq;
    }
}

// first[b] = number of non-empty key chunks of the valid requests before b
// (exclusive prefix sum), first[B] = their total.  One block.
__global__ __launch_bounds__(1024) void attn_items(const int32_t* __restrict__ seq_lens,
                                                   const int32_t* __restrict__ valid,
                                                   int32_t* __restrict__ first, int B, int NQ,
                                                   int chunk) {
    __shared__ int32_t s_sum[1024];
    __shared__ int32_t s_carry;
    if (threadIdx.x == 0) s_carry = 0;
    for (int b0 = 0; b0 < B; b0 += 1024) {
        const int b = b0 + threadIdx.x;
        const int n = (b < B && valid[b]) ? (seq_lens[b] + NQ + chunk - 1) / chunk : 0;
        s_sum[threadIdx.x] = n;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
            const int v = threadIdx.x >= off ? s_sum[threadIdx.x - off] : 0;
            __syncthreads();
            s_sum[threadIdx.x] += v;
            __syncthreads();
        }
        if (b < B) first[b] = s_carry + s_sum[threadIdx.x] - n;
        __syncthreads();
        if (threadIdx.x == 1023) s_carry += s_sum[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) first[B] = s_carry;
}

int g_num_cus = 0;

}  // namespace

// Item plan, then the persistent kernel: one 4-wave workgroup per CU.
int gqa_launch(const sd_attn_desc* d, const int32_t* valid, int32_t* first, float* po,
               float2* pml, int R, int chunk, int max_splits, float scale_log2, hipStream_t s) {
    if (g_num_cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            return fail(SD_EDEVICE, "sd_verify_attn: cannot query the CU count");
        g_num_cus = n;
    }
    const long n_items = (long)max_splits * d->batch * d->n_kv_heads;
    if (n_items > 0x7fffffffL) return fail(SD_EUNSUPPORTED, "sd_verify_attn: too many chunks");
    attn_items<<<1, 1024, 0, s>>>(d->seq_lens, valid, first, d->batch, d->num_q, chunk);
    int rc = check_launch("attn_items");
    if (rc != SD_OK) return rc;
    const int G = d->n_q_heads / d->n_kv_heads;
#define SDV_LAUNCH_GQA(DD, RBB)                                                                  \
    attn_gqa_stream<DD, RBB><<<g_num_cus, 256, 0, s>>>(                                          \
        (const uint16_t*)d->q, (const uint16_t*)d->k_cache, (const uint16_t*)d->v_cache,         \
        d->page_table, d->seq_lens, first, po, pml, d->out, (uint16_t*)d->out_lowp, d->batch,   \
        d->num_q, d->n_q_heads, d->n_kv_heads, G, R, d->max_pages, chunk, max_splits, scale_log2)
    if (d->d_qk == 128) {
        if (R <= 32) SDV_LAUNCH_GQA(128, 1); else SDV_LAUNCH_GQA(128, 2);
    } else {
        if (R <= 32) SDV_LAUNCH_GQA(64, 1); else SDV_LAUNCH_GQA(64, 2);
    }
#undef SDV_LAUNCH_GQA
    return check_launch("attn_gqa_stream");
}

}  // namespace sdv
