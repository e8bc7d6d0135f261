// GQA verify attention on gfx950, bf16 q with a bf16 or E4M3 (FP8) cache, fp32
// accumulation.
// [TRT-MTP] "支持 MTP 的注意力機制": the K+1 query positions of a request are
// verified together against its cache under a causal mask; [CSDN-MTP]
// "整体计算流程" step 2: softmax(QK^T/sqrt(d))V over the cached and new keys.
//
// The query rows of one (request, kv head) are the G heads of the group at
// each of the K+1 positions (row = i*G + g, at most 64), so every key/value
// row fetched from HBM serves all of them: the kernel is bound by streaming
// the cache.  The work is the sequence of 32-key tiles of all (kv head,
// request) pairs; each persistent wave takes an equal contiguous range of it
// (no workgroup barriers) and streams its tiles through private LDS rings
// filled by LDS DMA (S K stages and S - 1 V stages, as many as the LDS holds
// up to S = 5: 40 KiB per wave for bf16 at head dim 128), so that S - 1
// tiles per wave are in flight while one is computed, also across pair
// boundaries.  One 4-wave workgroup per CU (two for E4M3 with one row block,
// and for attn_gqa_f8_r16: E4M3 with 33..48 rows in three 16-row blocks).
// Per tile and 32-row block (attn_gqa_stream):
//   S^T = K Q^T    A = K rows from LDS (ds_read_b128; E4M3 bytes converted to
//                  bf16 exactly), B = Q^T in registers;
//   online softmax lane-local (one query row per lane column); the running
//                  max is raised only when a tile exceeds it by more than 2^8;
//   O^T += V^T P^T A = V^T fragments by ds_read_b64_tr_b16 (bf16) or
//                  ds_read_b64_tr_b8 + conversion (E4M3) from the row-major V
//                  tile; bf16 cache: P in bf16 hi + lo halves (two MFMAs);
//                  E4M3 cache: V exact in fp16, P rounded to fp16 (one MFMA).
// The refill DMAs of a tile's stages go out between its V^T blocks.  A
// wave's tiles of one pair form a segment, written once at its end: to the
// output when it covers the whole pair, else as an unnormalised partial
// (O^T, m, l) that attn_combine merges.
#include <math.h>

#include <algorithm>

#include "sdv_device.h"
#include "sdv_internal.h"
#include "sdv_lds.h"

namespace sdv {
namespace {

constexpr int kPage = 64;
constexpr int kTile = 32;
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int D, bool F8, int KS>
struct GqaTile {
    static constexpr int kRowBytes = D * (F8 ? 1 : 2);
    static constexpr int kRowChunks = kRowBytes / 16;
    static constexpr int kHalfBytes = kTile * kRowBytes;  // the K (or V) rows of a tile
    static constexpr int kDmaHalf = kHalfBytes / 1024;    // 1 KiB DMA ops per half tile
    static constexpr int kKStages = KS, kVStages = KS - 1;  // K runs one tile further ahead
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
// E4M3 tiles (one byte per element; V read by ds_read_b64_tr_b8, a pass
// covering 8 rows x 2 chunks 2c, 2c+1: rows r0 + {0..3, 8..11}):
// D = 128 (128-byte rows, row parity picks the bank half): with
// x = (row/2)%8, f takes bit 2 from x's bit 2, bit 1 from x's bit 0 and bit 0
// from x's bit 1 -- a bijection on x (K passes), and the four rows of one
// parity in a V pass (x = x0 + {0, 1, 4, 5}) differ in bits 2:1 of f, which
// the chunk pair's bit 0 does not touch.  D = 64 (64-byte rows, row%4 picks
// the bank quarter): f = (row/4)%4, a bijection on the 4 rows of one class in
// a 16-row group, differing in bit 1 between rows r and r+8.
template <int D, bool F8>
__device__ __forceinline__ int gqa_xor(int row) {
    if constexpr (F8) {
        if constexpr (D == 128) {
            const int x = (row >> 1) & 7;
            return (x & 4) | ((x & 1) << 1) | ((x >> 1) & 1);
        } else {
            return (row >> 2) & 3;
        }
    } else if constexpr (D == 128) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    }
}

// Eight E4M3 codes (bytes 0..7 of w, lowest first) -> eight bf16 in operand
// order, exactly (every E4M3 value is a bf16 value; scale 1).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    return u32x4{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true))};
}

// With an E4M3 cache the value codes convert to fp16 exactly (E4M3 values lie
// in fp16's range with at most 4 significant bits), so O^T += V^T P^T runs as
// one fp16 MFMA per fragment with P rounded to fp16 (relative error at most
// 2^-11 per weight, fp32 accumulation) instead of the bf16 hi + lo pair of the
// bf16 cache.  P = exp2(s - m) <= 2^8 is scaled by 2^7 before the rounding, so
// that weights down to 2^-31 of the reference stay representable (fp16
// subnormals start at 2^-24); the value scale absorbs the 2^-7.
constexpr float kPScale = 128.f, kPScaleInv = 1.f / 128.f;

__device__ __forceinline__ u32x4 e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
    return u32x4{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, true))};
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// Two floats -> packed fp16 (lo in the low half), round to nearest even.
__device__ __forceinline__ uint32_t cvt_pk_f16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{lo, hi}, f16x2_t));
}

// The fp16 form of mfma_32x32x16 (same operand and result layouts).
__device__ __forceinline__ f32x16 mfma_32x32x16_h(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// The work is the sequence of 32-key tiles of every (kv head, request) pair,
// kv-head-major: for each kv head, the requests in order, each request's
// tiles 0 .. P_b - 1 (P_b = ceil((L_b + K + 1) / 32), 0 for an invalid
// request).  first[b] is the exclusive prefix sum of P_b (first[B] = Th, the
// tiles of one kv head), written by attn_items; global tile g is tile
// g % Th of kv head g / Th.  With T = Th * Hkv tiles and n = min(nw, T) of
// the nw waves in use, wave w < n runs tiles [tile_lo(w), tile_lo(w + 1)),
// tile_lo(w) = floor(w T / n): every wave gets the same number of tiles to
// one, and at least one.  All cursor fields are wave-uniform.
struct TileCursor {
    int g, hi;          // global tile, end of the wave's range
    int kvh, b, t, P;   // kv head, request, tile within the pair, tiles of the pair
    int L;              // seq_lens[b]
    int pg;             // physical page of the tile (DMA cursors)
};

__device__ __forceinline__ void cursor_begin(TileCursor& c, int lo, int hi, int B, int Th,
                                             const int32_t* __restrict__ first,
                                             const int32_t* __restrict__ seq_lens) {
    c.g = lo;
    c.hi = hi;
    if (lo >= hi) return;
    c.kvh = lo / Th;
    const int r = lo - c.kvh * Th;
    int b0 = 0, b1 = B;  // largest b with first[b] <= r (first[B] = Th > r)
    while (b1 - b0 > 1) {
        const int mid = (b0 + b1) >> 1;
        if (first[mid] <= r) b0 = mid; else b1 = mid;
    }
    c.b = b0;
    c.t = r - first[b0];
    c.P = first[b0 + 1] - first[b0];
    c.L = seq_lens[b0];
}

__device__ __forceinline__ void cursor_next(TileCursor& c, int B,
                                            const int32_t* __restrict__ first,
                                            const int32_t* __restrict__ seq_lens) {
    if (++c.g >= c.hi) return;
    if (++c.t < c.P) return;
    // Next pair with tiles; one exists because g < hi <= T.
    c.t = 0;
    do {
        if (++c.b == B) {
            c.b = 0;
            ++c.kvh;
        }
        c.P = first[c.b + 1] - first[c.b];
    } while (c.P == 0);
    c.L = seq_lens[c.b];
}

// Workgroups per CU: two for E4M3 tiles with one row block (a 20 KiB ring per
// wave at head dim 128, 256 registers), so that one wave's softmax overlaps
// another's MFMAs and waits; one otherwise (the bf16 ring fills the LDS).
template <int D, int RB, bool F8>
constexpr int gqa_groups_per_cu() { return (F8 && RB == 1) ? 2 : 1; }

// K ring stages (V has one fewer): as deep as the LDS allows for the
// workgroups per CU, at most 5.
template <int D, int RB, bool F8>
constexpr int gqa_kstages() {
    constexpr int half = 32 * D * (F8 ? 1 : 2);
    constexpr int per_wave = 160 * 1024 / (4 * gqa_groups_per_cu<D, RB, F8>());
    constexpr int ks = (per_wave / half + 1) / 2;  // KS + (KS - 1) halves
    return ks > 5 ? 5 : ks;
}

// s_waitcnt for at most g half tiles of H vm ops each still in flight (a
// larger g than the counter can express waits for fewer, which is safe).
template <int H, int G = 0>
__device__ __forceinline__ void wait_halves(int g) {
    if constexpr ((G + 1) * H > 63) {
        wait_vmcnt<G * H>();
    } else {
        if (g <= G) wait_vmcnt<G * H>();
        else wait_halves<H, G + 1>(g);
    }
}

template <int D, int RB, bool F8>
__global__ __launch_bounds__(256, (gqa_groups_per_cu<D, RB, F8>())) void attn_gqa_stream(
    const uint16_t* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ first,
    float* __restrict__ part_o, float2* __restrict__ part_ml, float* __restrict__ out,
    uint16_t* __restrict__ out_lowp, int B, int NQ, int Hq, int Hkv, int G, int R, int max_pages,
    float scale_log2, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const uint64_t* __restrict__ anc) {
    using T = GqaTile<D, F8, gqa_kstages<D, RB, F8>()>;
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
        goff[j] = row * T::kRowBytes + 16 * ((n % T::kRowChunks) ^ gqa_xor<D, F8>(row));
    }
    const size_t head_bytes = (size_t)kPage * T::kRowBytes;
    char* const k_ring = ring;
    char* const v_ring = ring + T::kKStages * T::kHalfBytes;
    // The page-table entry of a DMA cursor's tile is read when the cursor
    // reaches the tile, one issue before it is needed, so the scalar load's
    // latency is not on the DMA's critical path.
    auto load_pg = [&](TileCursor& c) {
        if (c.g < c.hi) c.pg = page_table[(size_t)c.b * max_pages + (kTile * c.t) / kPage];
    };
    auto issue = [&](const char* __restrict__ cache, const TileCursor& c, const char* dst_p) {
        const int ks = kTile * c.t;
        const char* src = cache + ((size_t)c.pg * Hkv + c.kvh) * head_bytes +
                          (size_t)(ks % kPage) * T::kRowBytes;
        const uint32_t dst = lds_byte_addr(dst_p);
        // The stage's previous tile was read by this wave's ds_reads; make
        // sure they have returned before the DMA may overwrite it.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < T::kDmaHalf; ++j)
            dma16(src + goff[j], __builtin_amdgcn_readfirstlane(dst + 1024u * j));
    };

    // Per-lane LDS byte offsets within a half tile.
    //  K reads of k-step s: row ln, logical chunk 2s + lh (bf16); E4M3: one
    //  read per k-step pair j = s/2, logical chunk 2j + lh (dims 32j + 16lh
    //  .. +15), its bytes 0-7 for step 2j and 8-15 for step 2j+1 -- the
    //  contraction runs over the dims in that order, and Q follows it.
    constexpr int NKR = F8 ? NS / 2 : NS;
    int koff[NKR];
#pragma unroll
    for (int s = 0; s < NKR; ++s)
        koff[s] = ln * T::kRowBytes + 16 * ((2 * s + lh) ^ gqa_xor<D, F8>(ln));
    //  V reads (16-lane group g, lane sl) of dim block db, half h: key
    //  16tt + 4(g/2) + sl/4 + 8h, logical chunk 4db + 2(g&1) + (sl&3)/2, byte
    //  8(sl&1) of the chunk (the swizzle depends on the key only modulo 16).
    //  E4M3 (ds_read_b64_tr_b8: in each 16-lane group, lane t receives byte
    //  t%8 of the 8-byte reads of lanes t/8 + 2e, e = 0..7): lane sl reads
    //  key 16tt + 8(e/4) + 4(g/2) + e%4 with e = sl/2, bytes 16(g&1) + 8(sl&1)
    //  .. +7 of dim block db, so lane t receives its dim's 8 keys in operand
    //  slot order.
    const int g4 = lane >> 4, sl = lane & 15;
    int voff[NDB][F8 ? 1 : 2];
    if constexpr (F8) {
        const int e = sl >> 1;
        const int vr = 8 * (e >> 2) + 4 * (g4 >> 1) + (e & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            voff[db][0] = vr * T::kRowBytes + 16 * ((2 * db + (g4 & 1)) ^ gqa_xor<D, F8>(vr)) +
                          8 * (sl & 1);
    } else {
        const int vch = 2 * (g4 & 1) + ((sl & 3) >> 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int vr = 4 * (g4 >> 1) + (sl >> 2) + 8 * h;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                voff[db][h] = vr * T::kRowBytes + 16 * ((4 * db + vch) ^ gqa_xor<D, F8>(vr)) +
                              8 * (sl & 1);
        }
    }

    // Three cursors over the wave's tile stream: K DMA (S = kKStages tiles
    // ahead of the compute), V DMA (S - 1 ahead) and compute.  Issue order:
    // K0, then K(i) V(i-1) for i < S, then after computing tile c: K(c+S)
    // V(c+S-1).  nk / nv count the halves issued; vmcnt waits count the 1 KiB
    // ops issued after the one needed (DMAs complete in issue order).
    // With fewer tiles than waves only the first T waves take one tile each,
    // so that every wave in use has work (the combine relies on it).
    const int Th = first[B];
    const long n_tiles = (long)Th * Hkv;
    const int gw = blockIdx.x * 4 + wave;
    const int nwe = (int)min((long)nw, n_tiles);
    TileCursor kc;
    if (gw < nwe)
        cursor_begin(kc, (int)(n_tiles * gw / nwe), (int)(n_tiles * (gw + 1) / nwe), B, Th, first,
                     seq_lens);
    else
        kc.g = kc.hi = 0;
    load_pg(kc);
    TileCursor vc = kc, cc = kc;
    int nk = 0, nv = 0;
    // issue_k / issue_v advance their cursor without reading its next page
    // entry: the main loop reads both entries right after the tile's K
    // fragments have been read from LDS, so that the scalar loads complete
    // under the softmax instead of stalling the next LDS wait (LDS reads and
    // scalar loads share one counter).
    auto issue_k = [&]() {
        if (kc.g < kc.hi) {
            issue(k_cache, kc, k_ring + (nk % T::kKStages) * T::kHalfBytes);
            ++nk;
            cursor_next(kc, B, first, seq_lens);
        }
    };
    auto issue_v = [&]() {
        if (vc.g < vc.hi) {
            issue(v_cache, vc, v_ring + (nv % T::kVStages) * T::kHalfBytes);
            ++nv;
            cursor_next(vc, B, first, seq_lens);
        }
    };
    auto wait_groups = [&](int g) { wait_halves<T::kDmaHalf>(g); };
    issue_k();
    load_pg(kc);
#pragma unroll
    for (int i = 1; i < T::kKStages; ++i) {
        issue_k();
        load_pg(kc);
        issue_v();
        load_pg(vc);
    }
    int cseq = 0;

    u32x4 qf[RB][NS];
    int lim[RB];
    uint32_t vis_lo[RB], vis_hi[RB];  // draft tree: new keys L_b + a the row's node sees
    float m_r[RB], l_r[RB];
    float sl2 = scale_log2, vsc = 1.f;  // per pair: key scale folded in; value scale
    f32x16 o[RB][NDB];
    // The wave's tiles of one (request, kv head) pair form a segment: Q and the
    // online softmax state live in registers across it, and it is written
    // once, at its end.  Only the wave's first and last segments can miss
    // tiles of their pair (the others cover whole pairs).
    int seg_t0 = 0;
    bool first_seg = true;
    while (cc.g < cc.hi) {
        // K(cseq) has landed once at most the halves issued after it are in
        // flight: K(j > cseq) and V(j >= max(cseq - 1, 0)).
        wait_groups((nk - 1 - cseq) + (nv - max(cseq - 1, 0)));
        const int cend = cc.L + NQ;  // keys of the pair
        if (cc.t == 0 || cseq == 0) {
            seg_t0 = cc.t;
            if constexpr (F8) {
                sl2 = scale_log2 * k_scale[cc.kvh];
                vsc = v_scale[cc.kvh] * kPScaleInv;
            }
            // New segment: Q fragments (B operand; column = query row, k = d;
            // E4M3: the dims of k-step s are 32(s/2) + 16lh + 8(s%2) .. +7).
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = rb * 32 + ln;
                if (row < R) {
                    const int i = row / G, gq = row - i * G;
                    const uint16_t* qp = q + (((size_t)cc.b * NQ + i) * Hq + cc.kvh * G + gq) * D +
                                         (F8 ? 16 : 8) * lh;
#pragma unroll
                    for (int s = 0; s < NS; ++s)
                        qf[rb][s] = *(const u32x4*)(qp + (F8 ? 32 * (s >> 1) + 8 * (s & 1) : 16 * s));
                    lim[rb] = cc.L + i;  // causal: keys 0 .. L_b + i
                    const uint64_t m = anc ? anc[(size_t)cc.b * NQ + i] : ~0ull;
                    vis_lo[rb] = (uint32_t)m;
                    vis_hi[rb] = (uint32_t)(m >> 32);
                } else {
#pragma unroll
                    for (int s = 0; s < NS; ++s) qf[rb][s] = u32x4{0, 0, 0, 0};
                    lim[rb] = cc.L + NQ - 1;
                    vis_lo[rb] = vis_hi[rb] = ~0u;
                }
                m_r[rb] = -INFINITY;
                l_r[rb] = 0.f;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[rb][db][r] = 0.f;
            }
            // The Q loads share vmcnt with the LDS DMAs the compiler cannot
            // see: wait for them here, once per segment, so that the compiler
            // knows them complete on every path into the tile loop body and
            // inserts no vmcnt wait there (which would also drain the tiles
            // prefetched ahead).
            wait_vmcnt<0>();
        }
        const char* ktile = k_ring + (cseq % T::kKStages) * T::kHalfBytes;
        char* vtile = v_ring + (cseq % T::kVStages) * T::kHalfBytes;
        const int ks = kTile * cc.t;
        // S^T = K Q^T, the even and odd k-steps in two independent MFMA
        // chains (half the dependent latency), every K fragment read from LDS
        // before the first MFMA.
        f32x16 sacc[RB], sacc2[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[rb][r] = sacc2[rb][r] = 0.f;
        if constexpr (F8) {
            u32x4 raw[NKR];
#pragma unroll
            for (int j = 0; j < NKR; ++j) raw[j] = *(const u32x4*)(ktile + koff[j]);
#pragma unroll
            for (int j = 0; j < NKR; ++j) {
                const u32x4 k0 = e4m3x8_to_bf16(raw[j][0], raw[j][1]);
                const u32x4 k1 = e4m3x8_to_bf16(raw[j][2], raw[j][3]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    sacc[rb] = mfma_32x32x16(k0, qf[rb][2 * j], sacc[rb]);
                    sacc2[rb] = mfma_32x32x16(k1, qf[rb][2 * j + 1], sacc2[rb]);
                }
            }
        } else {
            u32x4 kf[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) kf[s] = *(const u32x4*)(ktile + koff[s]);
#pragma unroll
            for (int s = 0; s < NS; s += 2)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    sacc[rb] = mfma_32x32x16(kf[s], qf[rb][s], sacc[rb]);
                    sacc2[rb] = mfma_32x32x16(kf[s + 1], qf[rb][s + 1], sacc2[rb]);
                }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[rb] += sacc2[rb];
        load_pg(kc);
        load_pg(vc);

        // Online softmax; lane (ln, lh) holds 16 keys of query row ln.  A
        // tile whose keys all lie before the chunk end and at or before L_b
        // (the causal limit of the first query) needs no mask.
        const bool unmasked = ks + kTile <= cend && ks + kTile - 1 <= cc.L;
        u32x4 pb[RB][2], pbl[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float tmax = -INFINITY;
            if (unmasked) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[rb][r] *= sl2;
                    tmax = fmaxf(tmax, sacc[rb][r]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = ks + mfma_row(r, lane);
                    const float v = sacc[rb][r] * sl2;
                    bool seen;
                    if (anc) {  // a tree: key L_b + a is seen iff bit a of the node's mask
                        const int a = key - cc.L;
                        seen = a < 0 ||
                               (a < 64 &&
                                ((a < 32 ? vis_lo[rb] >> a : vis_hi[rb] >> (a - 32)) & 1u) != 0);
                    } else {
                        seen = key <= lim[rb];
                    }
                    sacc[rb][r] = (key >= cend || !seen) ? -INFINITY : v;
                    tmax = fmaxf(tmax, sacc[rb][r]);
                }
            }
            tmax = halves_max(tmax);
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
                psum += p0 + p1;
                if constexpr (F8) {
                    pk[r >> 1] = cvt_pk_f16(p0 * kPScale, p1 * kPScale);
                    pl[r >> 1] = 0u;
                } else {
                    const uint32_t hi = cvt_pk_bf16(p0, p1);
                    pk[r >> 1] = hi;
                    pl[r >> 1] = cvt_pk_bf16(p0 - __uint_as_float(hi << 16),
                                             p1 - __uint_as_float(hi & 0xffff0000u));
                }
            }
            psum = halves_sum(psum);
            l_r[rb] += psum;
            pb[rb][0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
            pb[rb][1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
            pbl[rb][0] = u32x4{pl[0], pl[1], pl[2], pl[3]};
            pbl[rb][1] = u32x4{pl[4], pl[5], pl[6], pl[7]};
        }

        // V(cseq) has landed once at most V(j > cseq) and K(j >= cseq + 2) are
        // in flight.
        wait_groups((nv - 1 - cseq) + max(0, nk - (cseq + 2)));
        if (ks + kTile > cend) {
            // Rows past the last key may hold anything (NaN included): zero
            // their values so that P = 0 contributes exactly nothing.
            const int nv = cend - ks;
            for (int idx = lane; idx < (kTile - nv) * T::kRowChunks; idx += 64) {
                const int row = nv + idx / T::kRowChunks, c = idx % T::kRowChunks;
                *(u32x4*)(vtile + row * T::kRowBytes + 16 * (c ^ gqa_xor<D, F8>(row))) =
                    u32x4{0, 0, 0, 0};
            }
        }

        // O^T += V^T P^T.  Slot 8h + 4a + r of step tt is key 16tt + 8a + 4h + r.
        // Every V fragment is read from LDS before the first MFMA.
        u32x4 vf[2][NDB];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const char* vp = vtile + 16 * tt * T::kRowBytes;
                if constexpr (F8) {
                    const u32x2 raw = lds_read_tr8(vp + voff[db][0]);
                    vf[tt][db] = u32x4{raw.x, raw.y, 0u, 0u};
                } else {
                    const u32x2 v0 = lds_read_tr16(vp + voff[db][0]);
                    const u32x2 v1 = lds_read_tr16(vp + voff[db][1]);
                    vf[tt][db] = u32x4{v0.x, v0.y, v1.x, v1.y};
                }
            }
        // This tile's stages are read (K in S^T; the V fragments above, which
        // the lgkmcnt wait below completes): refill them kKStages (K) and
        // kVStages (V) tiles ahead in the wave's stream, the DMA ops
        // interleaved with the V^T blocks (K ops in key half 0, V ops in key
        // half 1) so that their issue stalls overlap this wave's MFMAs.  The
        // issue order is unchanged (K before V), so the vmcnt waits hold.
        constexpr int OPB = T::kDmaHalf / NDB;  // DMA ops per V^T block
        static_assert(OPB * NDB == T::kDmaHalf, "refill ops split evenly over the blocks");
        const bool dk = kc.g < kc.hi, dv = vc.g < vc.hi;
        const char* ksrc = k_cache + ((size_t)kc.pg * Hkv + kc.kvh) * head_bytes +
                           (size_t)((kTile * kc.t) % kPage) * T::kRowBytes;
        const char* vsrc = v_cache + ((size_t)vc.pg * Hkv + vc.kvh) * head_bytes +
                           (size_t)((kTile * vc.t) % kPage) * T::kRowBytes;
        const uint32_t kdst = lds_byte_addr(k_ring + (nk % T::kKStages) * T::kHalfBytes);
        const uint32_t vdst = lds_byte_addr(v_ring + (nv % T::kVStages) * T::kHalfBytes);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if constexpr (F8) {
                    const u32x4 a = e4m3x8_to_f16(vf[tt][db][0], vf[tt][db][1]);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        o[rb][db] = mfma_32x32x16_h(a, pb[rb][tt], o[rb][db]);
                } else {
                    const u32x4 a = vf[tt][db];
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        o[rb][db] = mfma_32x32x16(a, pb[rb][tt], o[rb][db]);
                        o[rb][db] = mfma_32x32x16(a, pbl[rb][tt], o[rb][db]);
                    }
                }
#pragma unroll
                for (int u = 0; u < OPB; ++u) {
                    const int j = db * OPB + u;
                    if (tt == 0) {
                        if (dk)
                            dma16(ksrc + goff[j], __builtin_amdgcn_readfirstlane(kdst + 1024u * j));
                    } else if (dv) {
                        dma16(vsrc + goff[j], __builtin_amdgcn_readfirstlane(vdst + 1024u * j));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        if (dk) {
            ++nk;
            cursor_next(kc, B, first, seq_lens);
        }
        if (dv) {
            ++nv;
            cursor_next(vc, B, first, seq_lens);
        }
        const bool last_of_pair = cc.t == cc.P - 1;
        if (last_of_pair || cc.g + 1 >= cc.hi) {
            if (seg_t0 == 0 && last_of_pair) {
                // The segment covers the whole pair: normalised rows straight
                // to the output.  Lane (ln, lh) holds dims 8(r/4) + 4lh + r%4.
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int row = rb * 32 + ln;
                    if (row >= R) continue;
                    const int i = row / G, gq = row - i * G;
                    const size_t oi = (((size_t)cc.b * NQ + i) * Hq + cc.kvh * G + gq) * D;
                    const float inv = vsc / l_r[rb];
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
            } else {
                // Partial rows in the wave's slot: 2w for its first segment,
                // 2w + 1 for its last.
                const size_t pidx = 2 * (size_t)gw + (first_seg ? 0 : 1);
                // Dim d of row `row` at po[d * R + row], d = 32db + 8(r/4) +
                // 4lh + r%4: the lane's part (4lh) in the base pointer, the
                // rest a wave-uniform index.  R passes through an empty asm
                // so that the compiler computes the offsets in this (rare)
                // block instead of hoisting them out of the tile loop, where
                // they would be kept in (or spilled from) registers.
                int Ro = R;
                asm volatile("" : "+s"(Ro));
                float* po = part_o + pidx * D * Ro + 4 * lh * Ro;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int row = rb * 32 + ln;
                    if (row >= Ro) continue;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            po[(db * 32 + 8 * (r >> 2) + (r & 3)) * Ro + row] =
                                F8 ? o[rb][db][r] * vsc : o[rb][db][r];
                    if (lh == 0) part_ml[pidx * Ro + row] = make_float2(m_r[rb], l_r[rb]);
                }
            }
            first_seg = false;
        }
        cursor_next(cc, B, first, seq_lens);
        ++cseq;
    }
}

// E4M3 cache, head dim 128, 33..48 query rows per (request, kv head): the
// same tile stream with 16x16x32 MFMA blocks, so the rows pad to 48 instead
// of 64 (a quarter less MFMA and softmax work per tile) and the wave's state
// fits two waves per SIMD (two workgroups per CU, a 20 KiB ring per wave):
// one wave's softmax, conversions and DMA issue overlap the other's MFMAs.
// Operand layouts (lane l, g = l / 16): A row l%16, k = 8g..8g+7; B column
// l%16, same k; result: lane l holds column l%16, rows 4g..4g+3.
//   S^T block kb (kb = 0, 1) of a tile: MFMA row i is key 8(i/4) + 4kb + i%4,
//     so lane group g holds keys 8g..8g+7 of its query row (slot e = 4kb + r
//     is key 8g + e), which is the k order of the P^T operand of O^T += V^T P^T;
//   k-steps 2j and 2j+1 (j = 0, 1) of lane group g run over dims
//     16(4j + g) .. +7 and +8 .. +15: one 16-byte read of a K row, Q following.
// Swizzle: the 32-row kernels' E4M3 one (gqa_xor<128, true>).  Measured
// with SQ_LDS_BANK_CONFLICT on the two read patterns alone, it leaves both
// free of bank conflicts, while two swizzles derived for K-read passes of 16
// consecutive lanes (every lane group reads the same 16 rows at its own
// chunk) conflicted on 40% of the K-read cycles.

__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_h(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query row of a
// 16x16 result), the same value in all four lanes.
__device__ __forceinline__ float quads_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return halves_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quads_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return halves_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

template <int NB>
__global__ __launch_bounds__(256, 2) void attn_gqa_f8_r16(
    const uint16_t* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ first,
    float* __restrict__ part_o, float2* __restrict__ part_ml, float* __restrict__ out,
    uint16_t* __restrict__ out_lowp, int B, int NQ, int Hq, int Hkv, int G, int R, int max_pages,
    float scale_log2, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const uint64_t* __restrict__ anc) {
    constexpr int D = 128;
    using T = GqaTile<D, true, 3>;
    static_assert(T::kRingBytes * 8 <= 160 * 1024, "two workgroups of four rings per CU");
    constexpr int NDB = D / 16;  // 16-dim blocks of O^T
    __shared__ __attribute__((aligned(1024))) char s_ring[4][T::kRingBytes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int nw = gridDim.x * 4;
    char* ring = s_ring[wave];

    int goff[T::kDmaHalf];
#pragma unroll
    for (int j = 0; j < T::kDmaHalf; ++j) {
        const int n = 64 * j + lane;
        const int row = n / T::kRowChunks;
        goff[j] = row * T::kRowBytes + 16 * ((n % T::kRowChunks) ^ gqa_xor<D, true>(row));
    }
    const size_t head_bytes = (size_t)kPage * T::kRowBytes;
    char* const k_ring = ring;
    char* const v_ring = ring + T::kKStages * T::kHalfBytes;
    auto load_pg = [&](TileCursor& c) {
        if (c.g < c.hi) c.pg = page_table[(size_t)c.b * max_pages + (kTile * c.t) / kPage];
    };
    auto issue = [&](const char* __restrict__ cache, const TileCursor& c, const char* dst_p) {
        const int ks = kTile * c.t;
        const char* src = cache + ((size_t)c.pg * Hkv + c.kvh) * head_bytes +
                          (size_t)(ks % kPage) * T::kRowBytes;
        const uint32_t dst = lds_byte_addr(dst_p);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < T::kDmaHalf; ++j)
            dma16(src + goff[j], __builtin_amdgcn_readfirstlane(dst + 1024u * j));
    };

    // K reads of block kb, k-step pair j: key 8(li/4) + 4kb + li%4, logical
    // chunk 4j + lg.
    int koff[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int key = 8 * (li >> 2) + 4 * kb + (li & 3);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            koff[kb][j] = key * T::kRowBytes + 16 * ((4 * j + lg) ^ gqa_xor<D, true>(key));
    }
    // V reads of dim block db (ds_read_b64_tr_b8: lane t of a 16-lane group
    // receives byte t%8 of the reads of lanes t/8 + 2e as byte e): lane li
    // reads key 8lg + li/2, dims 16db + 8(li&1) .. +7, so lane t receives dim
    // 16db + t of keys 8lg .. 8lg+7 in slot order.
    const int vkey = 8 * lg + (li >> 1);
    const int vbase = vkey * T::kRowBytes + 8 * (li & 1), vx = gqa_xor<D, true>(vkey);

    const int Th = first[B];
    const long n_tiles = (long)Th * Hkv;
    const int gw = blockIdx.x * 4 + wave;
    const int nwe = (int)min((long)nw, n_tiles);
    TileCursor kc;
    if (gw < nwe)
        cursor_begin(kc, (int)(n_tiles * gw / nwe), (int)(n_tiles * (gw + 1) / nwe), B, Th, first,
                     seq_lens);
    else
        kc.g = kc.hi = 0;
    load_pg(kc);
    TileCursor vc = kc, cc = kc;
    int nk = 0, nv = 0;
    auto issue_k = [&]() {
        if (kc.g < kc.hi) {
            issue(k_cache, kc, k_ring + (nk % T::kKStages) * T::kHalfBytes);
            ++nk;
            cursor_next(kc, B, first, seq_lens);
        }
    };
    auto issue_v = [&]() {
        if (vc.g < vc.hi) {
            issue(v_cache, vc, v_ring + (nv % T::kVStages) * T::kHalfBytes);
            ++nv;
            cursor_next(vc, B, first, seq_lens);
        }
    };
    auto wait_groups = [&](int g) { wait_halves<T::kDmaHalf>(g); };
    issue_k();
    load_pg(kc);
#pragma unroll
    for (int i = 1; i < T::kKStages; ++i) {
        issue_k();
        load_pg(kc);
        issue_v();
        load_pg(vc);
    }
    int cseq = 0;

    u32x4 qf[NB][4];
    float m_r[NB], l_r[NB];
    float sl2 = scale_log2, vsc = 1.f;
    f32x4 o[NB][NDB];
    int seg_t0 = 0;
    bool first_seg = true;
    while (cc.g < cc.hi) {
        wait_groups((nk - 1 - cseq) + (nv - max(cseq - 1, 0)));
        const int cend = cc.L + NQ;
        if (cc.t == 0 || cseq == 0) {
            seg_t0 = cc.t;
            sl2 = scale_log2 * k_scale[cc.kvh];
            vsc = v_scale[cc.kvh] * kPScaleInv;
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                const int row = rb * 16 + li;
                if (row < R) {
                    const int i = row / G, gq = row - i * G;
                    const uint16_t* qp = q + (((size_t)cc.b * NQ + i) * Hq + cc.kvh * G + gq) * D +
                                         16 * lg;
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        qf[rb][s] = *(const u32x4*)(qp + 64 * (s >> 1) + 8 * (s & 1));
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s) qf[rb][s] = u32x4{0, 0, 0, 0};
                }
                m_r[rb] = -INFINITY;
                l_r[rb] = 0.f;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            wait_vmcnt<0>();
        }
        const char* ktile = k_ring + (cseq % T::kKStages) * T::kHalfBytes;
        char* vtile = v_ring + (cseq % T::kVStages) * T::kHalfBytes;
        const int ks = kTile * cc.t;

        // S^T = K Q^T: NB x 2 independent accumulators, four k-steps each.
        f32x4 sacc[NB][2];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sacc[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 raw[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j) raw[kb][j] = *(const u32x4*)(ktile + koff[kb][j]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 k0 = e4m3x8_to_bf16(raw[kb][j][0], raw[kb][j][1]);
                const u32x4 k1 = e4m3x8_to_bf16(raw[kb][j][2], raw[kb][j][3]);
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
                    sacc[rb][kb] = mfma_16x16x32(k0, qf[rb][2 * j], sacc[rb][kb]);
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
                    sacc[rb][kb] = mfma_16x16x32(k1, qf[rb][2 * j + 1], sacc[rb][kb]);
            }
        load_pg(kc);
        load_pg(vc);

        // Online softmax; lane (li, lg) holds keys 8lg .. 8lg+7 of query row
        // 16rb + li (slot e = 4kb + r).
        const bool unmasked = ks + kTile <= cend && ks + kTile - 1 <= cc.L;
        u32x4 pb[NB];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            float sv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[e] = sacc[rb][e >> 2][e & 3] * sl2;
            if (!unmasked) {
                // The row's position (padding rows see every key of the
                // pair) and, for a draft tree, its node's visibility mask,
                // read here: masked tiles are at most two per pair.
                const int row = rb * 16 + li;
                const int i = row < R ? row / G : NQ - 1;
                const uint64_t vis = (anc && row < R) ? anc[(size_t)cc.b * NQ + i] : ~0ull;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = ks + 8 * lg + e;
                    const int a = key - cc.L;
                    const bool seen = anc ? (a < 0 || (a < 64 && ((vis >> a) & 1u) != 0))
                                          : key <= cc.L + i;
                    if (key >= cend || !seen) sv[e] = -INFINITY;
                }
            }
            float tmax = sv[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, sv[e]);
            tmax = quads_max(tmax);
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
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(sv[e] - msafe);
                const float p1 = __builtin_amdgcn_exp2f(sv[e + 1] - msafe);
                psum += p0 + p1;
                pk[e >> 1] = cvt_pk_f16(p0 * kPScale, p1 * kPScale);
            }
            l_r[rb] += quads_sum(psum);
            pb[rb] = u32x4{pk[0], pk[1], pk[2], pk[3]};
        }

        wait_groups((nv - 1 - cseq) + max(0, nk - (cseq + 2)));
        if (ks + kTile > cend) {
            const int nvk = cend - ks;
            for (int idx = lane; idx < (kTile - nvk) * T::kRowChunks; idx += 64) {
                const int row = nvk + idx / T::kRowChunks, c = idx % T::kRowChunks;
                *(u32x4*)(vtile + row * T::kRowBytes + 16 * (c ^ gqa_xor<D, true>(row))) =
                    u32x4{0, 0, 0, 0};
            }
        }

        // O^T += V^T P^T, every V fragment read before the first MFMA.
        __builtin_amdgcn_sched_barrier(0);
        u32x2 vr[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) vr[db] = lds_read_tr8(vtile + vbase + 16 * (db ^ vx));
        // Refills of this tile's stages, one DMA op after each V^T block (as in
        // attn_gqa_stream: K ops first, then V).
        const bool dk = kc.g < kc.hi, dv = vc.g < vc.hi;
        const char* ksrc = k_cache + ((size_t)kc.pg * Hkv + kc.kvh) * head_bytes +
                           (size_t)((kTile * kc.t) % kPage) * T::kRowBytes;
        const char* vsrc = v_cache + ((size_t)vc.pg * Hkv + vc.kvh) * head_bytes +
                           (size_t)((kTile * vc.t) % kPage) * T::kRowBytes;
        const uint32_t kdst = lds_byte_addr(k_ring + (nk % T::kKStages) * T::kHalfBytes);
        const uint32_t vdst = lds_byte_addr(v_ring + (nv % T::kVStages) * T::kHalfBytes);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const u32x4 a = e4m3x8_to_f16(vr[db].x, vr[db].y);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) o[rb][db] = mfma_16x16x32_h(a, pb[rb], o[rb][db]);
            static_assert(NDB == 2 * T::kDmaHalf, "one refill op per V^T block");
            if (db < T::kDmaHalf) {
                if (dk) dma16(ksrc + goff[db], __builtin_amdgcn_readfirstlane(kdst + 1024u * db));
            } else if (dv) {
                const int j = db - T::kDmaHalf;
                dma16(vsrc + goff[j], __builtin_amdgcn_readfirstlane(vdst + 1024u * j));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (dk) {
            ++nk;
            cursor_next(kc, B, first, seq_lens);
        }
        if (dv) {
            ++nv;
            cursor_next(vc, B, first, seq_lens);
        }
        const bool last_of_pair = cc.t == cc.P - 1;
        if (last_of_pair || cc.g + 1 >= cc.hi) {
            if (seg_t0 == 0 && last_of_pair) {
                // Lane (li, lg) holds dims 16db + 4lg .. +3 of row 16rb + li.
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    const int row = rb * 16 + li;
                    if (row >= R) continue;
                    const int i = row / G, gq = row - i * G;
                    const size_t oi = (((size_t)cc.b * NQ + i) * Hq + cc.kvh * G + gq) * D;
                    const float inv = vsc / l_r[rb];
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const int d = db * 16 + 4 * lg;
                        const f32x4 v = o[rb][db] * inv;
                        *(f32x4*)(out + oi + d) = v;
                        if (out_lowp) {
                            u32x2 w;
                            w.x = pack_bf16x2(v[0], v[1]);
                            w.y = pack_bf16x2(v[2], v[3]);
                            *(u32x2*)(out_lowp + oi + d) = w;
                        }
                    }
                }
            } else {
                const size_t pidx = 2 * (size_t)gw + (first_seg ? 0 : 1);
                // Dim 16db + 4lg + r of row `row` at po[dim * R + row]; R
                // passes through an empty asm as in attn_gqa_stream.
                int Ro = R;
                asm volatile("" : "+s"(Ro));
                float* po = part_o + pidx * D * Ro + 4 * lg * Ro;
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    const int row = rb * 16 + li;
                    if (row >= Ro) continue;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            po[(db * 16 + r) * Ro + row] = o[rb][db][r] * vsc;
                    if (lg == 0) part_ml[pidx * Ro + row] = make_float2(m_r[rb], l_r[rb]);
                }
            }
            first_seg = false;
        }
        cursor_next(cc, B, first, seq_lens);
        ++cseq;
    }
}

// first[b] = number of 32-key tiles of the valid requests before b (exclusive
// prefix sum), first[B] = their total.  One block.
__global__ __launch_bounds__(1024) void attn_items(const int32_t* __restrict__ seq_lens,
                                                   const int32_t* __restrict__ valid,
                                                   int32_t* __restrict__ first, int B, int NQ) {
    __shared__ int32_t s_sum[1024];
    __shared__ int32_t s_carry;
    if (threadIdx.x == 0) s_carry = 0;
    for (int b0 = 0; b0 < B; b0 += 1024) {
        const int b = b0 + threadIdx.x;
        const int n = (b < B && valid[b]) ? (seq_lens[b] + NQ + kTile - 1) / kTile : 0;
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

}  // namespace

// Tile prefix, then the persistent kernel: gqa_groups_per_cu 4-wave
// workgroups per CU, at most max_waves waves in all.  *nw receives the number
// of waves launched (the combine needs it to find each pair's slots).
int gqa_launch(const sd_attn_desc* d, const int32_t* valid, int32_t* first, const uint64_t* anc,
               float* po, float2* pml, int R, int max_waves, float scale_log2, int* nw,
               hipStream_t s) {
    int num_cus = 0;
    int rc = cu_count("sd_verify_attn", &num_cus);
    if (rc != SD_OK) return rc;
    attn_items<<<1, 1024, 0, s>>>(d->seq_lens, valid, first, d->batch, d->num_q);
    rc = check_launch("attn_items");
    if (rc != SD_OK) return rc;
    const int G = d->n_q_heads / d->n_kv_heads;
    const bool f8 = d->kv_format == SD_KV_E4M3;
    // gqa_groups_per_cu of the variant launched (it does not depend on D)
    // 33..48 rows with an E4M3 cache at head dim 128: 16-row blocks
    // (attn_gqa_f8_r16, two workgroups per CU).
    const bool r16 = f8 && d->d_qk == 128 && R > 32 && R <= 48;
    const int groups = r16 ? 2
                       : (f8 && R <= 32) ? gqa_groups_per_cu<128, 1, true>()
                                         : gqa_groups_per_cu<128, 2, false>();
    const int grid = std::min(num_cus * groups, max_waves / 4);
    *nw = 4 * grid;
#define SDV_LAUNCH_GQA(DD, RBB, F8)                                                              \
    attn_gqa_stream<DD, RBB, F8><<<grid, 256, 0, s>>>(                                           \
        (const uint16_t*)d->q, (const char*)d->k_cache, (const char*)d->v_cache, d->page_table,  \
        d->seq_lens, first, po, pml, d->out, (uint16_t*)d->out_lowp, d->batch, d->num_q,         \
        d->n_q_heads, d->n_kv_heads, G, R, d->max_pages, scale_log2, d->k_scale, d->v_scale, anc)
    if (d->d_qk == 128) {
        if (f8) {
            if (R <= 32) {
                SDV_LAUNCH_GQA(128, 1, true);
            } else if (r16) {
                attn_gqa_f8_r16<3><<<grid, 256, 0, s>>>(
                    (const uint16_t*)d->q, (const char*)d->k_cache, (const char*)d->v_cache,
                    d->page_table, d->seq_lens, first, po, pml, d->out, (uint16_t*)d->out_lowp,
                    d->batch, d->num_q, d->n_q_heads, d->n_kv_heads, G, R, d->max_pages,
                    scale_log2, d->k_scale, d->v_scale, anc);
            } else {
                SDV_LAUNCH_GQA(128, 2, true);
            }
        } else {
            if (R <= 32) SDV_LAUNCH_GQA(128, 1, false); else SDV_LAUNCH_GQA(128, 2, false);
        }
    } else {
        if (f8) {
            if (R <= 32) SDV_LAUNCH_GQA(64, 1, true); else SDV_LAUNCH_GQA(64, 2, true);
        } else {
            if (R <= 32) SDV_LAUNCH_GQA(64, 1, false); else SDV_LAUNCH_GQA(64, 2, false);
        }
    }
#undef SDV_LAUNCH_GQA
    return check_launch("attn_gqa_stream");
}

}  // namespace sdv
