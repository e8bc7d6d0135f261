// Verify attention for speculative decoding on gfx950.
//
// [TRT-MTP] "支持 MTP 的注意力機制": the chain's K+1 tokens need only a causal
// mask in the generation attention; [CSDN-MTP] "整体计算流程" step 2: the
// new queries are batched against the cached keys, softmax(QK^T/sqrt(d))V,
// and each new key/value goes into the cache.
//
// Pipeline on one stream:
//   attn_validate   per request: capacity and page-table entries (flags)
//   attn_append     K+1 new keys/values -> cache positions L_b .. L_b+K
//   attn_gqa_bf16   split-KV flash decoding; one workgroup per (request,
//                   kv head, key chunk); every query row of the kv head's
//                   group (G heads x K+1 positions) shares each K/V tile, so
//                   a tile is read from HBM exactly once
//   attn_combine    log-sum-exp merge of the chunk partials
// plus attn_f32_rows, a plain fp32 path for small float32 problems.
//
// MFMA mapping (bf16, 32x32x16): S^T = K Q^T puts one query row per lane
// column, so the online-softmax state and the rescale of O^T = V^T P^T stay
// lane-local.  K tiles go straight from HBM into A-operand registers; V tiles
// are written transposed into a per-wave LDS buffer (keys permuted so each
// A-operand fragment is two 8-byte reads).
#include <math.h>

#include "sdv_device.h"
#include "sdv_internal.h"

namespace sdv {
namespace {

constexpr int kPage = 64;

// ---------------------------------------------------------------------------
// Per-request checks.  valid[b] = 1 when 0 <= L_b <= max_seq_len,
// L_b + NQ <= max_pages * 64 and every page entry covering 0 .. L_b+NQ-1 is a
// pool page.  Later kernels touch only valid requests.
// ---------------------------------------------------------------------------
__global__ void attn_validate(const int32_t* __restrict__ seq_lens,
                              const int32_t* __restrict__ page_table, int32_t* __restrict__ valid,
                              int32_t* err, int NQ, int max_pages, int num_pages, int max_seq_len) {
    const int b = blockIdx.x;
    const int L = seq_lens[b];
    const bool cap_ok =
        L >= 0 && L <= max_seq_len && (long)L + NQ <= (long)max_pages * kPage;
    int bad_page = 0;
    if (cap_ok) {
        const int npg = (L + NQ + kPage - 1) / kPage;
        for (int lp = threadIdx.x; lp < npg; lp += blockDim.x) {
            const int pg = page_table[(size_t)b * max_pages + lp];
            if (pg < 0 || pg >= num_pages) bad_page = 1;
        }
    }
    bad_page = __syncthreads_or(bad_page);
    if (threadIdx.x == 0) {
        valid[b] = (cap_ok && !bad_page) ? 1 : 0;
        if (!cap_ok) set_error(err, SD_DERR_CAPACITY);
        if (bad_page) set_error(err, SD_DERR_PAGE);
    }
}

// ---------------------------------------------------------------------------
// Append: row i of k_new / v_new -> position L_b + i.  One block per (i, b),
// 16-byte copies.  MLA copies the latent row into k_cache only.
// ---------------------------------------------------------------------------
__global__ void attn_append(const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
                            uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                            const int32_t* __restrict__ page_table,
                            const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ valid,
                            int NQ, int Hkv, int row_bytes_k, int row_bytes_v, int max_pages,
                            int mla) {
    const int i = blockIdx.x, b = blockIdx.y;
    if (!valid[b]) return;
    const long pos = (long)seq_lens[b] + i;
    const long pg = page_table[(size_t)b * max_pages + pos / kPage];
    const long off = pos % kPage;
    const int nk = row_bytes_k / 16, nv = row_bytes_v / 16;
    if (mla) {
        const u32x4* src = (const u32x4*)(k_new + ((size_t)b * NQ + i) * row_bytes_k);
        u32x4* dst = (u32x4*)(k_cache + ((size_t)pg * kPage + off) * row_bytes_k);
        for (int c = threadIdx.x; c < nk; c += blockDim.x) dst[c] = src[c];
        return;
    }
    for (int idx = threadIdx.x; idx < Hkv * nk; idx += blockDim.x) {
        const int h = idx / nk, c = idx - h * nk;
        const u32x4* src =
            (const u32x4*)(k_new + (((size_t)b * NQ + i) * Hkv + h) * row_bytes_k) + c;
        u32x4* dst = (u32x4*)(k_cache + (((size_t)pg * Hkv + h) * kPage + off) * row_bytes_k) + c;
        *dst = *src;
    }
    for (int idx = threadIdx.x; idx < Hkv * nv; idx += blockDim.x) {
        const int h = idx / nv, c = idx - h * nv;
        const u32x4* src =
            (const u32x4*)(v_new + (((size_t)b * NQ + i) * Hkv + h) * row_bytes_v) + c;
        u32x4* dst = (u32x4*)(v_cache + (((size_t)pg * Hkv + h) * kPage + off) * row_bytes_v) + c;
        *dst = *src;
    }
}

// Position of key kappa (0..31 within a tile) in a V^T row of LDS.  The
// PV MFMA's k-slot e of fragment half h at step t is key
// 16t + 8(e/4) + 4h + e%4 (that is where the softmax registers put it), so
// storing key kappa at this position makes each half's 8 keys contiguous.
__device__ __forceinline__ int vt_pos(int kappa) {
    return 16 * (kappa >> 4) + 8 * ((kappa & 7) >> 2) + 4 * ((kappa & 15) >> 3) + (kappa & 3);
}

__device__ __forceinline__ uint32_t half16(u32x4 v, int e) {
    return (v[e >> 1] >> (16 * (e & 1))) & 0xffffu;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kVtStride = 36;  // bf16 per V^T row in LDS (72 bytes: 8-byte aligned rows)

template <int D, int RB>
struct GqaSmem {
    static constexpr int kVt = 4 * D * kVtStride * 2;
    static constexpr int kRed = 2 * RB * 32 * D * 4 + 2 * RB * 32 * 8;
    static constexpr int kBytes = kVt > kRed ? kVt : kRed;
};

// ---------------------------------------------------------------------------
// Split-KV verify attention, bf16 in, fp32 accumulation.
// grid (split, kv head, request); 256 threads = 4 waves; wave w handles the
// chunk's 32-key tiles w, w+4, ...  Query rows of the group: row = i*G + g
// (position i, head kvh*G + g); RB blocks of 32 rows.
// Writes the chunk's unnormalised O^T (part_o [.][d][row]) and (m, l) per row.
// ---------------------------------------------------------------------------
template <int D, int RB>
__global__ __launch_bounds__(256, RB == 1 ? 2 : 1) void attn_gqa_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ valid,
    float* __restrict__ part_o, float2* __restrict__ part_ml, int NQ, int Hq, int Hkv, int G,
    int R, int max_pages, int chunk, int max_splits, float scale_log2) {
    constexpr int NS = D / 16;   // MFMA k-steps over the head dimension
    constexpr int NDB = D / 32;  // 32-row blocks of O^T
    constexpr int CPL = D / 8;   // 16-byte chunks per key row
    constexpr int NU = D / 16;   // keys per lane when a wave loads a 32-key V tile
    __shared__ __attribute__((aligned(16))) unsigned char smem[GqaSmem<D, RB>::kBytes];

    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    if (!valid[b]) return;
    const int L = seq_lens[b];
    const int Ltot = L + NQ;
    const int start = split * chunk;
    if (start >= Ltot) return;
    const int end = min(start + chunk, Ltot);
    const int ntiles = (end - start + 31) >> 5;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 31, lh = lane >> 5;

    // Q fragments: B operand of S^T = K Q^T (column = query row, k = d).
    u32x4 qf[RB][NS];
    int lim[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = rb * 32 + ln;
        if (row < R) {
            const int i = row / G, g = row - i * G;
            const uint16_t* qp = q + (((size_t)b * NQ + i) * Hq + kvh * G + g) * D + 8 * lh;
#pragma unroll
            for (int s = 0; s < NS; ++s) qf[rb][s] = *(const u32x4*)(qp + 16 * s);
            lim[rb] = L + i;  // causal: keys 0 .. L_b + i
        } else {
#pragma unroll
            for (int s = 0; s < NS; ++s) qf[rb][s] = u32x4{0, 0, 0, 0};
            lim[rb] = Ltot - 1;
        }
    }

    float m_r[RB], l_r[RB];
    f32x16 o[RB][NDB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_r[rb] = -INFINITY;
        l_r[rb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][db][r] = 0.f;
    }

    uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * D * kVtStride;
    const size_t head_elems = (size_t)kPage * D;
    const int vc = lane % CPL, vg = lane / CPL;

    auto tile_base = [&](int t) -> size_t {
        const int ks = start + 32 * t;
        const int pg = page_table[(size_t)b * max_pages + (ks >> 6)];
        return ((size_t)pg * Hkv + kvh) * head_elems + (size_t)(ks & 63) * D;
    };

    u32x4 kf[NS], vf[NU];
    auto load_k = [&](size_t base) {
        const uint16_t* p = k_cache + base + (size_t)ln * D + 8 * lh;
#pragma unroll
        for (int s = 0; s < NS; ++s) kf[s] = *(const u32x4*)(p + 16 * s);
    };
    auto load_v = [&](size_t base) {
        const uint16_t* p = v_cache + base + (size_t)(NU * vg) * D + 8 * vc;
#pragma unroll
        for (int u = 0; u < NU; ++u) vf[u] = *(const u32x4*)(p + (size_t)u * D);
    };

    int t = wave;
    if (t < ntiles) {
        const size_t base = tile_base(t);
        load_k(base);
        load_v(base);
    }
    for (; t < ntiles; t += 4) {
        // V tile -> LDS, transposed: V^T[d][vt_pos(key)].
#pragma unroll
        for (int qd = 0; qd < NU / 4; ++qd) {
            const int pos0 = vt_pos(NU * vg + 4 * qd);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x2 w;
                w.x = half16(vf[4 * qd + 0], e) | (half16(vf[4 * qd + 1], e) << 16);
                w.y = half16(vf[4 * qd + 2], e) | (half16(vf[4 * qd + 3], e) << 16);
                *(u32x2*)(vt + (8 * vc + e) * kVtStride + pos0) = w;
            }
        }
        const bool has_next = t + 4 < ntiles;
        const size_t nbase = has_next ? tile_base(t + 4) : 0;
        if (has_next) load_v(nbase);

        f32x16 sacc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) sacc[rb] = mfma_32x32x16(kf[s], qf[rb][s], sacc[rb]);
        }
        if (has_next) load_k(nbase);

        // Online softmax; lane (ln, lh) holds 16 keys of query row ln.
        const int ks = start + 32 * t;
        u32x4 pb[RB][2], pbl[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float x[16];
            float tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = ks + mfma_row(r, lane);
                float v = sacc[rb][r] * scale_log2;
                if (key >= end || key > lim[rb]) v = -INFINITY;
                x[r] = v;
                tmax = fmaxf(tmax, v);
            }
            tmax = fmaxf(tmax, shfl_xor(tmax, 32));
            const float mnew = fmaxf(m_r[rb], tmax);
            const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = exp2f(m_r[rb] - msafe);
            // P = P_hi + P_lo with both halves in bf16: the PV product runs as
            // two MFMAs, leaving a relative error of about 2^-17 in P.
            float psum = 0.f;
            uint32_t pk[8], pl[8];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = exp2f(x[r] - msafe), p1 = exp2f(x[r + 1] - msafe);
                const uint32_t h0 = f32_to_bf16_rne(p0), h1 = f32_to_bf16_rne(p1);
                const uint32_t l0 = f32_to_bf16_rne(p0 - bf16_to_f32(h0));
                const uint32_t l1 = f32_to_bf16_rne(p1 - bf16_to_f32(h1));
                psum += p0 + p1;
                pk[r >> 1] = h0 | (h1 << 16);
                pl[r >> 1] = l0 | (l1 << 16);
            }
            psum += shfl_xor(psum, 32);
            l_r[rb] = l_r[rb] * alpha + psum;
            m_r[rb] = mnew;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
            pb[rb][0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
            pb[rb][1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
            pbl[rb][0] = u32x4{pl[0], pl[1], pl[2], pl[3]};
            pbl[rb][1] = u32x4{pl[4], pl[5], pl[6], pl[7]};
        }

        wave_lds_sync();
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint16_t* vp = vt + (db * 32 + ln) * kVtStride + 16 * tt + 8 * lh;
                const u32x2 a0 = *(const u32x2*)vp;
                const u32x2 a1 = *(const u32x2*)(vp + 4);
                const u32x4 af = u32x4{a0.x, a0.y, a1.x, a1.y};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    o[rb][db] = mfma_32x32x16(af, pb[rb][tt], o[rb][db]);
                    o[rb][db] = mfma_32x32x16(af, pbl[rb][tt], o[rb][db]);
                }
            }
        }
        wave_lds_sync();
    }

    // Merge the four waves: 2,3 -> 0,1 through LDS, then 1 -> 0.
    float* red_o = reinterpret_cast<float*>(smem);
    float2* red_ml = reinterpret_cast<float2*>(red_o + 2 * RB * 32 * D);
    auto put = [&](int slot) {
        float* ro = red_o + slot * RB * 32 * D;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    ro[(rb * 32 + ln) * D + db * 32 + mfma_row(r, lane)] = o[rb][db][r];
            if (lh == 0) red_ml[slot * RB * 32 + rb * 32 + ln] = make_float2(m_r[rb], l_r[rb]);
        }
    };
    auto merge = [&](int slot) {
        const float* ro = red_o + slot * RB * 32 * D;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float2 oth = red_ml[slot * RB * 32 + rb * 32 + ln];
            const float M = fmaxf(m_r[rb], oth.x);
            const float ws = (m_r[rb] == -INFINITY) ? 0.f : exp2f(m_r[rb] - M);
            const float wo = (oth.x == -INFINITY) ? 0.f : exp2f(oth.x - M);
            l_r[rb] = l_r[rb] * ws + oth.y * wo;
            m_r[rb] = M;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o[rb][db][r] = o[rb][db][r] * ws +
                                   ro[(rb * 32 + ln) * D + db * 32 + mfma_row(r, lane)] * wo;
        }
    };
    __syncthreads();
    if (wave >= 2) put(wave - 2);
    __syncthreads();
    if (wave < 2) merge(wave);
    __syncthreads();
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    merge(0);

    const size_t pidx = ((size_t)b * Hkv + kvh) * max_splits + split;
    float* po = part_o + pidx * D * R;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = rb * 32 + ln;
        if (row >= R) continue;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) po[(size_t)(db * 32 + mfma_row(r, lane)) * R + row] = o[rb][db][r];
        if (lh == 0) part_ml[pidx * R + row] = make_float2(m_r[rb], l_r[rb]);
    }
}

// ---------------------------------------------------------------------------
// Merge of the chunk partials of one (request, kv head): for each row,
// M = max m_s, out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Invalid requests get NaN rows.
// ---------------------------------------------------------------------------
constexpr int kCombineRows = 64;
constexpr int kCombineCache = 8192;

// grid (kv head, request, block of 64 rows).  With `direct_single`, requests
// whose keys fit one chunk were written by the attention kernel already.
__global__ __launch_bounds__(256) void attn_combine(
    const float* __restrict__ part_o, const float2* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ valid,
    float* __restrict__ out, uint16_t* __restrict__ out_lowp, int NQ, int Hq, int Hkv, int G,
    int R, int D, int chunk, int max_splits, int direct_single) {
    __shared__ float s_m[kCombineRows], s_inv[kCombineRows];
    __shared__ float s_w[kCombineCache];
    const int kvh = blockIdx.x, b = blockIdx.y;
    const int r0 = blockIdx.z * kCombineRows;
    const int nr = min(kCombineRows, R - r0);
    if (nr <= 0) return;
    if (!valid[b]) {
        for (int idx = threadIdx.x; idx < nr * D; idx += blockDim.x) {
            const int row = r0 + idx / D, d = idx % D;
            const int i = row / G, g = row - i * G;
            const size_t oi = (((size_t)b * NQ + i) * Hq + kvh * G + g) * D + d;
            out[oi] = NAN;
            if (out_lowp) out_lowp[oi] = 0x7fc0u;
        }
        return;
    }
    const int ns = (seq_lens[b] + NQ + chunk - 1) / chunk;
    if (direct_single && ns == 1) return;
    const size_t pbase = ((size_t)b * Hkv + kvh) * max_splits;
    for (int lr = threadIdx.x; lr < nr; lr += blockDim.x) {
        const int row = r0 + lr;
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[(pbase + s) * R + row].x);
        float den = 0.f;
        for (int s = 0; s < ns; ++s) {
            const float2 ml = part_ml[(pbase + s) * R + row];
            if (ml.x != -INFINITY) den += exp2f(ml.x - M) * ml.y;
        }
        s_m[lr] = M;
        s_inv[lr] = 1.f / den;
    }
    __syncthreads();
    const bool cached = ns * nr <= kCombineCache;
    if (cached) {
        for (int idx = threadIdx.x; idx < ns * nr; idx += blockDim.x) {
            const int s = idx / nr, lr = idx - s * nr;
            const float m = part_ml[(pbase + s) * R + r0 + lr].x;
            s_w[idx] = (m == -INFINITY) ? 0.f : exp2f(m - s_m[lr]) * s_inv[lr];
        }
        __syncthreads();
    }
    for (int idx = threadIdx.x; idx < nr * D; idx += blockDim.x) {
        const int d = idx / nr, lr = idx - d * nr;
        const int row = r0 + lr;
        float acc = 0.f;
        for (int s = 0; s < ns; ++s) {
            float w;
            if (cached) {
                w = s_w[s * nr + lr];
            } else {
                const float m = part_ml[(pbase + s) * R + row].x;
                w = (m == -INFINITY) ? 0.f : exp2f(m - s_m[lr]) * s_inv[lr];
            }
            acc += w * part_o[((pbase + s) * D + d) * R + row];
        }
        const int i = row / G, g = row - i * G;
        const size_t oi = (((size_t)b * NQ + i) * Hq + kvh * G + g) * D + d;
        out[oi] = acc;
        if (out_lowp) out_lowp[oi] = (uint16_t)f32_to_bf16_rne(acc);
    }
}

// ---------------------------------------------------------------------------
// Plain fp32 verify attention: one block per (position i, query head h,
// request).  Keys in tiles of 256 (one score per thread); thread t
// accumulates output element t % D over keys k of the tile with
// k % (256 / D) == t / D.  Used for float32 caches (small problems).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_f32_rows(
    const float* __restrict__ q, const float* __restrict__ k_cache,
    const float* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ valid,
    float* __restrict__ out, float* __restrict__ out_lowp, int NQ, int Hq, int Hkv, int D,
    int max_pages, float scale) {
    __shared__ float s_q[256];
    __shared__ float s_e[256];
    __shared__ float s_red[256];
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const size_t oi = (((size_t)b * NQ + i) * Hq + h) * D;
    if (!valid[b]) {
        for (int d = tid; d < D; d += blockDim.x) {
            out[oi + d] = NAN;
            if (out_lowp) out_lowp[oi + d] = NAN;
        }
        return;
    }
    const int G = Hq / Hkv;
    const int kvh = h / G;
    const int n = seq_lens[b] + i + 1;
    for (int d = tid; d < D; d += blockDim.x) s_q[d] = q[oi + d];
    __syncthreads();
    const int NG = 256 / D;
    const int dd = tid % D, grp = tid / D;
    float m = -INFINITY, l = 0.f, acc = 0.f;
    for (int t0 = 0; t0 < n; t0 += 256) {
        const int p = t0 + tid;
        float s = -INFINITY;
        if (p < n) {
            const int pg = page_table[(size_t)b * max_pages + p / kPage];
            const float* kp = k_cache + (((size_t)pg * Hkv + kvh) * kPage + p % kPage) * D;
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot += s_q[d] * kp[d];
            s = dot * scale;
        }
        s_red[tid] = s;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
            __syncthreads();
        }
        const float mnew = fmaxf(m, s_red[0]);
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
        const float e = (p < n) ? expf(s - mnew) : 0.f;
        __syncthreads();
        s_e[tid] = e;
        s_red[tid] = e;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (tid < w) s_red[tid] += s_red[tid + w];
            __syncthreads();
        }
        l = l * alpha + s_red[0];
        m = mnew;
        acc *= alpha;
        const int cnt = min(256, n - t0);
        for (int k = grp; k < cnt; k += NG) {
            const int pk = t0 + k;
            const int pg = page_table[(size_t)b * max_pages + pk / kPage];
            acc += s_e[k] * v_cache[(((size_t)pg * Hkv + kvh) * kPage + pk % kPage) * D + dd];
        }
        __syncthreads();
    }
    s_red[tid] = acc;
    __syncthreads();
    if (tid < D) {
        float sum = 0.f;
        for (int g = 0; g < NG; ++g) sum += s_red[g * D + tid];
        const float val = sum / l;
        out[oi + tid] = val;
        if (out_lowp) out_lowp[oi + tid] = val;
    }
}

// ---------------------------------------------------------------------------
// Host planning.
// ---------------------------------------------------------------------------
struct AttnPlan {
    int G = 0, R = 0, chunk = 0, max_splits = 0;
    int path = 0;  // 0 gqa bf16 (MFMA), 1 gqa f32, 2 mla bf16
    size_t off_valid = 0, off_po = 0, off_pml = 0, total = 0;
};

int plan_attn(const sd_attn_desc* d, AttnPlan* p) {
    if (!d) return fail(SD_EINVAL, "sd_attn_desc is NULL");
    if (d->batch <= 0 || d->num_q <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 ||
        d->d_qk <= 0 || d->d_v <= 0 || d->max_pages <= 0 || d->num_pages <= 0 ||
        d->max_seq_len < 0)
        return fail(SD_EINVAL, "sd_verify_attn: non-positive size in descriptor");
    if (d->dtype != SD_F32 && d->dtype != SD_BF16)
        return fail(SD_EINVAL, "sd_verify_attn: unknown dtype %d", d->dtype);
    if (d->kind != SD_ATTN_GQA && d->kind != SD_ATTN_MLA)
        return fail(SD_EINVAL, "sd_verify_attn: unknown kind %d", d->kind);
    if (d->n_q_heads % d->n_kv_heads != 0)
        return fail(SD_EINVAL, "sd_verify_attn: n_q_heads %% n_kv_heads != 0");
    if (d->page_size != kPage)
        return fail(SD_EUNSUPPORTED, "sd_verify_attn: page_size must be 64");
    if ((long)d->max_seq_len + d->num_q > (long)d->max_pages * kPage)
        return fail(SD_EINVAL, "sd_verify_attn: max_seq_len + num_q exceeds max_pages * page_size");
    p->G = d->n_q_heads / d->n_kv_heads;
    p->R = p->G * d->num_q;
    const long maxkeys = (long)d->max_seq_len + d->num_q;
    if (d->kind == SD_ATTN_MLA) {
        if (d->dtype != SD_BF16 || d->d_qk != 576 || d->d_v != 512 || d->n_kv_heads != 1)
            return fail(SD_EUNSUPPORTED,
                        "sd_verify_attn: MLA needs bf16, d_qk 576, d_v 512, one kv head");
        p->path = 2;
        p->G = d->n_q_heads;
        p->R = d->n_q_heads * d->num_q;
        const int rc = mla_plan(d->batch, d->num_q, d->n_q_heads, d->max_seq_len, &p->chunk,
                                &p->max_splits);
        if (rc != SD_OK) return rc;
    }
    if (d->kind == SD_ATTN_MLA) {
        // planned above
    } else if (d->d_qk != d->d_v) {
        return fail(SD_EUNSUPPORTED, "sd_verify_attn: GQA needs d_qk == d_v");
    } else if (d->dtype == SD_BF16) {
        if (d->d_qk != 64 && d->d_qk != 128)
            return fail(SD_EUNSUPPORTED, "sd_verify_attn: bf16 GQA needs head dim 64 or 128");
        if (p->R > 64)
            return fail(SD_EUNSUPPORTED, "sd_verify_attn: (Hq/Hkv)*(K+1) = %d > 64", p->R);
        p->path = 0;
        const long pairs = (long)d->batch * d->n_kv_heads;
        int chunk = 1024;
        while (chunk > 128 && pairs * ((maxkeys + chunk - 1) / chunk) < 2048) chunk >>= 1;
        p->chunk = chunk;
        p->max_splits = (int)((maxkeys + chunk - 1) / chunk);
    } else {
        if (d->d_qk > 256 || 256 % d->d_qk != 0)
            return fail(SD_EUNSUPPORTED, "sd_verify_attn: f32 GQA needs head dim dividing 256");
        p->path = 1;
        p->chunk = 0;
        p->max_splits = 0;
    }
    size_t off = 0;
    p->off_valid = off;
    off = align_up(off + sizeof(int32_t) * d->batch, 256);
    p->off_po = off;
    const size_t nparts = (size_t)d->batch * d->n_kv_heads *
                          (p->path == 2 && p->max_splits == 1 ? 0 : p->max_splits) * p->R;
    off = align_up(off + nparts * d->d_v * sizeof(float), 256);
    p->off_pml = off;
    off = align_up(off + nparts * sizeof(float2), 256);
    p->total = off;
    return SD_OK;
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int sd_verify_attn_workspace_size(const sd_attn_desc* d, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(SD_EINVAL, "bytes is NULL");
    AttnPlan p;
    const int rc = plan_attn(d, &p);
    if (rc != SD_OK) return rc;
    *bytes = p.total;
    return SD_OK;
}

extern "C" int sd_verify_attn(const sd_attn_desc* d, void* workspace, size_t ws_bytes,
                              void* stream) {
    clear_error();
    AttnPlan p;
    int rc = plan_attn(d, &p);
    if (rc != SD_OK) return rc;
    if (!d->q || !d->k_cache || !d->page_table || !d->seq_lens || !d->out)
        return fail(SD_EINVAL, "sd_verify_attn: NULL q/k_cache/page_table/seq_lens/out");
    if (d->kind == SD_ATTN_GQA && (!d->v_cache || (d->k_new && !d->v_new)))
        return fail(SD_EINVAL, "sd_verify_attn: GQA needs v_cache (and v_new with k_new)");
    if (d->kind == SD_ATTN_MLA && (d->v_cache || d->v_new))
        return fail(SD_EINVAL, "sd_verify_attn: MLA takes the latent in k_cache/k_new only");
    if (!aligned16(d->q) || !aligned16(d->k_cache) || (d->v_cache && !aligned16(d->v_cache)) ||
        (d->k_new && !aligned16(d->k_new)) || (d->v_new && !aligned16(d->v_new)) ||
        (d->out_lowp && !aligned16(d->out_lowp)) || !aligned16(d->out))
        return fail(SD_EINVAL, "sd_verify_attn: tensor pointers must be 16-byte aligned");
    if (!workspace || !aligned256(workspace))
        return fail(SD_EINVAL, "sd_verify_attn: workspace NULL or not 256-byte aligned");
    if (ws_bytes < p.total)
        return fail(SD_EWORKSPACE, "sd_verify_attn: workspace %zu < %zu bytes", ws_bytes, p.total);
    const int es = d->dtype == SD_BF16 ? 2 : 4;
    if ((d->d_qk * es) % 16 != 0 || (d->d_v * es) % 16 != 0)
        return fail(SD_EUNSUPPORTED, "sd_verify_attn: head rows must be multiples of 16 bytes");

    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    int32_t* valid = (int32_t*)(ws + p.off_valid);
    const int B = d->batch, NQ = d->num_q;
    attn_validate<<<B, 256, 0, s>>>(d->seq_lens, d->page_table, valid, d->dev_error, NQ,
                                    d->max_pages, d->num_pages, d->max_seq_len);
    if ((rc = check_launch("attn_validate")) != SD_OK) return rc;
    if (d->k_new) {
        attn_append<<<dim3(NQ, B), 256, 0, s>>>(
            (const uint8_t*)d->k_new, (const uint8_t*)d->v_new, (uint8_t*)d->k_cache,
            (uint8_t*)d->v_cache, d->page_table, d->seq_lens, valid, NQ, d->n_kv_heads,
            d->d_qk * es, d->d_v * es, d->max_pages, d->kind == SD_ATTN_MLA);
        if ((rc = check_launch("attn_append")) != SD_OK) return rc;
    }
    const float scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.f / sqrtf((float)d->d_qk);
    if (p.path == 1) {
        attn_f32_rows<<<dim3(NQ, d->n_q_heads, B), 256, 0, s>>>(
            (const float*)d->q, (const float*)d->k_cache, (const float*)d->v_cache,
            d->page_table, d->seq_lens, valid, d->out, (float*)d->out_lowp, NQ, d->n_q_heads,
            d->n_kv_heads, d->d_qk, d->max_pages, scale);
        return check_launch("attn_f32_rows");
    }
    float* po = (float*)(ws + p.off_po);
    float2* pml = (float2*)(ws + p.off_pml);
    const float scale_log2 = scale * 1.4426950408889634f;
    if (p.path == 2) {
        if ((rc = mla_launch(d, valid, po, pml, p.chunk, p.max_splits, scale_log2, s)) != SD_OK)
            return rc;
        if (p.max_splits == 1) return SD_OK;
        attn_combine<<<dim3(1, B, (p.R + kCombineRows - 1) / kCombineRows), 256, 0, s>>>(
            po, pml, d->seq_lens, valid, d->out, (uint16_t*)d->out_lowp, NQ, d->n_q_heads, 1,
            p.G, p.R, d->d_v, p.chunk, p.max_splits, 1);
        return check_launch("attn_combine");
    }
    const dim3 grid(p.max_splits, d->n_kv_heads, B);
#define SDV_LAUNCH_GQA(DD, RBB)                                                                  \
    attn_gqa_bf16<DD, RBB><<<grid, 256, 0, s>>>(                                                 \
        (const uint16_t*)d->q, (const uint16_t*)d->k_cache, (const uint16_t*)d->v_cache,         \
        d->page_table, d->seq_lens, valid, po, pml, NQ, d->n_q_heads, d->n_kv_heads, p.G, p.R, \
        d->max_pages, p.chunk, p.max_splits, scale_log2)
    if (d->d_qk == 128) {
        if (p.R <= 32) SDV_LAUNCH_GQA(128, 1); else SDV_LAUNCH_GQA(128, 2);
    } else {
        if (p.R <= 32) SDV_LAUNCH_GQA(64, 1); else SDV_LAUNCH_GQA(64, 2);
    }
#undef SDV_LAUNCH_GQA
    if ((rc = check_launch("attn_gqa_bf16")) != SD_OK) return rc;
    attn_combine<<<dim3(d->n_kv_heads, B, (p.R + kCombineRows - 1) / kCombineRows), 256, 0, s>>>(
        po, pml, d->seq_lens, valid, d->out, (uint16_t*)d->out_lowp, NQ, d->n_q_heads,
        d->n_kv_heads, p.G, p.R, d->d_v, p.chunk, p.max_splits, 0);
    return check_launch("attn_combine");
}
