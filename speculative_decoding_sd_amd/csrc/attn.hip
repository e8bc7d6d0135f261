// Verify attention for speculative decoding on gfx950.
//
// [TRT-MTP] "支持 MTP 的注意力機制": the chain's K+1 tokens need only a causal
// mask in the generation attention; [CSDN-MTP] "整体计算流程" step 2: the
// new queries are batched against the cached keys, softmax(QK^T/sqrt(d))V,
// and each new key/value goes into the cache.
//
// Pipeline on one stream:
//   attn_validate_append  per request: capacity and page-table entries
//                   (flags), then the K+1 new keys/values -> cache positions
//                   L_b .. L_b+K
//   GQA, bf16 q with a bf16 or E4M3 cache:
//                   attn_items (prefix sum of the requests' key tiles) and
//                   attn_gqa_stream (attn_gqa.hip): persistent waves stream
//                   equal ranges of the 32-key tiles of all (kv head,
//                   request) pairs through LDS rings; every query row of the
//                   kv head's group shares each K/V tile, so a tile is read
//                   from HBM exactly once
//   MLA, bf16:      attn_mla_bf16 and its exact fallback (attn_mla.hip)
//   attn_combine    log-sum-exp merge of the chunk partials
// plus attn_f32_rows, a plain fp32 path for small float32 problems.

#include <math.h>

#include <algorithm>

#include "sdv_device.h"
#include "sdv_internal.h"

namespace sdv {
namespace {

constexpr int kPage = 64;

// ---------------------------------------------------------------------------
// Per-request checks and append, one block per (position i, request b).
// Every block of a request takes the same decision; block i = 0 records it.
// Blocks of an invalid request write its NaN output rows.
// valid[b] = 1 when
// 0 <= L_b <= max_seq_len, L_b + NQ <= max_pages * 64 and every page entry
// covering 0 .. L_b+NQ-1 is a pool page.  Later kernels touch only valid
// requests.  Then (k_new given) row i of k_new / v_new goes to position
// L_b + i with 16-byte copies; MLA copies the latent row into k_cache only.
// With an E4M3 cache (k_scale given) each bf16 element is stored as the code
// nearest to value / scale[kv head] instead, eight elements per thread.
// ---------------------------------------------------------------------------

// E4M3 ("fn") code of y: round to nearest, ties to even, magnitudes at or
// above 448 (infinities included) saturate to 448, NaN -> 0x7F.  Normal
// range: the float's exponent and top three mantissa bits, rounded on the
// 20 bits dropped (a carry moves into the exponent); below 2^-6 the codes
// are the multiples of 2^-9, code 8 being 2^-6 itself.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;
    const float m = __uint_as_float(a);
    if (m >= 448.f) return sign | 0x7eu;
    if (m < 0.015625f) return sign | (uint32_t)__builtin_rintf(m * 512.f);
    return sign | (((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3));
}

// Eight bf16 (one 16-byte load) -> eight codes of value / s (8 bytes).
__device__ __forceinline__ u32x2 e4m3_pack8(u32x4 src, float s) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t h = (src[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        w[e >> 2] |= e4m3_code(bf16_to_f32(h) / s) << (8 * (e & 3));
    }
    return u32x2{w[0], w[1]};
}

__global__ void attn_validate_append(const int32_t* __restrict__ seq_lens,
                                     const int32_t* __restrict__ page_table,
                                     int32_t* __restrict__ valid, int32_t* err,
                                     const uint8_t* __restrict__ k_new,
                                     const uint8_t* __restrict__ v_new,
                                     uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                     int NQ, int Hkv, int row_bytes_k, int row_bytes_v,
                                     int max_pages, int num_pages, int max_seq_len, int mla,
                                     float* __restrict__ out, void* __restrict__ out_lowp,
                                     int lowp_f32, int Hq, int Dv,
                                     const float* __restrict__ k_scale,
                                     const float* __restrict__ v_scale,
                                     const int32_t* __restrict__ tree_parent,
                                     uint64_t* __restrict__ anc) {
    const int i = blockIdx.x, b = blockIdx.y;
    const int L = seq_lens[b];
    const bool cap_ok =
        L >= 0 && L <= max_seq_len && (long)L + NQ <= (long)max_pages * kPage;
    int bad_page = 0, bad_tree = 0;
    if (cap_ok) {
        const int npg = (L + NQ + kPage - 1) / kPage;
        for (int lp = threadIdx.x; lp < npg; lp += blockDim.x) {
            const int pg = page_table[(size_t)b * max_pages + lp];
            if (pg < 0 || pg >= num_pages) bad_page = 1;
        }
    }
    if (tree_parent)
        for (int a = threadIdx.x; a < NQ; a += blockDim.x) {
            const int p = tree_parent[(size_t)b * NQ + a];
            if (a == 0 ? p != -1 : (p < 0 || p >= a)) bad_tree = 1;
        }
    bad_page = __syncthreads_or(bad_page);
    bad_tree = __syncthreads_or(bad_tree);
    const bool ok = cap_ok && !bad_page && !bad_tree;
    if (threadIdx.x == 0 && i == 0) {
        valid[b] = ok ? 1 : 0;
        if (!cap_ok) set_error(err, SD_DERR_CAPACITY);
        if (bad_page) set_error(err, SD_DERR_PAGE);
        if (bad_tree) set_error(err, SD_DERR_TREE);
    }
    if (tree_parent && ok && threadIdx.x == 0) {
        // Node i's mask: bit a set for a = i and every ancestor of i (the walk
        // ends because parents decrease).
        uint64_t m = 0;
        for (int a = i; a >= 0; a = tree_parent[(size_t)b * NQ + a]) m |= 1ull << a;
        anc[(size_t)b * NQ + i] = m;
    }
    if (!ok) {
        // Invalid request: NaN output rows (the attention kernels skip it).
        const size_t o0 = ((size_t)b * NQ + i) * Hq * Dv;
        for (int e = threadIdx.x; e < Hq * Dv; e += blockDim.x) {
            out[o0 + e] = NAN;
            if (out_lowp) {
                if (lowp_f32) ((float*)out_lowp)[o0 + e] = NAN;
                else ((uint16_t*)out_lowp)[o0 + e] = 0x7fc0u;
            }
        }
        return;
    }
    if (!k_new) return;
    const int nk = row_bytes_k / 16, nv = row_bytes_v / 16;
    {
        const long pos = (long)L + i;
        const long pg = page_table[(size_t)b * max_pages + pos / kPage];
        const long off = pos % kPage;
        if (k_scale) {
            // E4M3 cache: row_bytes_* are the cache rows (one byte per
            // element); the new rows are bf16, twice as long.
            const int n8k = row_bytes_k / 8, n8v = row_bytes_v / 8;
            for (int idx = threadIdx.x; idx < Hkv * n8k; idx += blockDim.x) {
                const int h = idx / n8k, c = idx - h * n8k;
                const u32x4 src = ((const u32x4*)(k_new + (((size_t)b * NQ + i) * Hkv + h) *
                                                              2 * row_bytes_k))[c];
                ((u32x2*)(k_cache + (((size_t)pg * Hkv + h) * kPage + off) * row_bytes_k))[c] =
                    e4m3_pack8(src, k_scale[h]);
            }
            for (int idx = threadIdx.x; idx < Hkv * n8v; idx += blockDim.x) {
                const int h = idx / n8v, c = idx - h * n8v;
                const u32x4 src = ((const u32x4*)(v_new + (((size_t)b * NQ + i) * Hkv + h) *
                                                              2 * row_bytes_v))[c];
                ((u32x2*)(v_cache + (((size_t)pg * Hkv + h) * kPage + off) * row_bytes_v))[c] =
                    e4m3_pack8(src, v_scale[h]);
            }
            return;
        }
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
            u32x4* dst =
                (u32x4*)(k_cache + (((size_t)pg * Hkv + h) * kPage + off) * row_bytes_k) + c;
            *dst = *src;
        }
        for (int idx = threadIdx.x; idx < Hkv * nv; idx += blockDim.x) {
            const int h = idx / nv, c = idx - h * nv;
            const u32x4* src =
                (const u32x4*)(v_new + (((size_t)b * NQ + i) * Hkv + h) * row_bytes_v) + c;
            u32x4* dst =
                (u32x4*)(v_cache + (((size_t)pg * Hkv + h) * kPage + off) * row_bytes_v) + c;
            *dst = *src;
        }
    }
}

// ---------------------------------------------------------------------------
// Merge of the chunk partials of one (request, kv head): for each row,
// M = max m_s, out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Invalid requests get NaN rows.
// ---------------------------------------------------------------------------
constexpr int kCombineRows = 64;
constexpr int kCombineCache = 12288;  // split weights cached per block (48 KiB)

// grid (kv head, request, 64-row block x dsplit): block z covers rows
// 64 (z / dsplit) .. +63 and the head dims D/dsplit * (z % dsplit) .. of
// them (the split gives small batches of long requests enough blocks; every
// block computes its rows' weights itself).
// mode 1 (MLA): slot k of request b is its key chunk k; requests whose keys
//   fit one chunk were written by the attention kernel already.
// mode 2 (GQA): n = min(nw, T) of the streaming kernel's nw waves split the
//   T = first[B] * Hkv tiles evenly, wave w < n taking [floor(w T / n),
//   floor((w+1) T / n)); a
//   pair whose tiles lie in one wave was written by that wave, otherwise its
//   waves w_lo .. w_hi each left one partial: wave w_lo in slot 2 w_lo + 1
//   (2 w_lo if its range starts at the pair's first tile), the others in
//   slot 2w.  Slots are merged in key order.
// Each block weighs its rows' partials once (weights cached in LDS when they
// fit), then reads the partial planes [d][R] with consecutive threads on
// consecutive rows.
__global__ __launch_bounds__(256) void attn_combine(
    const float* __restrict__ part_o, const float2* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ valid,
    const int32_t* __restrict__ first, float* __restrict__ out, uint16_t* __restrict__ out_lowp,
    int NQ, int Hq, int Hkv, int G, int R, int D, int chunk, int max_splits, int nw, int mode,
    int dsplit) {
    __shared__ float s_m[kCombineRows], s_inv[kCombineRows];
    __shared__ float s_red[4][kCombineRows];
    __shared__ __attribute__((aligned(16))) float s_w[kCombineCache];
    const int kvh = blockIdx.x, b = blockIdx.y;
    const int r0 = (blockIdx.z / dsplit) * kCombineRows;
    const int Dc = D / dsplit, d0 = Dc * (blockIdx.z % dsplit);
    const int nr = min(kCombineRows, R - r0);
    if (nr <= 0) return;
    if (!valid[b]) {
        for (int idx = threadIdx.x; idx < nr * Dc; idx += blockDim.x) {
            const int row = r0 + idx % nr, d = d0 + idx / nr;
            const int i = row / G, g = row - i * G;
            const size_t oi = (((size_t)b * NQ + i) * Hq + kvh * G + g) * D + d;
            out[oi] = NAN;
            if (out_lowp) out_lowp[oi] = 0x7fc0u;
        }
        return;
    }
    // Slot k (k < np) holds the k-th partial of this pair in key order.
    long slot0, slot_step;
    int np;
    if (mode == 1) {
        np = (seq_lens[b] + NQ + chunk - 1) / chunk;
        if (np == 1) return;
        slot0 = ((long)b * Hkv + kvh) * max_splits;
        slot_step = 1;
    } else {
        const long Th = first[gridDim.y], T = Th * Hkv;
        const long n = min((long)nw, T);  // waves in use
        const long g0 = (long)kvh * Th + first[b], g1 = g0 + (first[b + 1] - first[b]) - 1;
        // wave of tile x: the largest w with floor(w T / n) <= x
        const int w_lo = (int)(((g0 + 1) * n + T - 1) / T) - 1;
        const int w_hi = (int)(((g1 + 1) * n + T - 1) / T) - 1;
        if (w_lo == w_hi) return;
        np = w_hi - w_lo + 1;
        slot0 = 2L * w_lo + ((long)w_lo * T / n < g0 ? 1 : 0);
        slot_step = 2;
    }
    auto slot = [&](int k) -> long {
        return k == 0 ? slot0 : (mode == 1 ? slot0 + k : slot0 - (slot0 & 1) + slot_step * k);
    };
    // Row statistics: four threads per row, each over every fourth slot,
    // merged in a fixed order.
    const int lr4 = threadIdx.x % kCombineRows, q4 = threadIdx.x / kCombineRows;
    {
        float M = -INFINITY;
        if (lr4 < nr)
            for (int k = q4; k < np; k += 4)
                M = fmaxf(M, part_ml[slot(k) * R + r0 + lr4].x);
        s_red[q4][lr4] = M;
    }
    __syncthreads();
    if (threadIdx.x < nr)
        s_m[threadIdx.x] = fmaxf(fmaxf(s_red[0][threadIdx.x], s_red[1][threadIdx.x]),
                                 fmaxf(s_red[2][threadIdx.x], s_red[3][threadIdx.x]));
    __syncthreads();
    {
        float den = 0.f;
        if (lr4 < nr) {
            const float M = s_m[lr4];
            for (int k = q4; k < np; k += 4) {
                const float2 ml = part_ml[slot(k) * R + r0 + lr4];
                if (ml.x != -INFINITY) den += exp2f(ml.x - M) * ml.y;
            }
        }
        s_red[q4][lr4] = den;
    }
    __syncthreads();
    if (threadIdx.x < nr)
        s_inv[threadIdx.x] = 1.f / ((s_red[0][threadIdx.x] + s_red[1][threadIdx.x]) +
                                    (s_red[2][threadIdx.x] + s_red[3][threadIdx.x]));
    __syncthreads();
    const bool cached = np * nr <= kCombineCache;
    if (cached) {
        for (int idx = threadIdx.x; idx < np * nr; idx += blockDim.x) {
            const int k = idx / nr, lr = idx - k * nr;
            const float m = part_ml[slot(k) * R + r0 + lr].x;
            s_w[idx] = (m == -INFINITY) ? 0.f : exp2f(m - s_m[lr]) * s_inv[lr];
        }
        __syncthreads();
    }
    const size_t sstride = (size_t)D * R;
    auto emit = [&](int row, int d, float acc) {
        const int i = row / G, g = row - i * G;
        const size_t oi = (((size_t)b * NQ + i) * Hq + kvh * G + g) * D + d;
        out[oi] = acc;
        if (out_lowp) out_lowp[oi] = (uint16_t)f32_to_bf16_rne(acc);
    };
    if (cached && (R & 3) == 0 && (nr & 3) == 0) {
        // Four consecutive rows per thread (16-byte loads), eight slots in
        // flight per step.
        const int nq = nr >> 2;
        for (int idx = threadIdx.x; idx < nq * Dc; idx += blockDim.x) {
            const int dl = d0 + idx / nq, lq = 4 * (idx % nq);
            const float* po = part_o + (size_t)dl * R + r0 + lq;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            int k = 0;
            for (; k + 8 <= np; k += 8) {
                f32x4 v[8], w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = *(const f32x4*)(po + slot(k + u) * sstride);
#pragma unroll
                for (int u = 0; u < 8; ++u) w[u] = *(const f32x4*)(s_w + (k + u) * nr + lq);
#pragma unroll
                for (int u = 0; u < 8; ++u) acc += w[u] * v[u];
            }
            for (; k < np; ++k)
                acc += *(const f32x4*)(s_w + k * nr + lq) * *(const f32x4*)(po + slot(k) * sstride);
#pragma unroll
            for (int j = 0; j < 4; ++j) emit(r0 + lq + j, dl, acc[j]);
        }
        return;
    }
    for (int idx = threadIdx.x; idx < nr * Dc; idx += blockDim.x) {
        const int lr = idx % nr;
        const int row = r0 + lr, d = d0 + idx / nr;
        const float* po = part_o + (size_t)d * R + row;
        float acc = 0.f;
        for (int k = 0; k < np; ++k) {
            float w;
            if (cached) {
                w = s_w[k * nr + lr];
            } else {
                const float m = part_ml[slot(k) * R + row].x;
                w = (m == -INFINITY) ? 0.f : exp2f(m - s_m[lr]) * s_inv[lr];
            }
            acc += w * po[slot(k) * sstride];
        }
        emit(row, d, acc);
    }
}

// Head-dim split of the combine: doubled while the blocks number fewer than
// two per CU, keeping at least 32 dims per block.
static int combine_dsplit(int blocks, int D, int* ds) {
    int cus = 0;
    const int rc = cu_count("sd_verify_attn", &cus);
    if (rc != SD_OK) return rc;
    *ds = 1;
    while (D % (*ds * 2) == 0 && D / (*ds * 2) >= 32 && (long)blocks * *ds < 2L * cus) *ds *= 2;
    return SD_OK;
}

// ---------------------------------------------------------------------------
// Plain fp32 verify attention: one block per (position i, query head h,
// request), 256 threads.  Keys in tiles of 256 (one score per thread, the
// key row read VW floats at a time: head rows are whole 16-byte units, so
// VW = 4); the tile's max and sum by wave
// reductions and one exchange of the four waves' results.  Values: D / VW
// threads cover one value row (VW dims each), so 256 VW / D groups of
// threads take keys k % groups = group, every load of a thread's keys in
// flight at once (up to 16); the groups' partial sums are added in group
// order at the end.  Used for float32 caches (small problems, latency-bound).
// ---------------------------------------------------------------------------
template <int VW>
__global__ __launch_bounds__(256) void attn_f32_rows(
    const float* __restrict__ q, const float* __restrict__ k_cache,
    const float* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ valid,
    float* __restrict__ out, float* __restrict__ out_lowp, int NQ, int Hq, int Hkv, int D,
    int max_pages, float scale, const uint64_t* __restrict__ anc) {
    typedef float vec_t __attribute__((ext_vector_type(VW)));
    constexpr int kMaxLoads = 16;  // value loads in flight per thread
    __shared__ float s_q[256];
    __shared__ float s_e[256];
    __shared__ float s_red[256 * VW];
    __shared__ float s_w[2][4];
    __shared__ int s_pg[256 / kPage];  // the tile's physical pages
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6;
    const size_t oi = (((size_t)b * NQ + i) * Hq + h) * D;
    // The request's scalars, its query element and its first page-table
    // entries are all loaded before any of them is waited for (D <= 256).
    const int ok = valid[b];
    const int L = seq_lens[b];
    const uint64_t vis = anc ? anc[(size_t)b * NQ + i] : ~0ull;  // new keys visible to node i
    const float qv = tid < D ? q[oi + tid] : 0.f;
    const int n = L + i + 1;
    int pg0 = 0;
    if (ok && tid < 256 / kPage && kPage * tid < n)
        pg0 = page_table[(size_t)b * max_pages + tid];
    if (!ok) {
        for (int d = tid; d < D; d += blockDim.x) {
            out[oi + d] = NAN;
            if (out_lowp) out_lowp[oi + d] = NAN;
        }
        return;
    }
    const int G = Hq / Hkv;
    const int kvh = h / G;
    if (tid < D) s_q[tid] = qv;
    const int row_lanes = D / VW;   // threads per value row
    const int NG = 256 / row_lanes;  // key groups
    const int dv = (tid % row_lanes) * VW, grp = tid / row_lanes;
    float m = -INFINITY, l = 0.f;
    vec_t acc = {};
    for (int t0 = 0; t0 < n; t0 += 256) {
        // The tile's page-table entries, read once (they are the only
        // dependent loads in front of the key and value reads).
        if (tid < 256 / kPage && t0 + kPage * tid < n)
            s_pg[tid] = t0 == 0 ? pg0 : page_table[(size_t)b * max_pages + t0 / kPage + tid];
        __syncthreads();
        const int p = t0 + tid;
        float s = -INFINITY;
        if (p < n && (p < L || ((vis >> (p - L)) & 1ull))) {
            const int pg = s_pg[tid / kPage];
            const float* kp = k_cache + (((size_t)pg * Hkv + kvh) * kPage + p % kPage) * D;
            // The row in batches of 16 vector loads, all in flight before the
            // products (summed over the dims in order).
            float dot = 0.f;
            for (int d0 = 0; d0 < D; d0 += 16 * VW) {
                vec_t kv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (d0 + u * VW < D) kv[u] = *(const vec_t*)(kp + d0 + u * VW);
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (d0 + u * VW < D)
#pragma unroll
                        for (int e = 0; e < VW; ++e) dot += s_q[d0 + u * VW + e] * kv[u][e];
            }
            s = dot * scale;
        }
        float wm = s;
#pragma unroll
        for (int mk = 32; mk >= 1; mk >>= 1) wm = fmaxf(wm, shfl_xor(wm, mk));
        if ((tid & 63) == 0) s_w[0][wave] = wm;
        __syncthreads();
        const float tmax = fmaxf(fmaxf(s_w[0][0], s_w[0][1]), fmaxf(s_w[0][2], s_w[0][3]));
        const float mnew = fmaxf(m, tmax);
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
        const float e = (s != -INFINITY) ? expf(s - mnew) : 0.f;
        s_e[tid] = e;
        float ws = e;
#pragma unroll
        for (int mk = 32; mk >= 1; mk >>= 1) ws += shfl_xor(ws, mk);
        if ((tid & 63) == 0) s_w[1][wave] = ws;
        __syncthreads();
        l = l * alpha + (((s_w[1][0] + s_w[1][1]) + s_w[1][2]) + s_w[1][3]);
        m = mnew;
        acc *= alpha;
        // Values of this thread's keys (k = grp, grp + NG, ...), all loads of a
        // batch in flight, then summed over the keys in order.
        const int cnt = min(256, n - t0);
        for (int k0 = grp; k0 < cnt; k0 += kMaxLoads * NG) {
            vec_t v[kMaxLoads];
#pragma unroll
            for (int u = 0; u < kMaxLoads; ++u) {
                const int kk = k0 + u * NG;
                if (kk < cnt)
                    v[u] = *(const vec_t*)(v_cache +
                                           (((size_t)s_pg[kk / kPage] * Hkv + kvh) * kPage +
                                            kk % kPage) * D + dv);
            }
#pragma unroll
            for (int u = 0; u < kMaxLoads; ++u) {
                const int kk = k0 + u * NG;
                if (kk < cnt) acc += s_e[kk] * v[u];
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < VW; ++u) s_red[grp * D + dv + u] = acc[u];
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
    int max_waves = 0;  // GQA streaming kernel: waves sized for (two slots each)
    int path = 0;  // 0 gqa bf16 (MFMA), 1 gqa f32, 2 mla bf16
    size_t off_valid = 0, off_first = 0, off_flags = 0, off_anc = 0, off_po = 0, off_pml = 0,
           total = 0;
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
    if (d->kv_format != SD_KV_AS_DTYPE && d->kv_format != SD_KV_E4M3)
        return fail(SD_EINVAL, "sd_verify_attn: unknown kv_format %d", d->kv_format);
    if (d->kv_format == SD_KV_E4M3 &&
        (d->kind != SD_ATTN_GQA || d->dtype != SD_BF16))
        return fail(SD_EUNSUPPORTED, "sd_verify_attn: an E4M3 cache needs GQA with bf16 q");
    if (d->tree_parent && (d->kind != SD_ATTN_GQA || d->num_q > 64))
        return fail(SD_EUNSUPPORTED, "sd_verify_attn: a draft tree needs GQA and K+1 <= 64");
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
        if (p->max_splits > kCombineMaxSplits)
            return fail(SD_EUNSUPPORTED, "sd_verify_attn: more than %d key chunks per request",
                        kCombineMaxSplits);
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
        // No more waves than 4-wave groups of tiles at the longest length.
        const long max_tiles = (long)d->batch * d->n_kv_heads * ((maxkeys + 31) / 32);
        if (max_tiles > 0x7fffffffL / 4)
            return fail(SD_EUNSUPPORTED, "sd_verify_attn: too many key tiles");
        p->max_waves = (int)std::min<long>(kGqaMaxWaves, 4 * ((max_tiles + 3) / 4));
        if (p->max_waves + 1 > kCombineMaxSplits)
            return fail(SD_EUNSUPPORTED, "sd_verify_attn: too many waves for the combine");
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
    p->off_first = off;
    off = align_up(off + sizeof(int32_t) * (d->batch + 1), 256);
    p->off_anc = off;
    off = align_up(off + sizeof(uint64_t) * (size_t)d->batch * d->num_q, 256);
    p->off_flags = off;
    if (p->path == 2)
        off = align_up(off + sizeof(int32_t) *
                                 mla_flag_count(d->batch, d->num_q, d->n_q_heads, p->max_splits),
                       256);
    p->off_po = off;
    const size_t nparts =
        (p->path == 0 ? 2 * (size_t)p->max_waves
                      : (size_t)d->batch * d->n_kv_heads *
                            (p->path == 2 && p->max_splits == 1 ? 0 : p->max_splits)) *
        p->R;
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
    const bool fp8 = d->kv_format == SD_KV_E4M3;
    if (fp8 && (!d->k_scale || !d->v_scale))
        return fail(SD_EINVAL, "sd_verify_attn: an E4M3 cache needs k_scale and v_scale");
    if (!aligned16(d->q) || !aligned16(d->k_cache) || (d->v_cache && !aligned16(d->v_cache)) ||
        (d->k_new && !aligned16(d->k_new)) || (d->v_new && !aligned16(d->v_new)) ||
        (d->out_lowp && !aligned16(d->out_lowp)) || !aligned16(d->out))
        return fail(SD_EINVAL, "sd_verify_attn: tensor pointers must be 16-byte aligned");
    if (!workspace || !aligned256(workspace))
        return fail(SD_EINVAL, "sd_verify_attn: workspace NULL or not 256-byte aligned");
    if (ws_bytes < p.total)
        return fail(SD_EWORKSPACE, "sd_verify_attn: workspace %zu < %zu bytes", ws_bytes, p.total);
    const int es = fp8 ? 1 : d->dtype == SD_BF16 ? 2 : 4;  // cache element bytes
    if ((d->d_qk * es) % 16 != 0 || (d->d_v * es) % 16 != 0)
        return fail(SD_EUNSUPPORTED, "sd_verify_attn: head rows must be multiples of 16 bytes");

    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    int32_t* valid = (int32_t*)(ws + p.off_valid);
    uint64_t* anc = (uint64_t*)(ws + p.off_anc);
    const int B = d->batch, NQ = d->num_q;
    attn_validate_append<<<dim3(NQ, B), 256, 0, s>>>(
        d->seq_lens, d->page_table, valid, d->dev_error, (const uint8_t*)d->k_new,
        (const uint8_t*)d->v_new, (uint8_t*)d->k_cache, (uint8_t*)d->v_cache, NQ, d->n_kv_heads,
        d->d_qk * es, d->d_v * es, d->max_pages, d->num_pages, d->max_seq_len,
        d->kind == SD_ATTN_MLA, d->out, d->out_lowp, p.path == 1, d->n_q_heads, d->d_v,
        fp8 ? d->k_scale : nullptr, fp8 ? d->v_scale : nullptr, d->tree_parent, anc);
    if ((rc = check_launch("attn_validate_append")) != SD_OK) return rc;
    const float scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.f / sqrtf((float)d->d_qk);
    if (p.path == 1) {
        // Head rows are whole 16-byte units (checked above) in 16-byte aligned
        // caches: rows are read four floats at a time.
        attn_f32_rows<4><<<dim3(NQ, d->n_q_heads, B), 256, 0, s>>>(
            (const float*)d->q, (const float*)d->k_cache, (const float*)d->v_cache,
            d->page_table, d->seq_lens, valid, d->out, (float*)d->out_lowp, NQ, d->n_q_heads,
            d->n_kv_heads, d->d_qk, d->max_pages, scale, d->tree_parent ? anc : nullptr);
        return check_launch("attn_f32_rows");
    }
    float* po = (float*)(ws + p.off_po);
    float2* pml = (float2*)(ws + p.off_pml);
    const float scale_log2 = scale * 1.4426950408889634f;
    if (p.path == 2) {
        int32_t* flags = (int32_t*)(ws + p.off_flags);
        if ((rc = mla_launch(d, valid, flags, po, pml, p.chunk, p.max_splits, scale, s)) != SD_OK)
            return rc;
        if (p.max_splits == 1) return SD_OK;
        const int rblocks = (p.R + kCombineRows - 1) / kCombineRows;
        int ds = 1;
        if ((rc = combine_dsplit(B * rblocks, d->d_v, &ds)) != SD_OK) return rc;
        attn_combine<<<dim3(1, B, rblocks * ds), 256, 0, s>>>(
            po, pml, d->seq_lens, valid, nullptr, d->out, (uint16_t*)d->out_lowp, NQ,
            d->n_q_heads, 1, p.G, p.R, d->d_v, p.chunk, p.max_splits, 0, 1, ds);
        return check_launch("attn_combine");
    }
    int32_t* first = (int32_t*)(ws + p.off_first);
    int nw = 0;
    if ((rc = gqa_launch(d, valid, first, d->tree_parent ? anc : nullptr, po, pml, p.R,
                         p.max_waves, scale_log2, &nw, s)) != SD_OK)
        return rc;
    const int rblocks = (p.R + kCombineRows - 1) / kCombineRows;
    int ds = 1;
    if ((rc = combine_dsplit(d->n_kv_heads * B * rblocks, d->d_v, &ds)) != SD_OK) return rc;
    attn_combine<<<dim3(d->n_kv_heads, B, rblocks * ds), 256, 0, s>>>(
        po, pml, d->seq_lens, valid, first, d->out, (uint16_t*)d->out_lowp, NQ, d->n_q_heads,
        d->n_kv_heads, p.G, p.R, d->d_v, 0, 0, nw, 2, ds);
    return check_launch("attn_combine");
}
