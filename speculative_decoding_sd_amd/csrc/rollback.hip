// KV rollback on gfx950.
//
// [TRT-MTP] "MTP Vanilla" / "MTP Eagle": after verification the keys and
// values of the discarded drafts are removed from the cache; "基本實現方式"
// Fig. 4: this runs after the engine forward.  [CSDN-MTP] "回滚机制": the
// verified prefix is kept, nothing is recomputed.
//
// rollback_compact (one block): per request new_len = L_b + j_b + 1 (or L_b
// for an invalid j_b); an exclusive scan over requests gives the offsets of
// the compacted rejected-slot and freed-page lists; seq_lens is advanced.
// rollback_poison (optional): zeroes the rejected slots of the caches.
// rollback_gather (a tree of drafts, before the other two): moves the
// accepted path's rows to contiguous positions.
#include "sdv_device.h"
#include "sdv_internal.h"

namespace sdv {
namespace {

__device__ __forceinline__ int block_exclusive_scan_1024(int x, int* s_w, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int pre = 0, tot = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave) pre += s_w[w];
        tot += s_w[w];
    }
    __syncthreads();
    *total = tot;
    return pre + incl - x;
}

// A tree's accepted path (node indices 0, then j increasing, at most K):
// whether it is well formed.
__device__ __forceinline__ bool path_ok(const int32_t* __restrict__ path, int j, int K) {
    if (path[0] != 0) return false;
    for (int t = 1; t <= j; ++t)
        if (path[t] <= path[t - 1] || path[t] > K) return false;
    return true;
}

__global__ __launch_bounds__(1024) void rollback_compact(
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ num_accepted,
    int32_t* __restrict__ seq_lens, int32_t* __restrict__ slots, int32_t* __restrict__ slot_off,
    int32_t* __restrict__ freed, int32_t* __restrict__ freed_off, int32_t* err, int B, int K,
    int ps, int max_pages, const int32_t* __restrict__ accepted_nodes) {
    __shared__ int s_w[16];
    int carry_s = 0, carry_f = 0;
    const int tid = threadIdx.x;
    for (int base = 0; base < B; base += 1024) {
        const int b = base + tid;
        int ns = 0, nf = 0;
        long L = 0, new_len = 0, first_free = 0, first_touch = 0;
        if (b < B) {
            L = seq_lens[b];
            int j = num_accepted[b];
            if (j > K) set_error(err, SD_DERR_ACCEPT_COUNT);
            if (accepted_nodes && j >= 0 && j <= K &&
                !path_ok(accepted_nodes + (size_t)b * (K + 1), j, K)) {
                set_error(err, SD_DERR_TREE);
                j = -1;
            }
            new_len = (j < 0 || j > K) ? L : L + j + 1;
            ns = (int)(L + K + 1 - new_len);
            first_free = (new_len + ps - 1) / ps;
            first_touch = L / ps;
            const long last_touch = (L + K) / ps;
            const long f0 = first_free > first_touch ? first_free : first_touch;
            nf = last_touch >= f0 ? (int)(last_touch - f0 + 1) : 0;
            if (L < 0 || (L + K) / ps >= max_pages) {  // table cannot hold the step
                set_error(err, SD_DERR_CAPACITY);
                ns = 0;
                nf = 0;
            }
        }
        int tot_s, tot_f;
        const int off_s = carry_s + block_exclusive_scan_1024(ns, s_w, &tot_s);
        const int off_f = carry_f + block_exclusive_scan_1024(nf, s_w, &tot_f);
        if (b < B) {
            slot_off[b] = off_s;
            freed_off[b] = off_f;
            const int32_t* row = page_table + (size_t)b * max_pages;
            for (int k = 0; k < ns; ++k) {
                const long p = new_len + k;
                slots[off_s + k] = (int32_t)((long)row[p / ps] * ps + p % ps);
            }
            const long f0 = first_free > first_touch ? first_free : first_touch;
            for (int k = 0; k < nf; ++k) freed[off_f + k] = row[f0 + k];
            if (L >= 0) seq_lens[b] = (int32_t)new_len;
        }
        carry_s += tot_s;
        carry_f += tot_f;
    }
    if (tid == 0) {
        slot_off[B] = carry_s;
        freed_off[B] = carry_f;
    }
    for (int k = carry_s + tid; k < B * (K + 1); k += blockDim.x) slots[k] = -1;
    const int fcap = B * (K / ps + 2);
    for (int k = carry_f + tid; k < fcap; k += blockDim.x) freed[k] = -1;
}

// Tree of drafts: node a of request b sits at position L_b + a; the kept
// path's rows move to L_b + t for t = 1 .. j_b.  Block (b, h) copies kv head
// h (the latent row for MLA); each thread owns the same 16-byte chunks at
// every step, so when a step's destination is an earlier step's source that
// thread read it first, in program order.  Reads seq_lens before
// rollback_compact advances it; skips requests whose count or path the
// compaction rejects, and rows whose page entry is outside the pool.
__global__ __launch_bounds__(256) void rollback_gather(
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ num_accepted,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ accepted_nodes,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, int K, int ps, int max_pages,
    int num_pages, int Hkv, int row_bytes_k, int row_bytes_v, int mla) {
    const int b = blockIdx.x, h = blockIdx.y;
    const long L = seq_lens[b];
    const int j = num_accepted[b];
    if (j < 1 || j > K || L < 0 || (L + K) / ps >= max_pages) return;
    const int32_t* path = accepted_nodes + (size_t)b * (K + 1);
    if (!path_ok(path, j, K)) return;
    const int32_t* row = page_table + (size_t)b * max_pages;
    const int nk = row_bytes_k / 16, nv = mla ? 0 : row_bytes_v / 16;
    for (int t = 1; t <= j; ++t) {
        const int a = path[t];
        if (a == t) continue;
        const long ps_ = L + a, pd = L + t;
        const long gs = row[ps_ / ps], gd = row[pd / ps];
        if (gs < 0 || gs >= num_pages || gd < 0 || gd >= num_pages) continue;
        const long os = ps_ % ps, od = pd % ps;
        const size_t rs = mla ? (size_t)gs * ps + os : ((size_t)gs * Hkv + h) * ps + os;
        const size_t rd = mla ? (size_t)gd * ps + od : ((size_t)gd * Hkv + h) * ps + od;
        for (int c = threadIdx.x; c < nk; c += blockDim.x)
            ((u32x4*)(k_cache + rd * row_bytes_k))[c] = ((const u32x4*)(k_cache + rs * row_bytes_k))[c];
        for (int c = threadIdx.x; c < nv; c += blockDim.x)
            ((u32x4*)(v_cache + rd * row_bytes_v))[c] = ((const u32x4*)(v_cache + rs * row_bytes_v))[c];
    }
}

// Zeroes rejected slot k of request b (all kv heads; the latent row for MLA).
__global__ __launch_bounds__(256) void rollback_poison(
    const int32_t* __restrict__ slots, const int32_t* __restrict__ slot_off,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, int ps, int num_pages, int Hkv,
    int row_bytes_k, int row_bytes_v, int mla) {
    const int b = blockIdx.x, k = blockIdx.y;
    const int beg = slot_off[b], cnt = slot_off[b + 1] - beg;
    if (k >= cnt) return;
    const int slot = slots[beg + k];
    if (slot < 0) return;
    const long pg = slot / ps, off = slot % ps;
    if (pg >= num_pages) return;
    const u32x4 z = u32x4{0, 0, 0, 0};
    if (mla) {
        u32x4* dst = (u32x4*)(k_cache + ((size_t)pg * ps + off) * row_bytes_k);
        for (int c = threadIdx.x; c < row_bytes_k / 16; c += blockDim.x) dst[c] = z;
        return;
    }
    const int nk = row_bytes_k / 16, nv = row_bytes_v / 16;
    for (int idx = threadIdx.x; idx < Hkv * nk; idx += blockDim.x) {
        const int h = idx / nk, c = idx - h * nk;
        ((u32x4*)(k_cache + (((size_t)pg * Hkv + h) * ps + off) * row_bytes_k))[c] = z;
    }
    for (int idx = threadIdx.x; idx < Hkv * nv; idx += blockDim.x) {
        const int h = idx / nv, c = idx - h * nv;
        ((u32x4*)(v_cache + (((size_t)pg * Hkv + h) * ps + off) * row_bytes_v))[c] = z;
    }
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int sd_kv_rollback(const sd_rollback_desc* d, void* stream) {
    clear_error();
    if (!d) return fail(SD_EINVAL, "sd_rollback_desc is NULL");
    if (d->batch <= 0 || d->K < 0 || d->page_size <= 0 || d->max_pages <= 0)
        return fail(SD_EINVAL, "sd_kv_rollback: bad batch/K/page_size/max_pages");
    if (!d->page_table || !d->num_accepted || !d->seq_lens || !d->rollback_slots ||
        !d->rollback_offsets || !d->freed_pages || !d->freed_offsets)
        return fail(SD_EINVAL, "sd_kv_rollback: NULL required pointer");
    if ((long)d->batch * (d->K + 1) > 0x7fffffffL)
        return fail(SD_EUNSUPPORTED, "sd_kv_rollback: batch too large");
    int es = 0;
    if (d->poison_rejected || d->accepted_nodes) {
        if (d->dtype != SD_F32 && d->dtype != SD_BF16 && d->dtype != SD_E4M3)
            return fail(SD_EINVAL, "sd_kv_rollback: unknown dtype %d", d->dtype);
        if (d->kind != SD_ATTN_GQA && d->kind != SD_ATTN_MLA)
            return fail(SD_EINVAL, "sd_kv_rollback: unknown kind %d", d->kind);
        es = d->dtype == SD_BF16 ? 2 : d->dtype == SD_E4M3 ? 1 : 4;
        if (!d->k_cache || (d->kind == SD_ATTN_GQA && !d->v_cache) || d->num_pages <= 0 ||
            d->n_kv_heads <= 0 || d->d_k <= 0 || (d->kind == SD_ATTN_GQA && d->d_v <= 0))
            return fail(SD_EINVAL,
                        "sd_kv_rollback: poisoning or a tree gather needs the cache description");
        if ((d->d_k * es) % 16 || (d->kind == SD_ATTN_GQA && (d->d_v * es) % 16) ||
            !aligned16(d->k_cache) || (d->v_cache && !aligned16(d->v_cache)))
            return fail(SD_EUNSUPPORTED, "sd_kv_rollback: cache rows must be 16-byte multiples");
    }
    hipStream_t s = (hipStream_t)stream;
    int rc;
    if (d->accepted_nodes) {
        rollback_gather<<<dim3(d->batch, d->kind == SD_ATTN_MLA ? 1 : d->n_kv_heads), 256, 0, s>>>(
            d->page_table, d->num_accepted, d->seq_lens, d->accepted_nodes, (uint8_t*)d->k_cache,
            (uint8_t*)d->v_cache, d->K, d->page_size, d->max_pages, d->num_pages,
            d->kind == SD_ATTN_MLA ? 1 : d->n_kv_heads, d->d_k * es, d->d_v * es,
            d->kind == SD_ATTN_MLA);
        if ((rc = check_launch("rollback_gather")) != SD_OK) return rc;
    }
    rollback_compact<<<1, 1024, 0, s>>>(d->page_table, d->num_accepted, d->seq_lens,
                                        d->rollback_slots, d->rollback_offsets, d->freed_pages,
                                        d->freed_offsets, d->dev_error, d->batch, d->K,
                                        d->page_size, d->max_pages, d->accepted_nodes);
    rc = check_launch("rollback_compact");
    if (rc != SD_OK || !d->poison_rejected) return rc;
    rollback_poison<<<dim3(d->batch, d->K + 1), 256, 0, s>>>(
        d->rollback_slots, d->rollback_offsets, (uint8_t*)d->k_cache, (uint8_t*)d->v_cache,
        d->page_size, d->num_pages, d->kind == SD_ATTN_MLA ? 1 : d->n_kv_heads, d->d_k * es,
        d->d_v * es, d->kind == SD_ATTN_MLA);
    return check_launch("rollback_poison");
}
