// Acceptance of draft chains on gfx950: greedy longest-prefix match or
// rejection sampling, final (correction or bonus) token, packed output.
//
// [VLLM-MTP] s3 stage 3: greedy verify accepts drafts equal to the target
// argmax up to the first mismatch; rejection verify accepts when the
// target/draft probability ratio beats a uniform and otherwise resamples;
// stage 4: one step emits 1 .. D+1 tokens.  [SD-PRACTICE] s2.3: on the first
// rejection the replacement comes from the target's distribution at that
// position and later drafts are dropped; s4.4: accept with probability
// min(1, p_target/p_draft), temperature 0 means argmax matching.
// [TRT-MTP] Fig. 1: the target token after the last accepted draft is
// emitted too.
//
// Kernels (one stream):
//   accept_rowstats  one block per logits row: argmax (smallest id on ties),
//                    finiteness, and for sampled rows the max m, the mass
//                    Z = sum exp((l-m)/T) in fp64 and p_t of the row's draft
//   accept_topp_*    sampled rows with top_p < 1: the nucleus threshold
//                    lambda (exact: all tokens tied with the last kept logit
//                    are kept), the kept mass, p_t of the draft
//   accept_decide    one block per request: the sequential accept decision,
//                    then the fp64 inverse-CDF draw of the final token
//   accept_pack      exclusive scan of emitted counts, packed tokens
// Statistics and running sums that decide integers are fp64 and reduced in a
// fixed order, so results do not depend on scheduling.
#include <math.h>

#include "sdv_device.h"
#include "sdv_internal.h"

namespace sdv {
namespace {

struct RowStat {
    float m;        // row maximum
    float lambda;   // nucleus threshold; -inf keeps every token
    int argmax;     // smallest id among the maxima
    int flags;      // SD_DERR_* bits of this row
    double zkeep;   // sum over kept tokens of exp((l - m) / T)
    double pt_d;    // p_t of the draft this row judges (row i judges draft i+1)
};

template <typename T>
struct Logit;
template <>
struct Logit<uint16_t> {
    static constexpr int kPerVec = 8;
    __device__ static float at(const uint16_t* p, int v) { return bf16_to_f32(p[v]); }
    __device__ static float lane(u32x4 w, int e) { return bf16_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu); }
};
template <>
struct Logit<float> {
    static constexpr int kPerVec = 4;
    __device__ static float at(const float* p, int v) { return p[v]; }
    __device__ static float lane(u32x4 w, int e) { return __uint_as_float(w[e]); }
};

// Visits every element of a row: vectorised 16-byte loads when the row is
// aligned, with a fixed element -> thread assignment.
template <typename T, typename F>
__device__ __forceinline__ void for_row(const T* row, int V, bool vec_ok, F&& f) {
    constexpr int E = Logit<T>::kPerVec;
    int v0 = 0;
    if (vec_ok) {
        const int nvec = V / E;
        for (int c = threadIdx.x; c < nvec; c += blockDim.x) {
            const u32x4 w = *(const u32x4*)(row + (size_t)c * E);
#pragma unroll
            for (int e = 0; e < E; ++e) f(Logit<T>::lane(w, e), c * E + e);
        }
        v0 = nvec * E;
    }
    for (int v = v0 + threadIdx.x; v < V; v += blockDim.x) f(Logit<T>::at(row, v), v);
}

// Fixed-order block sum of one double (256 threads).
__device__ double block_sum(double x, double* s4) {
    x = wave_sum(x);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) s4[wave] = x;
    __syncthreads();
    const double r = ((s4[0] + s4[1]) + s4[2]) + s4[3];
    __syncthreads();
    return r;
}

// exp((x - m) / T) in fp64, with 1/T precomputed once per row.
__device__ __forceinline__ double tempered(float x, float m, double invT) {
    return exp(((double)x - (double)m) * invT);
}

template <typename T>
__global__ __launch_bounds__(256) void accept_rowstats(
    const T* __restrict__ logits, const int32_t* __restrict__ drafts,
    const float* __restrict__ temperature, const float* __restrict__ top_p, int has_probs,
    RowStat* __restrict__ stats, int K, int V, int vec_ok) {
    __shared__ float s_best[4];
    __shared__ int s_idx[4];
    __shared__ double s_sum[4];
    const int Q = K + 1;
    const int row = blockIdx.x, b = row / Q, i = row - b * Q;
    const T* lr = logits + (size_t)row * V;
    const float Tb = temperature[b];
    const float tp = top_p ? top_p[b] : 1.f;
    const bool stoch = Tb > 0.f;
    int flags = 0;
    if (isnan(Tb) || Tb < 0.f) flags |= SD_DERR_PARAM;
    if (stoch && (isnan(tp) || tp <= 0.f || (!has_probs && K > 0))) flags |= SD_DERR_PARAM;

    float best = -INFINITY;
    int bidx = 0x7fffffff;
    int nonfinite = 0, anyfin = 0;
    for_row(lr, V, vec_ok != 0, [&](float x, int v) {
        if (x != x || x == INFINITY) nonfinite = 1;
        if (x > -INFINITY) anyfin = 1;
        if (x > best || (x == best && v < bidx)) {
            best = x;
            bidx = v;
        }
    });
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) {
        const float ob = shfl_xor(best, msk);
        const int oi = shfl_xor(bidx, msk);
        if (ob > best || (ob == best && oi < bidx)) {
            best = ob;
            bidx = oi;
        }
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
        s_best[wave] = best;
        s_idx[wave] = bidx;
    }
    nonfinite = __syncthreads_or(nonfinite);
    anyfin = __syncthreads_or(anyfin);
    best = s_best[0];
    bidx = s_idx[0];
    for (int w = 1; w < 4; ++w)
        if (s_best[w] > best || (s_best[w] == best && s_idx[w] < bidx)) {
            best = s_best[w];
            bidx = s_idx[w];
        }
    if (nonfinite || !anyfin) flags |= SD_DERR_NONFINITE;

    double z = 0.0, pt_d = 0.0;
    if (stoch && !flags) {
        double part = 0.0;
        const float m = best;
        const double invT = 1.0 / (double)Tb;
        for_row(lr, V, vec_ok != 0, [&](float x, int) { part += tempered(x, m, invT); });
        z = block_sum(part, s_sum);
        const int d = (i < K) ? drafts[(size_t)b * K + i] : -1;
        if (d >= 0 && d < V) pt_d = tempered(Logit<T>::at(lr, d), m, invT) / z;
    }
    if (threadIdx.x == 0) {
        RowStat st;
        st.m = best;
        st.lambda = -INFINITY;
        st.argmax = bidx;
        st.flags = flags;
        st.zkeep = z;
        st.pt_d = pt_d;
        stats[row] = st;
    }
}

// ---------------------------------------------------------------------------
// Nucleus threshold for bf16 rows.  Walks the 65536 orderable bf16 keys down
// from the row maximum in windows of 8192: an exact u32 count per key (LDS
// atomics), the mass of each level = count * exp((value - m) / T), a fixed
// order prefix over levels until the running mass reaches top_p * Z.  The
// level where it does is lambda; every token with logit >= lambda is kept.
// ---------------------------------------------------------------------------
constexpr int kWin = 8192;

__global__ __launch_bounds__(256) void accept_topp_bf16(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ drafts,
    const float* __restrict__ temperature, const float* __restrict__ top_p,
    RowStat* __restrict__ stats, int K, int V, int vec_ok) {
    extern __shared__ __attribute__((aligned(16))) uint32_t s_hist[];  // kWin
    __shared__ double s_part[257];
    __shared__ int s_found, s_lkey;
    __shared__ double s_zkeep;
    const int Q = K + 1;
    const int row = blockIdx.x, b = row / Q, i = row - b * Q;
    const float Tb = temperature[b];
    const float tp = top_p[b];
    const RowStat st = stats[row];
    if (!(Tb > 0.f) || !(tp < 1.f) || st.flags) return;
    const uint16_t* lr = logits + (size_t)row * V;
    const double target = (double)tp * st.zkeep;
    const float m = st.m;
    const double invT = 1.0 / (double)Tb;
    const int tid = threadIdx.x;
    double cum = 0.0;
    int lkey = -1;
    double zkeep = st.zkeep;
    for (int top = (int)bf16_key(__float_as_uint(m) >> 16);; top -= kWin) {
        const int bottom = top - (kWin - 1) > 0 ? top - (kWin - 1) : 0;
        for (int w = tid; w < kWin; w += blockDim.x) s_hist[w] = 0;
        __syncthreads();
        for_row(lr, V, vec_ok != 0, [&](float x, int) {
            const int k = (int)bf16_key(__float_as_uint(x) >> 16);
            if (k <= top && k >= bottom) atomicAdd(&s_hist[top - k], 1u);
        });
        __syncthreads();
        // Thread t owns levels [nl*t, nl*t + nl) of the window, highest first.
        const int nl = kWin / 256;
        double part = 0.0;
        for (int j = 0; j < nl; ++j) {
            const int idx = tid * nl + j;
            const uint32_t c = s_hist[idx];
            if (c && top - idx >= bottom)
                part += (double)c * tempered(bf16_to_f32(key_to_bf16(top - idx)), m, invT);
        }
        s_part[tid] = part;
        __syncthreads();
        if (tid == 0) {
            double run = cum;
            for (int t = 0; t < 256; ++t) {
                const double p = s_part[t];
                s_part[t] = run;  // exclusive prefix, offset by the mass above the window
                run += p;
            }
            s_part[256] = run;
            s_found = 0;
        }
        __syncthreads();
        const double pre = s_part[tid], nxt = s_part[tid + 1];
        if (pre < target && nxt >= target) {
            double run = pre;
            int last = -1;
            double at_last = pre;
            for (int j = 0; j < nl; ++j) {
                const int idx = tid * nl + j;
                const uint32_t c = s_hist[idx];
                if (!c || top - idx < bottom) continue;
                run += (double)c * tempered(bf16_to_f32(key_to_bf16(top - idx)), m, invT);
                last = top - idx;
                at_last = run;
                if (run >= target) break;
            }
            s_lkey = last;
            s_zkeep = at_last;
            s_found = 1;
        }
        __syncthreads();
        if (s_found) {
            lkey = s_lkey;
            zkeep = s_zkeep;
            break;
        }
        cum = s_part[256];
        __syncthreads();
        if (bottom == 0) break;  // never reached: keep every token
    }
    if (tid == 0) {
        RowStat out = st;
        out.lambda = lkey >= 0 ? bf16_to_f32(key_to_bf16((uint32_t)lkey)) : -INFINITY;
        out.zkeep = lkey >= 0 ? zkeep : st.zkeep;
        const int d = (i < K) ? drafts[(size_t)b * K + i] : -1;
        out.pt_d = 0.0;
        if (d >= 0 && d < V) {
            const float xd = bf16_to_f32(lr[d]);
            if (xd >= out.lambda) out.pt_d = tempered(xd, m, invT) / out.zkeep;
        }
        stats[row] = out;
    }
}

// Nucleus threshold for float32 rows: bisection over the 32-bit orderable
// key space for the largest key l with mass(key >= l) >= top_p * Z (32
// passes over the row, fp64 mass, fixed-order sums).
__global__ __launch_bounds__(256) void accept_topp_f32(
    const float* __restrict__ logits, const int32_t* __restrict__ drafts,
    const float* __restrict__ temperature, const float* __restrict__ top_p,
    RowStat* __restrict__ stats, int K, int V, int vec_ok) {
    __shared__ double s_sum[4];
    const int Q = K + 1;
    const int row = blockIdx.x, b = row / Q, i = row - b * Q;
    const float Tb = temperature[b];
    const float tp = top_p[b];
    const RowStat st = stats[row];
    if (!(Tb > 0.f) || !(tp < 1.f) || st.flags) return;
    const float* lr = logits + (size_t)row * V;
    const double target = (double)tp * st.zkeep;
    const float m = st.m;
    const double invT = 1.0 / (double)Tb;
    // Invariant: mass(key >= lo) >= target, mass(key >= hi) < target.
    uint64_t lo = 0, hi = (uint64_t)f32_key(__float_as_uint(m)) + 1;
    double mass_lo = st.zkeep;
    while (hi - lo > 1) {
        const uint64_t mid = (lo + hi) / 2;
        double part = 0.0;
        for_row(lr, V, vec_ok != 0, [&](float x, int) {
            if (f32_key(__float_as_uint(x)) >= mid) part += tempered(x, m, invT);
        });
        const double mass = block_sum(part, s_sum);
        if (mass >= target) {
            lo = mid;
            mass_lo = mass;
        } else {
            hi = mid;
        }
    }
    if (threadIdx.x == 0) {
        RowStat out = st;
        out.lambda = __uint_as_float(key_to_f32((uint32_t)lo));
        out.zkeep = mass_lo;
        const int d = (i < K) ? drafts[(size_t)b * K + i] : -1;
        out.pt_d = 0.0;
        if (d >= 0 && d < V && lr[d] >= out.lambda) out.pt_d = tempered(lr[d], m, invT) / out.zkeep;
        stats[row] = out;
    }
}

enum { kModeInvalid = 0, kModeDone = 1, kModeResidual = 2, kModeTarget = 3 };

// ---------------------------------------------------------------------------
// Per-request decision and final-token draw.  One block of 1024 threads (16
// waves) per request.  Thread 0 takes the sequential accept decision from the
// row statistics.  A sampled final token is an inverse-CDF draw in token-id
// order: wave w owns a contiguous run of ids, read 64 at a time (one id per
// lane, coalesced); each 64-id chunk's fp64 weight sum is reduced in a fixed
// lane order and kept in LDS.  A fixed-order scan over waves, then over the
// crossing wave's chunks, finds the chunk whose running sum first exceeds
// u * total; a lane-order prefix scan inside that chunk picks the token.
// ---------------------------------------------------------------------------
constexpr int kDecThreads = 1024;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecMaxChunks = 160;  // per wave: V <= 16 * 160 * 64 = 163840

template <typename T>
__device__ __forceinline__ double draw_weight(const T* lr, const float* pd, int v, bool resid,
                                             float lambda, float m, double invT, double invZ) {
    const float x = Logit<T>::at(lr, v);
    const double p = (x >= lambda) ? tempered(x, m, invT) * invZ : 0.0;
    if (!resid) return p;
    const double r = p - (double)pd[v];
    return r > 0.0 ? r : 0.0;
}

template <typename T>
__global__ __launch_bounds__(kDecThreads) void accept_decide(
    const T* __restrict__ logits, const int32_t* __restrict__ drafts,
    const float* __restrict__ temperature, const float* __restrict__ draft_probs,
    const float* __restrict__ u_accept, const float* __restrict__ u_sample,
    const RowStat* __restrict__ stats, int32_t* __restrict__ num_accepted,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ next_token, int32_t* err, int K,
    int V) {
    __shared__ int s_mode, s_j, s_row, s_f, s_wave, s_chunk;
    __shared__ double s_u, s_pre, s_total;
    __shared__ double s_wsum[kDecWaves];
    __shared__ double s_chunk_sum[kDecWaves * kDecMaxChunks];
    __shared__ int s_cand[kDecWaves];
    const int Q = K + 1;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        int flags = 0;
        for (int r = 0; r < Q; ++r) flags |= stats[(size_t)b * Q + r].flags;
        for (int n = 0; n < K; ++n)
            if (drafts[(size_t)b * K + n] >= V) flags |= SD_DERR_TOKEN;
        int mode = kModeInvalid, j = -1, row = 0, f = -1;
        if (flags) {
            set_error(err, flags);
        } else if (temperature[b] == 0.f) {
            j = 0;
            while (j < K) {
                const int d = drafts[(size_t)b * K + j];
                if (d < 0 || d != stats[(size_t)b * Q + j].argmax) break;
                ++j;
            }
            f = stats[(size_t)b * Q + j].argmax;
            mode = kModeDone;
        } else {
            j = K;
            mode = kModeTarget;
            row = K;
            for (int n = 1; n <= K; ++n) {
                const int d = drafts[(size_t)b * K + n - 1];
                if (d < 0) {
                    j = n - 1;
                    row = n - 1;
                    mode = kModeTarget;
                    break;
                }
                const double a = stats[(size_t)b * Q + n - 1].pt_d;
                const double qd = draft_probs[((size_t)b * K + n - 1) * V + d];
                const double ratio = qd > 0.0 ? a / qd : (a > 0.0 ? INFINITY : 0.0);
                const double acc = ratio < 1.0 ? ratio : 1.0;
                if ((double)u_accept[(size_t)b * Q + n - 1] < acc) continue;
                j = n - 1;
                row = n - 1;
                mode = kModeResidual;
                break;
            }
        }
        s_mode = mode;
        s_j = j;
        s_row = row;
        s_f = f;
        s_u = (double)u_sample[(size_t)b * Q + row];
    }
    __syncthreads();
    const int mode = s_mode;
    if (mode == kModeResidual || mode == kModeTarget) {
        const int row = s_row;
        const RowStat st = stats[(size_t)b * Q + row];
        const T* lr = logits + ((size_t)b * Q + row) * V;
        const float* pd = draft_probs ? draft_probs + ((size_t)b * K + row) * V : nullptr;
        const double invT = 1.0 / (double)temperature[b];
        const double invZ = 1.0 / st.zkeep;
        const int nchunks = (V + 63) / 64;
        const int cpw = (nchunks + kDecWaves - 1) / kDecWaves;  // chunks per wave
        const int c_begin = wave * cpw, c_end = min(nchunks, c_begin + cpw);
        bool resid = mode == kModeResidual;
        for (int pass = 0; pass < 2; ++pass) {
            double wsum = 0.0;
            for (int c = c_begin; c < c_end; ++c) {
                const int v = c * 64 + lane;
                double w = v < V ? draw_weight(lr, pd, v, resid, st.lambda, st.m, invT, invZ) : 0.0;
                w = wave_sum(w);
                if (lane == 0) s_chunk_sum[wave * kDecMaxChunks + (c - c_begin)] = w;
                wsum += w;
            }
            if (lane == 0) s_wsum[wave] = wsum;
            __syncthreads();
            if (tid == 0) {
                double tot = 0.0;
                for (int w = 0; w < kDecWaves; ++w) tot += s_wsum[w];
                s_total = tot;
            }
            __syncthreads();
            if (!(resid && s_total == 0.0)) break;
            resid = false;  // residual empty: draw from p_t itself
            __syncthreads();
        }
        if (tid == 0) {
            // Locate the first chunk whose running sum exceeds u * total.
            const double target = s_u * s_total;
            double run = 0.0;
            int fw = -1, fc = -1;
            for (int w = 0; w < kDecWaves && fw < 0; ++w) {
                if (run + s_wsum[w] > target) {
                    const int cb = w * cpw, ce = min(nchunks, cb + cpw);
                    for (int c = cb; c < ce; ++c) {
                        const double cs = s_chunk_sum[w * kDecMaxChunks + (c - cb)];
                        if (run + cs > target) {
                            fw = w;
                            fc = c;
                            break;
                        }
                        run += cs;
                    }
                    if (fw < 0) fw = -2;  // rounding: fall back below
                } else {
                    run += s_wsum[w];
                }
            }
            s_wave = fw;
            s_chunk = fc;
            s_pre = run;
        }
        __syncthreads();
        if (s_chunk >= 0 && wave == 0) {
            const int v = s_chunk * 64 + lane;
            const double w = v < V ? draw_weight(lr, pd, v, resid, st.lambda, st.m, invT, invZ) : 0.0;
            double incl = w;  // lane-order inclusive scan
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const double y = __shfl_up(incl, o, 64);
                if (lane >= o) incl += y;
            }
            const double target = s_u * s_total;
            const bool hit = v < V && s_pre + incl > target;
            const unsigned long long mask = __ballot(hit);
            if (lane == 0) s_f = mask ? s_chunk * 64 + __ffsll((long long)mask) - 1 : -1;
        }
        __syncthreads();
        if (s_chunk < 0 || s_f < 0) {
            // Rounding left no bucket above the target: the largest id with
            // positive weight.
            int cand = -1;
            for (int c = c_end - 1; c >= c_begin && cand < 0; --c) {
                const int v = c * 64 + lane;
                const bool pos = v < V && draw_weight(lr, pd, v, resid, st.lambda, st.m, invT, invZ) > 0.0;
                const unsigned long long mask = __ballot(pos);
                if (mask) cand = c * 64 + 63 - __clzll((long long)mask);
            }
            if (lane == 0) s_cand[wave] = cand;
            __syncthreads();
            if (tid == 0) {
                int f = -1;
                for (int w = 0; w < kDecWaves; ++w) f = max(f, s_cand[w]);
                s_f = f;
            }
            __syncthreads();
        }
    }
    if (tid == 0) {
        const int j = s_j;
        const int f = mode == kModeInvalid ? -1 : s_f;
        num_accepted[b] = j;
        next_token[b] = f;
        for (int k = 0; k < Q; ++k) {
            int tok = -1;
            if (mode != kModeInvalid) {
                if (k < j) tok = drafts[(size_t)b * K + k];
                else if (k == j) tok = f;
            }
            out_tokens[(size_t)b * Q + k] = tok;
        }
    }
}

// ---------------------------------------------------------------------------
// Packing: out_offsets = exclusive scan of emitted counts (j_b + 1, or 0 for
// an invalid request), packed tokens back to back, the rest -1.  One block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void accept_pack(const int32_t* __restrict__ num_accepted,
                                                    const int32_t* __restrict__ out_tokens,
                                                    int32_t* __restrict__ out_offsets,
                                                    int32_t* __restrict__ packed, int B, int Q) {
    __shared__ int s_wsum[16];
    __shared__ int s_carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < B; base += 1024) {
        const int b = base + tid;
        const int cnt = (b < B && num_accepted[b] >= 0) ? num_accepted[b] + 1 : 0;
        int x = cnt;  // inclusive wave scan
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) s_wsum[wave] = x;
        __syncthreads();
        int wpre = 0;
        for (int w = 0; w < wave; ++w) wpre += s_wsum[w];
        const int carry = s_carry;
        const int off = carry + wpre + x - cnt;
        if (b < B) {
            out_offsets[b] = off;
            for (int k = 0; k < cnt; ++k) packed[off + k] = out_tokens[(size_t)b * Q + k];
        }
        __syncthreads();
        if (tid == 0) {
            int tot = 0;
            for (int w = 0; w < 16; ++w) tot += s_wsum[w];
            s_carry = carry + tot;
        }
        __syncthreads();
    }
    const int total = s_carry;
    if (tid == 0) out_offsets[B] = total;
    for (int k = total + tid; k < B * Q; k += blockDim.x) packed[k] = -1;
}

size_t accept_ws_bytes(const sd_accept_desc* d) {
    return align_up(sizeof(RowStat) * (size_t)d->batch * (d->K + 1), 256);
}

int check_accept(const sd_accept_desc* d) {
    if (!d) return fail(SD_EINVAL, "sd_accept_desc is NULL");
    if (d->batch <= 0 || d->K < 0 || d->vocab <= 0)
        return fail(SD_EINVAL, "sd_accept: bad batch/K/vocab");
    if (d->logits_dtype != SD_BF16 && d->logits_dtype != SD_F32)
        return fail(SD_EINVAL, "sd_accept: unknown logits dtype %d", d->logits_dtype);
    if ((long)d->batch * (d->K + 1) > 0x7fffffffL)
        return fail(SD_EUNSUPPORTED, "sd_accept: too many rows");
    if ((long)d->vocab > (long)kDecWaves * kDecMaxChunks * 64)
        return fail(SD_EUNSUPPORTED, "sd_accept: vocab above %d", kDecWaves * kDecMaxChunks * 64);
    return SD_OK;
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int sd_accept_workspace_size(const sd_accept_desc* d, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(SD_EINVAL, "bytes is NULL");
    const int rc = check_accept(d);
    if (rc != SD_OK) return rc;
    *bytes = accept_ws_bytes(d);
    return SD_OK;
}

extern "C" int sd_accept(const sd_accept_desc* d, void* workspace, size_t ws_bytes, void* stream) {
    clear_error();
    int rc = check_accept(d);
    if (rc != SD_OK) return rc;
    if (!d->logits || !d->temperature || !d->u_accept || !d->u_sample || !d->num_accepted ||
        !d->out_tokens || !d->next_token || !d->out_offsets || !d->packed_tokens ||
        (d->K > 0 && !d->draft_tokens))
        return fail(SD_EINVAL, "sd_accept: NULL required pointer");
    if (!workspace || !aligned256(workspace))
        return fail(SD_EINVAL, "sd_accept: workspace NULL or not 256-byte aligned");
    const size_t need = accept_ws_bytes(d);
    if (ws_bytes < need) return fail(SD_EWORKSPACE, "sd_accept: workspace %zu < %zu", ws_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    RowStat* stats = (RowStat*)workspace;
    const int B = d->batch, K = d->K, V = d->vocab, Q = K + 1;
    const int rows = B * Q;
    const int es = d->logits_dtype == SD_BF16 ? 2 : 4;
    const int vec_ok = aligned16(d->logits) && ((size_t)V * es) % 16 == 0;
    const int has_probs = d->draft_probs != nullptr;
    if (d->logits_dtype == SD_BF16) {
        const uint16_t* lg = (const uint16_t*)d->logits;
        accept_rowstats<uint16_t><<<rows, 256, 0, s>>>(lg, d->draft_tokens, d->temperature,
                                                       d->top_p, has_probs, stats, K, V, vec_ok);
        if ((rc = check_launch("accept_rowstats")) != SD_OK) return rc;
        if (d->top_p) {
            accept_topp_bf16<<<rows, 256, kWin * sizeof(uint32_t), s>>>(
                lg, d->draft_tokens, d->temperature, d->top_p, stats, K, V, vec_ok);
            if ((rc = check_launch("accept_topp_bf16")) != SD_OK) return rc;
        }
        accept_decide<uint16_t><<<B, kDecThreads, 0, s>>>(lg, d->draft_tokens, d->temperature,
                                                  d->draft_probs, d->u_accept, d->u_sample, stats,
                                                  d->num_accepted, d->out_tokens, d->next_token,
                                                  d->dev_error, K, V);
    } else {
        const float* lg = (const float*)d->logits;
        accept_rowstats<float><<<rows, 256, 0, s>>>(lg, d->draft_tokens, d->temperature,
                                                    d->top_p, has_probs, stats, K, V, vec_ok);
        if ((rc = check_launch("accept_rowstats")) != SD_OK) return rc;
        if (d->top_p) {
            accept_topp_f32<<<rows, 256, 0, s>>>(lg, d->draft_tokens, d->temperature, d->top_p,
                                                 stats, K, V, vec_ok);
            if ((rc = check_launch("accept_topp_f32")) != SD_OK) return rc;
        }
        accept_decide<float><<<B, kDecThreads, 0, s>>>(lg, d->draft_tokens, d->temperature,
                                               d->draft_probs, d->u_accept, d->u_sample, stats,
                                               d->num_accepted, d->out_tokens, d->next_token,
                                               d->dev_error, K, V);
    }
    if ((rc = check_launch("accept_decide")) != SD_OK) return rc;
    accept_pack<<<1, 1024, 0, s>>>(d->num_accepted, d->out_tokens, d->out_offsets,
                                   d->packed_tokens, B, Q);
    return check_launch("accept_pack");
}
